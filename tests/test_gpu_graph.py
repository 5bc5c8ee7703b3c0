"""One step of the hot path captured in a HIP graph (as bench.py times it)
gives, on every replay, exactly the outputs of the same step run eagerly:
the replays are separated by other eager work and synchronizations, and
every output (Hdiag, scores, bit map, permutation, planes, Y, K/V codes) is
compared bit for bit after each replay."""
import pytest
import torch

from bit_gemm_hdiag_amd import synth

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def mx():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import bit_gemm_hdiag_amd as mx
    return mx


def test_step_graph_replays_match_eager(mx):
    M, N, K, C = 256, 384, 1024, 512
    gains = synth.outlier_gains(K, 3)
    Xc = synth.activations(C, K, 1, gains, device=DEV)
    X = synth.activations(M, K, 2, gains, device=DEV)
    W = synth.weights(N, K, 0, device=DEV)
    Kc = synth.kv(128, 8, 128, 4, device=DEV)
    Vc = synth.kv(128, 8, 128, 12, device=DEV)
    n8, n6, n4 = mx.mxs_budget_blocks(K, 500, 1500)
    hd = torch.zeros(K, dtype=torch.float64, device=DEV)
    sc = torch.empty(K, dtype=torch.float64, device=DEV)
    bits = torch.empty(K, dtype=torch.uint8, device=DEV)
    perm = torch.empty(K, dtype=torch.int32, device=DEV)
    Aq = mx.qmat_alloc(M, K, n8, n6, n4, DEV)
    Wq = mx.qmat_alloc(N, K, n8, n6, n4, DEV)
    Y = torch.empty(M, N, device=DEV)
    u8 = dict(dtype=torch.uint8, device=DEV)
    wsc = torch.empty(max(1, mx.mxs_calibrate_workspace(C, K)), **u8)
    wss = torch.empty(max(1, mx.mxs_score_workspace(N, K)), **u8)
    wsg = torch.empty(max(1, mx.mxs_mixed_gemm_workspace(Aq, Wq)), **u8)
    kc = [torch.empty(128, 8, 64, **u8) for _ in range(2)]
    ks = [torch.empty(128, 8, 4, **u8) for _ in range(2)]

    def step():
        hd.zero_()
        mx.mxs_calibrate(Xc, hd, ws=wsc)
        mx.mxs_score(W, hd, sc, ws=wss)
        mx.mxs_allocate(sc, 500, 1500, bits, perm)
        mx.mxs_quantize(W, perm, n8, n6, n4, out=Wq)
        mx.mxs_quantize(X, perm, n8, n6, n4, out=Aq)
        mx.mxs_mixed_gemm(Aq, Wq, Y, ws=wsg)
        mx.mxs_quantize_kv(Kc, kc[0], ks[0])
        mx.mxs_quantize_kv(Vc, kc[1], ks[1])

    def outputs():
        return [t.clone() for t in (hd, sc, bits, perm, Aq.q8, Aq.q6, Aq.q4, Aq.sc, Wq.q8, Wq.q6, Wq.q4, Wq.sc, Y,
                                    kc[0], ks[0], kc[1], ks[1])]

    step()
    torch.cuda.synchronize()
    ref = outputs()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for t in (hd, sc, Y):                      # eager work between replays
            t.fill_(float(rep + 7))
        perm.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outputs(), ref):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), rep
