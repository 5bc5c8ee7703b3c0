"""Attention over the 4-bit K/V cache on the GPU against the oracle (through
the C ABI). K and V are quantized on the GPU (mxs_quantize_kv), the same
codes go to the oracle.

Tolerance: the GPU score of token t differs from the fp64 one by at most
eps_t = scale (D + 2) 2^-24 sum_d |q_d K_td| (fp32 products and a D-term sum),
so the normalised weights p_t / L carry a relative error of at most
expm1(2 max_t eps_t + c (T + D) 2^-24) (exponentials and the T-term sums
included), which bounds |o - o_ref| by that factor times sum_t p_t |V_t| / L;
the test allows twice that.
"""
import numpy as np
import pytest
import torch

from bit_gemm_hdiag_amd import synth

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
U = 2.0 ** -24


@pytest.fixture(scope="module")
def mx():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import bit_gemm_hdiag_amd as mx
    return mx


def dequant(codes, scales):
    lo = (codes & 15).astype(np.int32)
    hi = (codes >> 4).astype(np.int32)
    c = np.stack([lo, hi], -1).reshape(*codes.shape[:-1], -1)
    c = np.where(c >= 8, c - 16, c)
    e = np.repeat(scales.astype(np.float64) - 127, 32, axis=-1)
    return c * np.exp2(e)


def bound(q, K, V, scale):
    Hq, D = q.shape
    T, Hkv = K.shape[0], K.shape[1]
    G = Hq // Hkv
    tol = np.zeros((Hq, D))
    for h in range(Hq):
        g = h // G
        qk = K[:, g, :] * q[h].astype(np.float64)
        s = scale * qk.sum(1)
        eps = scale * (D + 2) * U * np.abs(qk).sum(1)
        p = np.exp(s - s.max())
        rel = np.expm1(2 * eps.max() + 8 * (T + D) * U)
        tol[h] = 2 * rel * (p[:, None] * np.abs(V[:, g, :])).sum(0) / p.sum()
    return tol + 1e-30


# the long cases run the workgroups that hold two KV heads and several token
# parts: 32740 ends in a ragged part, 30000 in an empty part, 12000 (three KV
# heads) in a workgroup with one head missing; then plain multi-head (32 KV
# heads), the largest group (16 query heads per KV head) and one KV head with
# D = 160
@pytest.mark.parametrize("T,Hq,Hkv,D", [(1, 8, 8, 32), (5, 4, 2, 64), (300, 64, 8, 128), (2048, 64, 8, 128),
                                        (257, 16, 1, 256), (1000, 32, 4, 96), (513, 12, 3, 64),
                                        (32740, 32, 8, 128), (30000, 16, 8, 64), (12000, 12, 3, 64),
                                        (20000, 8, 4, 96), (40000, 4, 2, 256),
                                        (1000, 32, 32, 128), (4000, 64, 4, 64), (9000, 16, 1, 160)])
def test_attend_kv4_matches_oracle(mx, orc, T, Hq, Hkv, D):
    seed = T * 7 + Hq + D
    Kf = synth.kv(T, Hkv, D, seed, device=DEV)
    Vf = synth.kv(T, Hkv, D, seed + 1, device=DEV)
    kc, ks = mx.mxs_quantize_kv(Kf)
    vc, vs = mx.mxs_quantize_kv(Vf)
    g = torch.Generator(device="cpu").manual_seed(seed)
    q = torch.randn(Hq, D, generator=g).to(DEV)
    scale = 1.0 / np.sqrt(D)
    out = mx.mxs_attend_kv4(q, (kc, ks), (vc, vs), scale)
    out2 = mx.mxs_attend_kv4(q, (kc, ks), (vc, vs), scale)
    assert torch.equal(out, out2)                       # deterministic
    h = lambda t: t.cpu().numpy()
    ref = orc.attend_kv4(h(q), h(kc), h(ks), h(vc), h(vs), np.float32(scale))
    # the GPU cache equals the oracle's own quantization of the same values
    okc, oks = orc.quantize_kv(Kf.float().cpu().numpy())
    assert np.array_equal(okc, h(kc)) and np.array_equal(oks, h(ks))
    K, V = dequant(h(kc), h(ks)), dequant(h(vc), h(vs))
    err = np.abs(h(out).astype(np.float64) - ref)
    assert np.all(err <= bound(h(q), K, V, float(np.float32(scale)))), float((err / bound(h(q), K, V, scale)).max())


def test_attend_kv4_one_token_and_sharp_scores(mx, orc):
    # one token: the output is that token's V row exactly; a score far above
    # the rest selects its token
    kv = synth.kv(1, 2, 64, 77, device=DEV)
    kc, ks = mx.mxs_quantize_kv(kv)
    q = torch.randn(4, 64).to(DEV)
    out = mx.mxs_attend_kv4(q, (kc, ks), (kc, ks), 0.125).cpu().numpy()
    V = dequant(kc.cpu().numpy(), ks.cpu().numpy())
    for hh in range(4):
        assert np.array_equal(out[hh].astype(np.float64), V[0, hh // 2])
    T = 300
    K = torch.zeros(T, 1, 64, device=DEV)
    K[123, 0, :] = 1.0
    kc, ks = mx.mxs_quantize_kv(K)
    Vf = synth.kv(T, 1, 64, 78, device=DEV)
    vc, vs = mx.mxs_quantize_kv(Vf)
    out = mx.mxs_attend_kv4(torch.ones(1, 64, device=DEV), (kc, ks), (vc, vs), 100.0).cpu().numpy()
    V = dequant(vc.cpu().numpy(), vs.cpu().numpy())
    assert np.array_equal(out[0].astype(np.float64), V[123, 0])
