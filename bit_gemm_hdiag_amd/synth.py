"""Seeded synthetic inputs shaped like the layers the MXSens pages evaluate.

This module only draws random numbers: it holds none of the method's
arithmetic, and both the HIP path and the CPU oracle receive exactly the
tensors it returns (the oracle gets host copies).

Activation model (outlier channels, [NL] §1 and [REV] "Prior limitations":
outliers range from rare extreme channels to frequent mild ones):
    X = Z * g,  Z ~ N(0, 1) i.i.d.,  g_k = 50 on the extreme set, 4 on the
    mild set, 1 elsewhere; the sets are a seeded draw per layer input and are
    shared by that input's calibration and inference tokens.
Weight model: W = 0.02 * T, T ~ Student-t with 4 degrees of freedom,
drawn as Z / sqrt(chi2_4 / 4) from five standard normals.
Values are drawn in fp32 and rounded to bf16 (round-to-nearest-even) where
the workload is bf16.

Seeds: seed = 1000 * config + role (+ 16 * layer for multi-layer runs), with
roles W = 0, calibration X = 1, inference X = 2, channel sets = 3, KV = 4.
"""
from __future__ import annotations

import torch

ROLE_W, ROLE_CALIB, ROLE_X, ROLE_CHANNELS, ROLE_KV = 0, 1, 2, 3, 4


def seed_of(config: int, role: int, layer: int = 0) -> int:
    return 1000 * config + role + 16 * layer


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def outlier_gains(K: int, seed: int, n_extreme: int | None = None, n_mild: int | None = None,
                  extreme: float = 50.0, mild: float = 4.0) -> torch.Tensor:
    """fp32 [K] channel gains: 0.1% extreme (x50) and 1% mild (x4) channels by default."""
    if n_extreme is None:
        n_extreme = int(round(0.001 * K))
    if n_mild is None:
        n_mild = int(round(0.01 * K))
    order = torch.randperm(K, generator=_gen(seed, "cpu"))
    g = torch.ones(K, dtype=torch.float32)
    g[order[:n_extreme]] = extreme
    g[order[n_extreme:n_extreme + n_mild]] = mild
    return g


def activations(M: int, K: int, seed: int, gains: torch.Tensor, dtype=torch.bfloat16,
                device="cpu", chunk_rows: int = 8192) -> torch.Tensor:
    """[M, K] tokens x channels, N(0,1) times the channel gains."""
    out = torch.empty((M, K), dtype=dtype, device=device)
    gen = _gen(seed, device)
    g = gains.to(device=device, dtype=torch.float32)
    for r0 in range(0, M, chunk_rows):
        r1 = min(M, r0 + chunk_rows)
        z = torch.randn((r1 - r0, K), generator=gen, device=device, dtype=torch.float32)
        out[r0:r1] = (z * g).to(dtype)
    return out


def weights(N: int, K: int, seed: int, dtype=torch.bfloat16, device="cpu",
            chunk_rows: int = 2048, scale: float = 0.02) -> torch.Tensor:
    """[N, K] out x in, 0.02 * Student-t(df=4)."""
    out = torch.empty((N, K), dtype=dtype, device=device)
    gen = _gen(seed, device)
    for r0 in range(0, N, chunk_rows):
        r1 = min(N, r0 + chunk_rows)
        z = torch.randn((5, r1 - r0, K), generator=gen, device=device, dtype=torch.float32)
        chi2 = (z[1:] * z[1:]).sum(0)
        t = z[0] / torch.sqrt(chi2 / 4.0)
        out[r0:r1] = (scale * t).to(dtype)
    return out


def kv(T: int, H: int, D: int, seed: int, dtype=torch.bfloat16, device="cpu") -> torch.Tensor:
    """[T, H, D] keys or values with the same outlier-channel model over H*D channels."""
    gains = outlier_gains(H * D, seed + 7)
    return activations(T, H * D, seed, gains, dtype=dtype, device=device).reshape(T, H, D)


# Workloads of the benchmark and the parity tests. Budgets are per layer,
# in basis points of columns at 8 and 6 bits.
CONFIGS = {
    1: dict(name="tiny linear 64x256x256 fp32", M=64, N=256, K=256, calib_rows=64,
            dtype="f32", n_extreme=2, n_mild=8, budget=(500, 1500)),
    2: dict(name="Llama-3-8B q_proj prefill 2048x4096x4096 bf16", M=2048, N=4096, K=4096,
            calib_rows=8 * 2048, dtype="bf16", budget=(500, 1500),
            kv=dict(T=2048, H=8, D=128)),
    3: dict(name="Llama-3-8B MLP W4A4 prefill, M=4096", M=4096,
            layers=[dict(name="gate", N=14336, K=4096, budget=(300, 1000)),
                    dict(name="up", N=14336, K=4096, budget=(300, 1000)),
                    dict(name="down", N=4096, K=14336, budget=(800, 2000))],
            calib_rows=8 * 2048, dtype="bf16"),
    4: dict(name="Llama-2-70B decode GEMV", Ms=(1, 8, 32),
            layers=[dict(name="up", N=28672, K=8192, budget=(500, 1500)),
                    dict(name="down", N=8192, K=28672, budget=(500, 1500))],
            dtype="bf16"),
    5: dict(name="Llama-2-70B pipeline", M=2048, n_layers=80, calib_rows=128 * 2048,
            layers=[dict(name="q", N=8192, K=8192), dict(name="k", N=1024, K=8192),
                    dict(name="v", N=1024, K=8192), dict(name="o", N=8192, K=8192),
                    dict(name="gate", N=28672, K=8192), dict(name="up", N=28672, K=8192),
                    dict(name="down", N=8192, K=28672)],
            budget=(500, 1500), kv=dict(T=2048, H=8, D=128), dtype="bf16"),
}
