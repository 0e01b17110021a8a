"""Seeded synthetic inputs shared by the GPU path and the CPU oracle.

This module draws random numbers and nothing else: it contains none of the
quantisation arithmetic.  Both sides receive the tensors it returns.

The key/value model follows the workload description used for the
LLaMA-2-7B / LLaMA-3.1-8B shaped test cases (the pages evaluate NSNQuant on
those models; their weights are not available, so synthetic K/V of the same
shape stands in for them):

    x[t, c] = g_t * (sigma_c * z[t, c] + mu_c),   then token 0 is scaled by 20

with z ~ N(0, 1), mu_c ~ N(0, 0.5^2) drawn once per (head, K/V), per-token gain
g_t ~ LogNormal(0, 0.5), and four fixed outlier channels whose std sigma_c is 10
(30 in the first two layers of the LLaMA-3.1-8B shaped case).  The pages note
that such outlier channels are where the standard-normal alignment is weakest
(NSNQuant summary pages, "Limitations" / referee major comment 3, Figs. 12-13).
The result is cast to fp16 with round-to-nearest-even.
"""
from __future__ import annotations

import torch

OUTLIER_CHANNELS = (5, 37, 77, 113)
KIND_K, KIND_V, KIND_Q = 0, 1, 2


def unit_seed(config_id: int, layer: int, b: int, head: int, kind: int) -> int:
    """Seed of one (config, layer, batch row, head, K/V/Q) unit."""
    return 1_000_000 * config_id + 10_000 * layer + 10 * head + kind + 100_000_000 * b


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def kv_unit(seed: int, L: int, d: int = 128, outlier_std: float = 10.0,
            device="cpu", token0_scale: float = 20.0) -> torch.Tensor:
    """One head's K or V stream: fp16 [L, d]."""
    g = _gen(seed, device)
    z = torch.randn(L, d, generator=g, device=device, dtype=torch.float32)
    sigma = torch.ones(d, device=device, dtype=torch.float32)
    for c in OUTLIER_CHANNELS:
        if c < d:
            sigma[c] = outlier_std
    mu = 0.5 * torch.randn(d, generator=g, device=device, dtype=torch.float32)
    gain = torch.exp(0.5 * torch.randn(L, generator=g, device=device, dtype=torch.float32))
    x = gain[:, None] * (z * sigma[None, :] + mu[None, :])
    if L > 0:
        x[0] *= token0_scale
    return x.to(torch.float16)


def query_unit(seed: int, d: int = 128, device="cpu") -> torch.Tensor:
    """One query head: fp16 [d], q ~ N(0, I)."""
    g = _gen(seed, device)
    return torch.randn(d, generator=g, device=device, dtype=torch.float32).to(torch.float16)


def kv_layer(config_id: int, layer: int, B: int, H: int, L: int, d: int = 128,
             outlier_std: float = 10.0, device="cpu"):
    """K and V of one layer: two fp16 tensors [B, H, L, d]."""
    k = torch.empty(B, H, L, d, dtype=torch.float16, device=device)
    v = torch.empty(B, H, L, d, dtype=torch.float16, device=device)
    for b in range(B):
        for h in range(H):
            k[b, h] = kv_unit(unit_seed(config_id, layer, b, h, KIND_K), L, d, outlier_std, device)
            v[b, h] = kv_unit(unit_seed(config_id, layer, b, h, KIND_V), L, d, outlier_std, device)
    return k, v


def queries(config_id: int, layer: int, B: int, Hq: int, d: int = 128, device="cpu"):
    """Decode queries of one layer: fp16 [B, Hq, d]."""
    q = torch.empty(B, Hq, d, dtype=torch.float16, device=device)
    for b in range(B):
        for h in range(Hq):
            q[b, h] = query_unit(unit_seed(config_id, layer, b, h, KIND_Q), d, device)
    return q


def randn_samples(seed: int, n: int, s: int) -> torch.Tensor:
    """Standard-normal training samples for the codebook, fp32 [n, s], drawn on
    the CPU generator so the same array feeds every consumer (the pages fit the
    codebook with k-means on torch.randn data)."""
    g = _gen(seed, "cpu")
    return torch.randn(n, s, generator=g, dtype=torch.float32)


def uniform_unit(seed: int, shape, device="cpu") -> torch.Tensor:
    """Plain N(0,1) fp16 tensor (used for invariance tests)."""
    g = _gen(seed, device)
    return torch.randn(*shape, generator=g, device=device, dtype=torch.float32).to(torch.float16)


# The workloads, as (name, dict) pairs.  Sizes mirror the LLaMA shapes named in
# the evaluation; "config_id" feeds unit_seed().
WORKLOADS = {
    "tiny": dict(config_id=0, layers=1, B=1, Hq=1, Hkv=1, L=512, d=128, bits=2, R=64),
    "llama2-7b-layer-b1-2bit": dict(config_id=1, layers=1, B=1, Hq=32, Hkv=32, L=4096, d=128, bits=2, R=128),
    "llama2-7b-layer-b16-1bit": dict(config_id=2, layers=1, B=16, Hq=32, Hkv=32, L=4096, d=128, bits=1, R=128),
    "llama3.1-8b-gqa-b4-32k-2bit": dict(config_id=3, layers=32, B=4, Hq=32, Hkv=8, L=32768, d=128, bits=2, R=128),
    "llama2-7b-b256-2bit": dict(config_id=4, layers=32, B=256, Hq=32, Hkv=32, L=4096, d=128, bits=2, R=128),
}


def outlier_std_for(workload: str, layer: int) -> float:
    if workload.startswith("llama3.1") and layer < 2:
        return 30.0
    return 10.0


def hadamard_signs(seed: int, d: int = 128) -> torch.Tensor:
    """+-1 int8 [d] for the randomised Hadamard transform (fair coin per channel)."""
    g = _gen(seed, "cpu")
    return (torch.randint(0, 2, (d,), generator=g, dtype=torch.int8) * 2 - 1).to(torch.int8)


def rope_tables(max_pos: int, base: float = 10000.0, d: int = 128):
    """Rotary-embedding tables cos, sin fp32 [max_pos, d/2] with the standard
    frequencies theta_c = base^(-2c/d) (angles formed in float64)."""
    c = torch.arange(d // 2, dtype=torch.float64)
    theta = base ** (-2.0 * c / d)
    ang = torch.arange(max_pos, dtype=torch.float64)[:, None] * theta[None, :]
    return torch.cos(ang).to(torch.float32), torch.sin(ang).to(torch.float32)
