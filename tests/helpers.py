"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI,
pull results back, and compare them with the oracle under the stated bars:

  codes     bit-exact, except where the oracle's best/second distance gap is
            below 1e-4 relative; such near-tie flips at most 0.01% of codes;
  scalars   fp16 n1, n2, mu within one fp16 ulp (fp32 vs fp64 rounding);
  dequant   max |x_hat_gpu - x_hat_oracle| <= 1e-3 * ||x_t||;
  attention relative L2 error <= 2e-3 per output head.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from kv_cache_bit_amd import nsnq

DEV = "cuda"
NEAR_TIE = 1e-4
MAX_TIE_FRAC = 1e-4
DEQUANT_TOL = 1e-3
ATTN_TOL = 2e-3


def f16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().numpy().view(np.uint16)


def cb_tensor(cb_bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(cb_bits).view(np.float16)).to(DEV)


def capacity(L: int, R: int, extra_blocks: int = 1) -> int:
    r = ((L - 1) % R) + 1 if L > 0 else 0
    nq = L - r
    return max(R, nq + extra_blocks * R)


def gpu_encode(k: torch.Tensor, v: torch.Tensor, bits: int, R: int, cb_bits: np.ndarray, cap: int | None = None,
               flags: int = 0, signs: torch.Tensor | None = None, cand: bool = False):
    """Encode on the GPU; cand=True searches the per-orthant candidate lists."""
    p = nsnq.params(bits, R, flags=flags, signs=None if signs is None else signs.to(DEV))
    B, H, L, d = k.shape
    cache = nsnq.KVCache(p, B, H, cap or capacity(L, R), DEV)
    cb = cb_tensor(cb_bits)
    if cand:
        p = nsnq.with_candidates(p, cb)
    nsnq.nsnq_encode_kv(p, cb, k.to(DEV), v.to(DEV), L, cache)
    torch.cuda.synchronize()
    return p, cb, cache


def half_np(cache: nsnq.KVCache, which: int, n_tokens: int | None = None) -> dict:
    h = cache.k if which == 0 else cache.v
    nq = cache.n_quant if n_tokens is None else n_tokens
    R = h.resid.shape[2]
    if getattr(cache, "dq", False):
        return dict(codes=h.codes[:, :, :nq].cpu().numpy(), scales=h.scales[:, :, :nq // R].cpu().numpy(),
                    mu=h.mu[:, :, :nq // R].cpu().numpy(), resid=f16_bits(h.resid))
    return dict(codes=h.codes[:, :, :nq].cpu().numpy(), scales=f16_bits(h.scales[:, :, :nq]),
                mu=f16_bits(h.mu[:, :, :nq // R]), resid=f16_bits(h.resid))


def upload_half(cache: nsnq.KVCache, which: int, enc: dict):
    """Copy an oracle-encoded half (codes/scales/mu/resid) into a GPU cache."""
    h = cache.k if which == 0 else cache.v
    nq = enc["codes"].shape[-2]
    R = h.resid.shape[2]
    h.codes[:, :, :nq].copy_(torch.from_numpy(enc["codes"]))
    if enc.get("dq", False):
        h.scales[:, :, :nq // R].copy_(torch.from_numpy(enc["scales"]))
        h.mu[:, :, :nq // R].copy_(torch.from_numpy(enc["mu"]))
    else:
        h.scales[:, :, :nq].copy_(torch.from_numpy(enc["scales"].view(np.float16)))
        h.mu[:, :, :nq // R].copy_(torch.from_numpy(enc["mu"].view(np.float16)))
    h.resid.copy_(torch.from_numpy(enc["resid"].view(np.float16)))


def check_codes(g: np.ndarray, o: np.ndarray, gap: np.ndarray, u: np.ndarray, cb_bits: np.ndarray,
                what: str = "codes", pooled: bool = False):
    """Codes equal outside the near-tie band; near-tie flips within the rate
    bound.  Every differing code must itself be a near-best choice: with u the
    oracle's Hadamard-domain vectors [..., n, d] (fp64), the distance of the
    GPU's codeword exceeds the oracle's minimum by less than 1e-4 relative.
    pooled=True leaves the rate bound to the caller, who applies it to the
    whole test's population (check_tie_rate)."""
    assert g.shape == o.shape, (g.shape, o.shape)
    mism = g != o
    n = int(mism.sum())
    bad = int((mism & (gap >= NEAR_TIE)).sum())
    assert bad == 0, f"{what}: {bad} mismatches outside the near-tie band (of {n} total, {g.size} codes)"
    if n:
        s = cb_bits.shape[1]
        assert u.shape[:-1] == g.shape[:-1] and u.shape[-1] == g.shape[-1] * s, (u.shape, g.shape)
        us = u.reshape(*g.shape, s)[mism]
        cbd = np.ascontiguousarray(cb_bits).view(np.float16).astype(np.float64)
        d_gpu = ((us - cbd[g[mism]]) ** 2).sum(-1)
        d_best = ((us - cbd[o[mism]]) ** 2).sum(-1)
        assert np.all(d_best > 0), f"{what}: a differing code where the oracle's distance is 0"
        excess = (d_gpu - d_best) / d_best
        assert excess.max() < NEAR_TIE, f"{what}: a differing GPU code is {excess.max():.2e} (relative) from the best"
    if not pooled:
        check_tie_rate(n, g.size, what)
    return n


def check_tie_rate(n: int, total: int, what: str = "codes"):
    assert n <= max(MAX_TIE_FRAC * total, 1), f"{what}: {n} near-tie mismatches of {total} codes"


def check_f16_ulp(g_bits: np.ndarray, o_bits: np.ndarray, what: str, max_flip_frac: float = 1e-2):
    g = g_bits.view(np.float16).astype(np.float64)
    o = o_bits.view(np.float16).astype(np.float64)
    ulp = np.spacing(np.abs(o_bits.view(np.float16))).astype(np.float64)
    diff = np.abs(g - o)
    assert np.all(diff <= ulp * 1.0001), f"{what}: max diff {diff.max()} exceeds one fp16 ulp"
    flips = int((diff > 0).sum())
    assert flips <= max(max_flip_frac * g.size, 2), f"{what}: {flips} of {g.size} values off by one ulp"
    return flips


def token_norms(x_f16: np.ndarray) -> np.ndarray:
    return np.linalg.norm(x_f16.astype(np.float64), axis=-1)


def check_dequant(g: np.ndarray, o: np.ndarray, norms: np.ndarray, mask: np.ndarray | None = None,
                  tol: float = DEQUANT_TOL):
    err = np.abs(g.astype(np.float64) - o).max(axis=-1) / np.maximum(norms, 1e-30)
    if mask is not None:
        err = err[mask]
    assert err.size == 0 or err.max() <= tol, f"dequant: max error {err.max():.3e} of token norm"
    return float(err.max()) if err.size else 0.0


def check_attention(g: np.ndarray, o: np.ndarray, tol: float = ATTN_TOL):
    g = g.astype(np.float64)
    rel = np.linalg.norm(g - o, axis=-1) / np.maximum(np.linalg.norm(o, axis=-1), 1e-30)
    assert rel.max() <= tol, f"attention: max relative L2 error {rel.max():.3e}"
    return float(rel.max())


def oracle_encode(x, R: int, cb_bits: np.ndarray, **kw) -> dict:
    """The oracle's encoding of streams x, with the Hadamard-domain vectors u
    (fp64) the code checks need and the codebook it used."""
    xc = x.cpu() if hasattr(x, "cpu") else x
    e = oracle.encode(xc, R, cb_bits, with_u=True, **kw)
    e["cb"] = cb_bits
    e["x"], e["kw"] = xc, kw  # for re-encodes with another encoder's 4-bit decisions
    return e


def oracle_encode_pair(k: torch.Tensor, v: torch.Tensor, R: int, cb_bits: np.ndarray, signs=None,
                      scale_adjust: bool = False, dq: bool = False):
    kw = dict(signs=signs, scale_adjust=scale_adjust, dq=dq)
    return oracle_encode(k, R, cb_bits, **kw), oracle_encode(v, R, cb_bits, **kw)


def gpu_records(cache: nsnq.KVCache, which: int) -> dict:
    """One half of a GPU cache in the oracle's dict layout (codes, scales, mu,
    resid; the double-quantised flag), for oracle.reference_decode over the
    GPU's own records."""
    h = half_np(cache, which)
    h["dq"] = bool(getattr(cache, "dq", False))
    return h


def compare_encoded(cache: nsnq.KVCache, ek: dict, ev: dict, units=None, scale_adjust: bool = False):
    """Compare a GPU cache with the oracle's encodings (optionally only the
    (b, h) pairs in `units`).  Returns per-half code mismatch counts.  With
    scale adjustment n2 depends on every code of its token, so tokens with a
    near-tie code flip are left out of the n2 comparison."""
    out = []
    for which, e in ((0, ek), (1, ev)):
        gh = half_np(cache, which)
        if units is not None:
            gh = {key: np.stack([val[b, h] for b, h in units]) for key, val in gh.items()}
        n = check_codes(gh["codes"], e["codes"], e["gap"], e["u"], e["cb"], "K codes" if which == 0 else "V codes")
        if scale_adjust:
            same = np.all(gh["codes"] == e["codes"], axis=-1)
            check_f16_ulp(gh["scales"][..., 0], e["scales"][..., 0], "n1")
            check_f16_ulp(gh["scales"][..., 1][same], e["scales"][..., 1][same], "n2 (adjusted)")
        else:
            check_f16_ulp(gh["scales"], e["scales"], "scales")
        check_f16_ulp(gh["mu"], e["mu"], "mu")
        assert np.array_equal(gh["resid"][..., :e["n_resid"], :], e["resid"][..., :e["n_resid"], :])
        out.append(n)
    return out


# ---------------------------------------------------- double quantisation --

DQ_MARGIN = 0.02  # 4-bit decisions this close (in steps) to a rounding tie may differ (fp32 vs fp64)


def _dq_fields(sc: np.ndarray, mu: np.ndarray, R: int):
    """Parse double-quantised records [..., nb, bytes] into (n2 bits [..., nb, R],
    q1 [..., nb, R], s1 (S, Z) bits [..., nb, 2], qm [..., nb, 128], mu (S, Z)
    bits [..., nb, 4, 2])."""
    n2 = np.ascontiguousarray(sc[..., :2 * R]).view(np.uint16)
    nib = sc[..., 2 * R:2 * R + R // 2]
    q1 = np.stack([nib & 15, nib >> 4], axis=-1).reshape(*nib.shape[:-1], R)
    sz = np.ascontiguousarray(sc[..., 2 * R + R // 2:2 * R + R // 2 + 4]).view(np.uint16)
    qm = np.stack([mu[..., :64] & 15, mu[..., :64] >> 4], axis=-1).reshape(*mu.shape[:-1], 128)
    msz = np.ascontiguousarray(mu[..., 64:80]).view(np.uint16).reshape(*mu.shape[:-1], 4, 2)
    return n2, q1, sz, qm, msz


def compare_encoded_dq(cache: nsnq.KVCache, ek: dict, ev: dict, R: int, scale_adjust: bool = False):
    """Double-quantised caches against the oracle.  Per block: the fp16 (S, Z)
    pairs within one ulp; every 4-bit code equal to the oracle's or one level
    from it, and equal unless the decision is within DQ_MARGIN of a rounding
    tie where the block's (S, Z) pair is the oracle's; a block whose 4-bit
    decisions all agree is then held to the plain bars (codes with the
    near-tie rule, each differing code near-best for the oracle's u; n2 within
    one ulp).  Blocks with a differing decision (expected rarely) are at most
    2% of blocks; the oracle re-encodes them with the GPU's own 4-bit records
    (its decisions taken as given), and their codes and n2 are held to the
    same bars against that re-encode.  Returns the list of per-half boolean
    block masks (True = the 4-bit decisions agree)."""
    masks = []
    for which, e in ((0, ek), (1, ev)):
        gh = half_np(cache, which)
        gn2, gq1, gsz, gqm, gmsz = _dq_fields(gh["scales"], gh["mu"], R)
        on2, oq1, osz, oqm, omsz = _dq_fields(e["scales"], e["mu"], R)
        nb = gq1.shape[-2]
        # (S, Z) pairs within one fp16 ulp
        check_f16_ulp(gsz, osz, "s1 (S, Z)", max_flip_frac=0.05)
        check_f16_ulp(gmsz, omsz, "mean (S, Z)", max_flip_frac=0.05)
        m1 = e["m1"].reshape(oq1.shape)
        mmu = e["mmu"].reshape(oqm.shape)
        same_par = np.all(gsz == osz, axis=-1) & np.all(gmsz == omsz, axis=(-1, -2))
        d1 = (gq1 != oq1)
        dm = (gqm != oqm)
        # a differing 4-bit code is always the neighbouring level
        assert np.all(np.abs(gq1.astype(np.int32) - oq1.astype(np.int32)) <= 1), "s1 code off by more than one level"
        assert np.all(np.abs(gqm.astype(np.int32) - oqm.astype(np.int32)) <= 1), "mean code off by more than one level"
        # with equal (S, Z), differing codes only near a tie
        assert not np.any(d1 & same_par[..., None] & (m1 >= DQ_MARGIN)), "s1 code differs away from a tie"
        assert not np.any(dm & same_par[..., None] & (mmu >= DQ_MARGIN)), "mean code differs away from a tie"
        full = same_par & ~np.any(d1, axis=-1) & ~np.any(dm, axis=-1)
        assert (~full).sum() <= max(0.02 * full.size, 1), f"{(~full).sum()} of {full.size} blocks differ in 4-bit decisions"
        S = gh["codes"].shape[-1]
        cg = gh["codes"].reshape(*gh["codes"].shape[:-2], nb, R, S)
        co = e["codes"].reshape(cg.shape)
        gap = e["gap"].reshape(cg.shape)
        u = e["u"].reshape(*cg.shape[:-1], -1)
        n = check_codes(cg[full], co[full], gap[full], u[full], e["cb"], "codes (double-quantised)")
        if scale_adjust:
            same = np.all(cg[full] == co[full], axis=-1)
            check_f16_ulp(gn2[full][same], on2[full][same], "n2")
        else:
            check_f16_ulp(gn2[full], on2[full], "n2")
        assert np.array_equal(gh["resid"][..., :e["n_resid"], :], e["resid"][..., :e["n_resid"], :])
        if (~full).any():
            fe = oracle.encode(e["x"], R, e["cb"], with_u=True, force_records=(gh["scales"], gh["mu"]), **e["kw"])
            fn2 = _dq_fields(fe["scales"], fe["mu"], R)[0]
            fc = fe["codes"].reshape(cg.shape)
            fgap = fe["gap"].reshape(cg.shape)
            fu = fe["u"].reshape(*cg.shape[:-1], -1)
            part = ~full
            check_codes(cg[part], fc[part], fgap[part], fu[part], e["cb"], "codes (double-quantised, GPU's 4-bit records)")
            if scale_adjust:
                same = np.all(cg[part] == fc[part], axis=-1)
                check_f16_ulp(gn2[part][same], fn2[part][same], "n2 (GPU's 4-bit records)")
            else:
                check_f16_ulp(gn2[part], fn2[part], "n2 (GPU's 4-bit records)")
        masks.append(full)
    return masks
