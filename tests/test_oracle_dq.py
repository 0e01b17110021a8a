"""Pins of the oracle's double-quantised format (technical summary sec. 3, DQ;
machine review, implementation details: 4-bit round-to-nearest, groups of 32
channels for the mean and of R tokens for s1): the 4-bit quantiser against an
independent nearest-level search and exactly representable groups, the record
layout parsed independently, and the exact inverse that holds because the
forward pass divides by and subtracts the stored values."""
import numpy as np
import pytest
import scipy.linalg

import oracle
from kv_cache_bit_amd import synth

D = 128


def _h(bits) -> float:
    return float(np.array([bits], np.uint16).view(np.float16)[0])


def test_rtn4_exact_grid_and_nearest_level():
    # a group whose levels are exact: Z and S representable, max - min = 15 S
    Z, S = -1.25, 0.0625
    k = np.array([0, 15, 3, 7, 7, 12, 1, 15, 0, 9], np.float64)
    o = oracle.rtn4(Z + S * k)
    assert _h(o["Z"]) == Z and _h(o["S"]) == S
    assert np.array_equal(o["q"], k.astype(np.uint8))
    assert np.array_equal(o["vhat"], Z + S * k)
    assert np.allclose(o["margin"], 0.5)
    # random groups: q is the nearest of the 16 levels (independent search),
    # and the read-back error is at most half a step plus the fp16 rounding
    rng = np.random.default_rng(3)
    for _ in range(50):
        v = rng.standard_normal(32) * rng.uniform(0.01, 30) + rng.uniform(-5, 5)
        o = oracle.rtn4(v)
        Zv, Sv = _h(o["Z"]), _h(o["S"])
        levels = Zv + Sv * np.arange(16)
        near = np.argmin(np.abs(v[:, None] - levels[None, :]), axis=1)
        ok = o["margin"] > 1e-9  # exact ties may round either way
        assert np.array_equal(o["q"][ok], near[ok])
        bound = Sv / 2 + 16 * Sv * 2.0 ** -11 + abs(Zv) * 2.0 ** -11
        assert np.all(np.abs(v - o["vhat"]) <= bound * (1 + 1e-12))
    # a constant group has step 0 and every code 0
    o = oracle.rtn4(np.full(8, 2.5))
    assert _h(o["S"]) == 0.0 and np.all(o["q"] == 0) and np.all(o["vhat"] == 2.5)


def _parse(enc, R):
    """Independent reading of the byte records (layout in include/nsnq.h)."""
    sc, mu = enc["scales"][0], enc["mu"][0]
    nb = sc.shape[0]
    n2 = sc[:, :2 * R].copy().view(np.float16).astype(np.float64)
    nib = sc[:, 2 * R:2 * R + R // 2]
    q1 = np.stack([nib & 15, nib >> 4], axis=-1).reshape(nb, R)
    sz = sc[:, 2 * R + R // 2:2 * R + R // 2 + 4].copy().view(np.float16).astype(np.float64)
    n1hat = sz[:, 1:2] + sz[:, 0:1] * q1
    qm = np.stack([mu[:, :64] & 15, mu[:, :64] >> 4], axis=-1).reshape(nb, D)
    msz = mu[:, 64:80].copy().view(np.float16).astype(np.float64).reshape(nb, 4, 2)
    muhat = msz[:, np.arange(D) // 32, 1] + msz[:, np.arange(D) // 32, 0] * qm
    assert np.all(sc[:, 2 * R + R // 2 + 4:] == 0)
    return n2.reshape(-1), n1hat.reshape(-1), muhat


@pytest.mark.parametrize("bits,R", [(2, 64), (1, 128), (2, 128)])
def test_dq_records_and_exact_inverse(oracle_codebooks, bits, R):
    cb = oracle_codebooks[bits]
    L = 3 * R + 5
    x = synth.kv_unit(51 + bits, L, D).numpy()
    enc = oracle.encode(x[None], R, cb, with_u=True, dq=True)
    nq = enc["n_quant"]
    assert enc["scales"].shape[-1] == oracle.dq_scales_bytes(R) == 16 * -(-(2 * R + R // 2 + 4) // 16)
    n2_st, n1hat, muhat = _parse(enc, R)
    assert np.array_equal(n1hat, enc["n1hat"][0])
    # the forward pass used the stored values: x = n1_hat (n2 H^T u + mu_hat) exactly,
    # with n2 = || x / n1_hat - mu_hat || / sqrt(d) (unrounded)
    Hs = scipy.linalg.hadamard(D).astype(np.float64) / np.sqrt(D)
    xd = x[:nq].astype(np.float64)
    mub = np.repeat(muhat, R, axis=0)
    z = xd / n1hat[:, None] - mub
    n2 = np.linalg.norm(z, axis=1) / np.sqrt(D)
    rec = n1hat[:, None] * (n2[:, None] * (enc["u"][0] @ Hs) + mub)
    assert np.allclose(rec, xd, rtol=0, atol=1e-10 * np.abs(xd).max())
    assert np.allclose(n2_st, n2, rtol=2.0 ** -11)
    # 4-bit codes of s1 and of the mean per group: within half a step (+ fp16 slack)
    n1 = np.linalg.norm(xd, axis=1) / np.sqrt(D)
    for b in range(nq // R):
        span = n1[b * R:(b + 1) * R]
        step = (span.max() - span.min()) / 15
        assert np.all(np.abs(span - n1hat[b * R:(b + 1) * R]) <= step / 2 + 2e-3 * span.max())
    # dequant from the records equals the same formula with the codewords
    xh = oracle.dequant(enc["codes"], enc["scales"], enc["mu"], R, cb, dq=True)[0]
    chat = oracle.f16_to_f64(cb)[enc["codes"][0].astype(np.int64)].reshape(nq, D)
    ref = n1hat[:, None] * (n2_st[:, None] * (chat @ Hs) + mub)
    assert np.allclose(xh, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    # same VQ codes as the plain format would pick for these u, and the
    # reconstruction error is the scaled VQ error
    pred = n1hat * n2_st * np.linalg.norm(enc["u"][0] - chat, axis=1)
    assert np.allclose(np.linalg.norm(xd - xh, axis=1), pred, rtol=1e-2)


@pytest.mark.parametrize("bits,R", [(2, 64), (1, 128)])
def test_dq_forced_records(oracle_codebooks, bits, R):
    """Encoding with given 4-bit records: its own records reproduce the plain
    encode byte for byte; records with some decisions moved by one level are
    taken as given (n1_hat and mu_hat read back from them), and the rest of the
    encode then follows from those values exactly as it does from rounded ones:
    x = n1_hat (n2 H^T u + mu_hat), with the codes the nearest codewords of u."""
    cb = oracle_codebooks[bits]
    L = 3 * R + 7
    x = synth.kv_unit(61 + bits, L, D).numpy()
    enc = oracle.encode(x[None], R, cb, with_u=True, dq=True)
    same = oracle.encode(x[None], R, cb, with_u=True, dq=True, force_records=(enc["scales"], enc["mu"]))
    for k in ("codes", "scales", "mu", "resid", "n1hat", "u"):
        assert np.array_equal(same[k], enc[k]), k
    # move some s1 and mean codes one level (kept within 0..15)
    sc, mu = enc["scales"].copy(), enc["mu"].copy()
    nb = sc.shape[1]
    rng = np.random.default_rng(5)
    for b in range(nb):
        for t in rng.choice(R, 5, replace=False):
            byte = 2 * R + t // 2
            q = (sc[0, b, byte] >> (4 * (t & 1))) & 15
            q2 = q + 1 if q < 15 else q - 1
            sc[0, b, byte] = (sc[0, b, byte] & (0xF0 if t & 1 == 0 else 0x0F)) | (q2 << (4 * (t & 1)))
        for c in rng.choice(D, 7, replace=False):
            q = (mu[0, b, c // 2] >> (4 * (c & 1))) & 15
            q2 = q + 1 if q < 15 else q - 1
            mu[0, b, c // 2] = (mu[0, b, c // 2] & (0xF0 if c & 1 == 0 else 0x0F)) | (q2 << (4 * (c & 1)))
    f = oracle.encode(x[None], R, cb, with_u=True, dq=True, force_records=(sc, mu))
    n2_st, n1hat, muhat = _parse(f, R)
    # the records came through unchanged apart from the n2 bytes
    assert np.array_equal(f["scales"][..., 2 * R:], sc[..., 2 * R:]) and np.array_equal(f["mu"], mu)
    assert np.array_equal(n1hat, f["n1hat"][0])
    assert not np.array_equal(n1hat, enc["n1hat"][0])
    nq = f["n_quant"]
    Hs = scipy.linalg.hadamard(D).astype(np.float64) / np.sqrt(D)
    xd = x[:nq].astype(np.float64)
    mub = np.repeat(muhat, R, axis=0)
    n2 = np.linalg.norm(xd / n1hat[:, None] - mub, axis=1) / np.sqrt(D)
    rec = n1hat[:, None] * (n2[:, None] * (f["u"][0] @ Hs) + mub)
    assert np.allclose(rec, xd, rtol=0, atol=1e-10 * np.abs(xd).max())
    assert np.allclose(n2_st, n2, rtol=2.0 ** -11)
    # codes: the nearest codeword of each sub-vector of u (brute force)
    c64 = oracle.f16_to_f64(cb)
    s = c64.shape[1]
    sub = f["u"][0].reshape(-1, s)
    dist = ((sub[:, None, :] - c64[None, :, :]) ** 2).sum(-1)
    assert np.array_equal(f["codes"][0].reshape(-1), np.argmin(dist, axis=1).astype(np.uint8))


def test_dq_bits_per_element():
    """Overhead of the stored NSN parameters per element (d = 128): at R = 64
    the unpadded records cost 0.238 bits (n2 fp16, s1 in 4 bits with its
    (S, Z) per R tokens, the mean in 4 bits with (S, Z) per 32 channels); the
    pages quote about 0.23.  The 16-byte padded records used here cost 0.250
    (R = 64) and 0.203 (R = 128)."""
    def over(R, padded):
        sc = oracle.dq_scales_bytes(R) if padded else 2 * R + R // 2 + 4
        return 8 * (sc + oracle.DQ_MU_BYTES) / (R * D)
    assert abs(over(64, False) - 0.2383) < 1e-3
    assert abs(over(64, True) - 0.25) < 1e-12
    assert abs(over(128, True) - 0.203125) < 1e-12


def test_dq_degenerate_blocks(oracle_codebooks):
    """A block of identical tokens (zero mean step after the shift) and a zero
    token: finite, and reconstructed from the records."""
    cb = oracle_codebooks[2]
    R = 64
    x = synth.kv_unit(61, 3 * R + 1, D).numpy()
    x[R:2 * R] = x[R]
    x[5] = 0
    enc = oracle.encode(x[None], R, cb, dq=True)
    xh = oracle.dequant(enc["codes"], enc["scales"], enc["mu"], R, cb, dq=True)[0]
    assert np.all(np.isfinite(xh))
    assert np.all(xh[5] == 0)
    # the constant block reconstructs to its token up to the 4-bit mean and VQ of the remainder
    blk = x[R:2 * R].astype(np.float64)
    err = np.linalg.norm(xh[R:2 * R] - blk, axis=1) / np.linalg.norm(blk, axis=1)
    assert err.max() < 0.5


def _parse_codebook_record(rec, n, group):
    """Independent reading of a codebook record: n/2 bytes of 4-bit codes
    (entry i: byte i/2, low nibble for even i), then (S, Z) fp16 per group."""
    nib = rec[:n // 2]
    q = np.stack([nib & 15, nib >> 4], axis=-1).reshape(n)
    sz = rec[n // 2:].copy().view(np.float16).astype(np.float64).reshape(n // group, 2)
    return q, sz[:, 0], sz[:, 1]


@pytest.mark.parametrize("bits", [2, 1])
def test_codebook_dq_nearest_level_and_layout(oracle_codebooks, bits):
    """The codebook entries in 4 bits (technical summary sec. 3, DQ): each
    group of 32 consecutive entries has Z = fp16(min), S = fp16(range / 15);
    every code is the nearest of the group's 16 levels (independent search),
    the read-back codebook is fp16(Z + S q), and it stays within half a step
    (plus the fp16 roundings) of the input."""
    cb = oracle_codebooks[bits]
    n = cb.size
    o = oracle.codebook_dq(cb, 32)
    assert o["record"].size == n // 2 + 4 * (n // 32)
    q, S, Z = _parse_codebook_record(o["record"], n, 32)
    v = cb.reshape(-1).view(np.float16).astype(np.float64)
    g = np.arange(n) // 32
    vg = v.reshape(-1, 32)
    assert np.array_equal(Z, vg.min(1).astype(np.float16).astype(np.float64))
    assert np.array_equal(S, ((vg.max(1) - vg.min(1)) / 15).astype(np.float16).astype(np.float64))
    levels = Z[:, None] + S[:, None] * np.arange(16)[None, :]
    near = np.argmin(np.abs(v[:, None] - levels[g]), axis=1)
    ok = o["margin"].reshape(-1) > 1e-9
    assert np.array_equal(q[ok], near[ok])
    hat = (Z[g] + S[g] * q).astype(np.float16)
    assert np.array_equal(o["cb_hat"].reshape(-1), hat.view(np.uint16))
    err = np.abs(hat.astype(np.float64) - v)
    assert np.all(err <= S[g] / 2 + 2.0 ** -11 * (np.abs(v) + 16 * S[g]) + 2.0 ** -24)
    # the codebook keeps its shape; 4-bit codes cost 0.5 B per entry
    assert o["cb_hat"].shape == cb.shape


def test_codebook_dq_exact_grid_duplicates_and_constant_group():
    """A codebook whose groups sit exactly on 4-bit grids comes back bit for
    bit; a constant group has step 0 (every code 0, value kept); duplicated
    codewords stay duplicated."""
    rng = np.random.default_rng(11)
    n = 256 * 4
    Z = rng.integers(-64, 0, n // 32) / 16.0          # multiples of 1/16
    S = rng.integers(1, 8, n // 32) / 64.0            # multiples of 1/64
    k = rng.integers(0, 16, (n // 32, 32))
    k[:, 0], k[:, 1] = 0, 15                            # span the whole range
    vals = (Z[:, None] + S[:, None] * k).reshape(256, 4)
    vals[40:48] = 0.75                                  # a constant group (entries 160..191)
    vals[3] = vals[2]                                   # duplicated codewords
    cb = vals.astype(np.float16)
    assert np.array_equal(cb.astype(np.float64), vals)
    o = oracle.codebook_dq(cb.view(np.uint16), 32)
    assert np.array_equal(o["cb_hat"], cb.view(np.uint16))
    q, Sq, Zq = _parse_codebook_record(o["record"], n, 32)
    kk = k.reshape(-1).copy()
    const = np.arange(n) // 32 == 5
    assert Sq[5] == 0.0 and Zq[5] == 0.75 and np.all(q[const] == 0)
    grid = ~const
    grid[8:16] = False   # codewords 2 and 3 (entries 8..15) were overwritten
    assert np.array_equal(q[grid], kk[grid])
    hat = o["cb_hat"].view(np.float16).reshape(256, 4)
    assert np.array_equal(hat[2], hat[3])
