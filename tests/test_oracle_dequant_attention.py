"""Pins of the oracle's dequantisation and attention: an exactly quantisable
special case, the orthonormality identity that ties reconstruction error to the
VQ distortion, and textbook attention checked against torch's softmax."""
import numpy as np
import pytest
import torch

import oracle
from kv_cache_bit_amd import synth

D = 128


def _sign_codebook(seed=0):
    """256 fp16 codewords of dim 4: the 16 patterns {+1,-1}^4 at indices
    0,16,32,... and random others far from them."""
    rng = np.random.default_rng(seed)
    cb = (rng.standard_normal((256, 4)) * 0.3 + 3.0).astype(np.float16)
    pats = np.array([[1.0 if (p >> i) & 1 else -1.0 for i in range(4)] for p in range(16)])
    cb[::16] = pats.astype(np.float16)
    return cb.view(np.uint16), pats


def test_dequant_exact_on_signed_one_hot_tokens():
    """x_t = +-c_t e_i in sign pairs: the block mean is 0, n2 = 1 and
    u = H(sqrt(d) e_i) has entries +-1, which the codebook holds exactly; the
    reconstruction is then x up to the fp16 rounding of n1."""
    R = 8
    cb, pats = _sign_codebook()
    rng = np.random.default_rng(1)
    x = np.zeros((2 * R, D), np.float16)
    for k in range(R // 2):
        i = int(rng.integers(0, D))
        c = float(rng.uniform(0.5, 40.0))
        x[2 * k, i] = c
        x[2 * k + 1, i] = -c * 0.5
    x[R:] = x[:R]
    enc = oracle.encode(x[None], R, cb, with_u=True)
    assert enc["n_quant"] == R
    u = enc["u"][0]
    assert np.allclose(np.abs(u), 1.0, atol=1e-12)
    # every slot's code is the sign pattern of its 4 values
    for t in range(R):
        for j in range(D // 4):
            sub = u[t, 4 * j:4 * j + 4]
            p = sum(1 << e for e in range(4) if sub[e] > 0)
            assert enc["codes"][0, t, j] == 16 * p
    assert np.all(oracle.f16_to_f64(enc["mu"]) == 0.0)
    assert np.all(oracle.f16_to_f64(enc["scales"][..., 1]) == 1.0)
    xh = oracle.dequant(enc["codes"], enc["scales"], enc["mu"], R, cb)[0]
    xd = x[:R].astype(np.float64)
    nz = xd != 0
    assert np.all(np.abs(xh[~nz]) <= 1e-12 * np.abs(xd).max())
    assert np.allclose(xh[nz], xd[nz], rtol=2.0 ** -11, atol=0)


@pytest.mark.parametrize("bits", [2, 1])
def test_reconstruction_error_equals_scaled_vq_distortion(oracle_codebooks, bits):
    """H is orthonormal, so ||x - x_hat|| = n1 n2 ||u - c_hat|| up to the fp16
    rounding of the stored scalars; ||u - c_hat||^2 is the VQ distortion."""
    cb = oracle_codebooks[bits]
    s = cb.shape[1]
    R, L = 64, 257
    x = synth.kv_unit(21, L, D).numpy()
    enc = oracle.encode(x[None], R, cb, with_u=True)
    nq = enc["n_quant"]
    xh = oracle.dequant(enc["codes"], enc["scales"], enc["mu"], R, cb)[0]
    cbd = oracle.f16_to_f64(cb)
    chat = cbd[enc["codes"][0].astype(np.int64)].reshape(nq, D)
    vq_err = np.linalg.norm(enc["u"][0] - chat, axis=1)
    sc = oracle.f16_to_f64(enc["scales"][0])
    pred = sc[:, 0] * sc[:, 1] * vq_err
    got = np.linalg.norm(x[:nq].astype(np.float64) - xh, axis=1)
    assert np.allclose(got, pred, rtol=1e-2)


def _torch_attention(q, K, V, scale):
    qd = torch.from_numpy(q.astype(np.float64))
    Kd, Vd = torch.from_numpy(K), torch.from_numpy(V)
    B, Hq, d = qd.shape
    Hkv = Kd.shape[1]
    Kr = Kd.repeat_interleave(Hq // Hkv, dim=1)
    Vr = Vd.repeat_interleave(Hq // Hkv, dim=1)
    p = torch.softmax(torch.einsum("bhd,bhtd->bht", qd, Kr) * scale, dim=-1)
    return torch.einsum("bht,bhtd->bhd", p, Vr).numpy()


def test_attention_matches_torch_softmax_and_special_cases():
    rng = np.random.default_rng(4)
    B, Hq, Hkv, T = 2, 8, 2, 37
    q = rng.standard_normal((B, Hq, D)).astype(np.float16)
    K = rng.standard_normal((B, Hkv, T, D)) * 2
    V = rng.standard_normal((B, Hkv, T, D))
    sc = 1 / np.sqrt(D)
    out = oracle.attention(q, K, V, sc)
    assert np.allclose(out, _torch_attention(q, K, V, sc), rtol=1e-12, atol=1e-13)
    # one token: the output is that token's value
    o1 = oracle.attention(q, K[:, :, :1], V[:, :, :1], sc)
    assert np.allclose(o1, np.repeat(V[:, :, 0], Hq // Hkv, axis=1), atol=1e-15)
    # zero query: uniform weights, the mean value
    o0 = oracle.attention(np.zeros_like(q), K, V, sc)
    assert np.allclose(o0, np.repeat(V.mean(2), Hq // Hkv, axis=1), atol=1e-13)
    # grouped heads: the same as one call per query head on its KV head
    for h in range(Hq):
        oh = oracle.attention(q[:, h:h + 1], K[:, h // (Hq // Hkv):h // (Hq // Hkv) + 1],
                              V[:, h // (Hq // Hkv):h // (Hq // Hkv) + 1], sc)
        assert np.allclose(oh[:, 0], out[:, h], atol=1e-14)


def test_reference_decode_without_quantised_tokens_is_fp16_attention(oracle_codebooks):
    cb = oracle_codebooks[2]
    R, L = 64, 40
    k = synth.kv_unit(31, L, D).numpy()[None, None]
    v = synth.kv_unit(32, L, D).numpy()[None, None]
    ek, ev = oracle.encode(k, R, cb), oracle.encode(v, R, cb)
    assert ek["n_quant"] == 0 and ek["n_resid"] == L
    q = synth.query_unit(33, D).numpy()[None, None]
    out = oracle.reference_decode(q, ek, ev, 0, L, R, cb)
    ref = _torch_attention(q, k.astype(np.float64), v.astype(np.float64), 1 / np.sqrt(D))
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)
