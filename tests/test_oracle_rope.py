"""Pins of the oracle's rotary embedding of keys stored before RoPE
(technical summary sec. 4, Attention Computation): identity at position 0,
an independent complex-number formulation, norm preservation and the
relative-position property of the standard tables, and the pre-RoPE
reference decode against attention over explicitly rotated keys."""
import numpy as np
import torch

import oracle
from kv_cache_bit_amd import synth

D = 128


def test_rope_identity_complex_form_and_norms():
    cos, sin = synth.rope_tables(300, 10000.0, D)
    rng = np.random.default_rng(0)
    k = rng.standard_normal((2, 17, D))
    # position 0 is the identity
    assert np.array_equal(oracle.rope(k[:, :1], cos, sin, 0), k[:, :1])
    # complex form: (k_c + i k_{c+64}) * (cos + i sin)
    pos0 = 101
    r = oracle.rope(k, cos, sin, pos0)
    z = (k[..., :64] + 1j * k[..., 64:]) * (cos.numpy()[pos0:pos0 + 17].astype(np.float64)
                                            + 1j * sin.numpy()[pos0:pos0 + 17].astype(np.float64))
    assert np.allclose(r[..., :64], z.real, atol=1e-12) and np.allclose(r[..., 64:], z.imag, atol=1e-12)
    # rotations keep norms (up to the fp32 rounding of the tables)
    assert np.allclose(np.linalg.norm(r, axis=-1), np.linalg.norm(k, axis=-1), rtol=1e-6)


def test_rope_scores_depend_on_relative_position_only():
    cos, sin = synth.rope_tables(400, 10000.0, D)
    rng = np.random.default_rng(1)
    q = rng.standard_normal(D)
    k = rng.standard_normal((1, 20, D))
    s = []
    for shift in (0, 57, 180):
        qr = oracle.rope(q[None, None], cos, sin, 150 + shift)[0, 0]
        kr = oracle.rope(k, cos, sin, 10 + shift)[0]
        s.append(kr @ qr)
    assert np.allclose(s[0], s[1], rtol=1e-5, atol=1e-5) and np.allclose(s[0], s[2], rtol=1e-5, atol=1e-5)


def test_prerope_reference_decode_is_attention_over_rotated_keys(oracle_codebooks):
    cb = oracle_codebooks[2]
    R, L, pos0 = 64, 200, 5
    cos, sin = synth.rope_tables(L + pos0, 10000.0, D)
    k = synth.kv_unit(71, L, D).numpy()[None, None]
    v = synth.kv_unit(72, L, D).numpy()[None, None]
    ek, ev = oracle.encode(k, R, cb), oracle.encode(v, R, cb)
    q = synth.query_unit(73, D).numpy()[None, None]
    out = oracle.reference_decode(q, ek, ev, ek["n_quant"], ek["n_resid"], R, cb, rope_tables=(cos, sin), pos0=pos0)
    K = np.concatenate([oracle.dequant(ek["codes"], ek["scales"], ek["mu"], R, cb),
                        oracle.f16_to_f64(ek["resid"][..., :ek["n_resid"], :])], axis=-2)
    V = np.concatenate([oracle.dequant(ev["codes"], ev["scales"], ev["mu"], R, cb),
                        oracle.f16_to_f64(ev["resid"][..., :ev["n_resid"], :])], axis=-2)
    kr = oracle.rope(K, cos, sin, pos0)
    qd = torch.from_numpy(q.astype(np.float64))
    p = torch.softmax(torch.from_numpy(kr[0, 0]) @ qd[0, 0] / np.sqrt(D), dim=0)
    ref = (p[:, None] * torch.from_numpy(V[0, 0])).sum(0).numpy()
    assert np.allclose(out[0, 0], ref, rtol=1e-12, atol=1e-12)
    # and it differs from the decode that ignores the rotation
    plain = oracle.reference_decode(q, ek, ev, ek["n_quant"], ek["n_resid"], R, cb)
    assert not np.allclose(plain, out, rtol=1e-3)
