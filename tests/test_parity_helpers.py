"""CPU checks of the parity helpers themselves, with mistakes planted on the
CPU: a double-quantised cache whose 4-bit decisions differ from the oracle's
in one block is compared against the oracle's re-encode with those
decisions, and a wrong code there is caught; the VQ code check accepts a
near-tie flip to the runner-up and rejects a far code at a near tie, any
change outside the near-tie band, and flips beyond the rate bound; the
attention, dequant and fp16-ulp checks sit at their stated bars.  The caches
live in host memory (the records are plain tensors); no kernel runs."""
import numpy as np
import pytest

from kv_cache_bit_amd import nsnq, synth
from helpers import capacity, compare_encoded_dq, oracle_encode_pair, upload_half
import oracle

D = 128


def _dq_cache(cb, R, L, seed):
    k, v = synth.kv_layer(seed, 0, 1, 2, L, D)
    ek, ev = oracle_encode_pair(k, v, R, cb, dq=True)
    p = nsnq.params(2, R, flags=nsnq.NSNQ_DOUBLE_QUANT)
    cache = nsnq.KVCache(p, 1, 2, capacity(L, R), "cpu")
    upload_half(cache, 0, ek)
    upload_half(cache, 1, ev)
    cache.n_quant, cache.n_resid = ek["n_quant"], ek["n_resid"]
    return cache, ek, ev


def test_dq_block_with_other_decisions(oracle_codebooks):
    cb = oracle_codebooks[2]
    R, L = 64, 4 * 64 + 3
    cache, ek, ev = _dq_cache(cb, R, L, 71)
    assert all(m.all() for m in compare_encoded_dq(cache, ek, ev, R))
    # block 1 of head 0 (K): the s1 step one ulp larger, the way another
    # encoder's rounding of (max - min) / 15 could land, with that block's
    # codes and n2 as the oracle encodes them under the changed record
    sc = cache.k.scales.numpy()
    off = 2 * R + R // 2
    s1 = sc[0, 0, 1, off:off + 2].copy().view(np.uint16)[0] + 1
    sc[0, 0, 1, off:off + 2] = np.array([s1], np.uint16).view(np.uint8)
    nb = ek["n_quant"] // R
    fe = oracle.encode(ek["x"], R, cb, with_u=True, dq=True,
                       force_records=(sc[:, :, :nb].copy(), cache.k.mu.numpy()[:, :, :nb].copy()))
    assert not np.array_equal(fe["n1hat"][0, 0, R:2 * R], ek["n1hat"][0, 0, R:2 * R])
    cache.k.codes.numpy()[0, 0, R:2 * R] = fe["codes"][0, 0, R:2 * R]
    sc[0, 0, 1, :2 * R] = fe["scales"][0, 0, 1, :2 * R]
    masks = compare_encoded_dq(cache, ek, ev, R)
    assert not masks[0][0, 0, 1] and masks[0].sum() == masks[0].size - 1 and masks[1].all()
    # a far-off code in that block is caught by the re-encode comparison
    codes = cache.k.codes.numpy()
    t, j = R + 5, 3
    c = int(codes[0, 0, t, j])
    u = fe["u"][0, 0, t, 4 * j:4 * j + 4]
    c64 = oracle.f16_to_f64(cb)
    far = int(np.argmax(((c64 - u) ** 2).sum(-1)))
    assert far != c
    codes[0, 0, t, j] = far
    with pytest.raises(AssertionError, match="GPU's 4-bit records"):
        compare_encoded_dq(cache, ek, ev, R)


def _near_tie_point(cb_bits, rng):
    """A 4-element point between a codeword and its nearest neighbour, just
    nearer the first: the oracle's gap is far inside the near-tie band."""
    c = oracle.f16_to_f64(cb_bits)
    for _ in range(200):
        a = int(rng.integers(len(c)))
        d = ((c - c[a]) ** 2).sum(-1)
        d[a] = np.inf
        b = int(np.argmin(d))
        u = 0.5 * (c[a] + c[b]) + 1e-7 * (c[a] - c[b])
        code, _, gap = oracle.vq(u, cb_bits)
        if code == a and 0 < gap < 1e-5:
            return u, a, b
    raise AssertionError("no near-tie point found")


def test_check_codes_catches_planted_mistakes(oracle_codebooks):
    """check_codes against codes planted on the CPU: a near-tie flip to the
    runner-up passes; a far code at a near tie, any change outside the band,
    and more flips than the rate bound allows all fail."""
    from helpers import check_codes
    cb = oracle_codebooks[2]
    rng = np.random.default_rng(5)
    n_tok, S, s = 40, 32, 4
    u = rng.standard_normal((n_tok, S * s))
    ties = [(3, 5), (17, 30)]
    runner_up = {}
    for t, j in ties:
        p, a, b = _near_tie_point(cb, rng)
        u[t, s * j:s * (j + 1)] = p
        runner_up[(t, j)] = b
    o = np.zeros((n_tok, S), np.uint8)
    gap = np.zeros((n_tok, S))
    for t in range(n_tok):
        for j in range(S):
            code, _, g = oracle.vq(u[t, s * j:s * (j + 1)], cb)
            o[t, j], gap[t, j] = code, g
    assert all(gap[t, j] < 1e-4 for t, j in ties)

    assert check_codes(o.copy(), o, gap, u, cb) == 0
    g = o.copy()
    g[ties[0]] = runner_up[ties[0]]
    assert check_codes(g, o, gap, u, cb) == 1  # one flip in 1280 codes: within the bound of max(0.0001 n, 1)

    c64 = oracle.f16_to_f64(cb)
    t, j = ties[0]
    far = int(np.argmax(((c64 - u[t, s * j:s * (j + 1)]) ** 2).sum(-1)))
    g = o.copy()
    g[t, j] = far
    with pytest.raises(AssertionError, match="from the best"):
        check_codes(g, o, gap, u, cb)

    t2, j2 = next((t, j) for t in range(n_tok) for j in range(S) if gap[t, j] >= 1e-4)
    g = o.copy()
    g[t2, j2] = (int(o[t2, j2]) + 1) % 256
    with pytest.raises(AssertionError, match="outside the near-tie band"):
        check_codes(g, o, gap, u, cb)

    g = o.copy()
    for tj in ties:
        g[tj] = runner_up[tj]
    with pytest.raises(AssertionError, match="near-tie mismatches"):
        check_codes(g, o, gap, u, cb)
    assert check_codes(g, o, gap, u, cb, pooled=True) == 2


def test_tolerance_checks_sit_at_the_stated_bars():
    """The attention check (2e-3 relative L2 per output row), the dequant check
    (1e-3 of the token norm, max-abs per token) and the one-ulp check of the
    stored fp16 scalars, each against errors planted just inside and just
    outside its bar."""
    from helpers import check_attention, check_dequant, check_f16_ulp
    rng = np.random.default_rng(11)
    o = rng.standard_normal((6, 128))
    e = rng.standard_normal((6, 128))
    e /= np.linalg.norm(e, axis=-1, keepdims=True)
    nrm = np.linalg.norm(o, axis=-1, keepdims=True)
    assert check_attention(o + 1.9e-3 * nrm * e, o) < 2e-3
    bad = o.copy()
    bad[4] += 2.1e-3 * nrm[4] * e[4]
    with pytest.raises(AssertionError, match="attention"):
        check_attention(bad, o)

    x = rng.standard_normal((5, 128))
    norms = np.linalg.norm(x, axis=-1)
    g = x.copy()
    g[:, 7] += 0.9e-3 * norms
    assert check_dequant(g, x, norms) < 1e-3
    g[2, 9] -= 1.1e-3 * norms[2]
    with pytest.raises(AssertionError, match="dequant"):
        check_dequant(g, x, norms)
    # tokens outside the mask (a near-tie flip moved a codeword) are not held to the bar
    assert check_dequant(g, x, norms, mask=np.arange(5) != 2) < 1e-3

    vals = np.abs(rng.standard_normal(4000)).astype(np.float16) + np.float16(0.01)
    ob = vals.view(np.uint16)
    gb = ob.copy()
    gb[:40] += 1  # one ulp up on 1 % of the values
    assert check_f16_ulp(gb, ob, "n1") == 40
    two = ob.copy()
    two[3] += 2
    with pytest.raises(AssertionError, match="exceeds one fp16 ulp"):
        check_f16_ulp(two, ob, "n1")
    many = ob.copy()
    many[:41] += 1
    with pytest.raises(AssertionError, match="off by one ulp"):
        check_f16_ulp(many, ob, "n1")
