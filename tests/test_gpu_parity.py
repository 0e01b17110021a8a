"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle
on the same seeded inputs."""
import math

import numpy as np
import pytest
import torch

import oracle
from kv_cache_bit_amd import nsnq, synth

from helpers import (DEV, capacity, check_attention, check_codes, check_dequant, check_f16_ulp, check_tie_rate,
                     compare_encoded_dq,
                     compare_encoded, f16_bits, gpu_encode, gpu_records, half_np, oracle_encode, oracle_encode_pair,
                     token_norms, upload_half, cb_tensor)

pytestmark = pytest.mark.gpu

D = 128


def _kv(config_id, B, H, L, outlier=10.0):
    return synth.kv_layer(config_id, 0, B, H, L, D, outlier_std=outlier)


# ------------------------------------------------------------------ encode --

@pytest.mark.parametrize("bits,R,B,H,L", [
    (2, 64, 1, 1, 512),     # the tiny workload
    (2, 128, 2, 3, 300),    # ragged: 256 encoded, 44 residual
    (1, 128, 1, 2, 385),
    (1, 64, 2, 1, 200),
    (2, 64, 1, 1, 64),      # everything stays in the residual window
    (2, 128, 1, 2, 1),
])
def test_encode_matches_oracle(oracle_codebooks, bits, R, B, H, L):
    cb = oracle_codebooks[bits]
    k, v = _kv(100 + bits, B, H, L)
    p, cbt, cache = gpu_encode(k, v, bits, R, cb)
    ek, ev = oracle_encode_pair(k, v, R, cb)
    assert (cache.n_quant, cache.n_resid) == (ek["n_quant"], ek["n_resid"])
    compare_encoded(cache, ek, ev)


def test_encode_degenerate_tokens(oracle_codebooks):
    """A zero token (n1 = 0) and a block of identical tokens (n2 = 0)."""
    cb = oracle_codebooks[2]
    R = 64
    k, v = _kv(7, 1, 1, 3 * R + 5)
    k[0, 0, 10] = 0
    v[0, 0, R:2 * R] = v[0, 0, R]
    p, cbt, cache = gpu_encode(k, v, 2, R, cb)
    ek, ev = oracle_encode_pair(k, v, R, cb)
    compare_encoded(cache, ek, ev)
    assert np.all(half_np(cache, 1)["scales"][0, 0, R:2 * R, 1] == 0)  # n2 = 0 stored
    assert np.all(half_np(cache, 0)["scales"][0, 0, 10, 0] == 0)


# ------------------------------------------------ candidate-list encode --

@pytest.mark.parametrize("R,B,H,L,flags,use_signs", [
    (64, 1, 1, 512, 0, False),
    (128, 2, 3, 300, 0, False),
    (128, 1, 2, 1000, nsnq.NSNQ_DOUBLE_QUANT, False),
    (128, 2, 2, 700, nsnq.NSNQ_SCALE_ADJUST, True),
    (64, 1, 2, 450, nsnq.NSNQ_DOUBLE_QUANT | nsnq.NSNQ_SCALE_ADJUST, True),
])
def test_encode_candidate_lists(oracle_codebooks, R, B, H, L, flags, use_signs):
    """2 bits, searching only the orthant box's candidate list: the oracle's
    codes and scalars under the same bars as the exhaustive search, and the
    same codes as the exhaustive GPU search outside the near-tie band."""
    cb = oracle_codebooks[2]
    k, v = _kv(150 + L, B, H, L)
    signs = synth.hadamard_signs(15 + R) if use_signs else None
    adjust = bool(flags & nsnq.NSNQ_SCALE_ADJUST)
    p, cbt, cache = gpu_encode(k, v, 2, R, cb, flags=flags, signs=signs, cand=True)
    assert p.vq_span in (64, 80, 96)
    _, _, full = gpu_encode(k, v, 2, R, cb, flags=flags, signs=signs)
    dq = bool(flags & nsnq.NSNQ_DOUBLE_QUANT)
    kw = dict(signs=None if signs is None else signs.numpy(), scale_adjust=adjust, dq=dq)
    ek, ev = oracle_encode_pair(k, v, R, cb, **kw)
    if dq:
        compare_encoded_dq(cache, ek, ev, R, scale_adjust=adjust)
    else:
        compare_encoded(cache, ek, ev, scale_adjust=adjust)
    for which, e in ((0, ek), (1, ev)):
        g, f = half_np(cache, which)["codes"], half_np(full, which)["codes"]
        assert not np.any((g != f) & (e["gap"] >= 1e-4)), "pruned and exhaustive codes differ away from a tie"
    # decode reads the list-encoded cache as usual: against the oracle's
    # attention over the GPU cache's own records (every case, double-quantised
    # ones included), over the oracle's records placed in a GPU cache, and end
    # to end where every code equals the oracle's
    q = synth.queries(150 + L, 0, B, 2 * H, D)
    o = nsnq.nsnq_decode_attention(p, cbt, q.to(DEV), cache).float().cpu().numpy()
    gk, gv = gpu_records(cache, 0), gpu_records(cache, 1)
    check_attention(o, oracle.reference_decode(q, gk, gv, cache.n_quant, cache.n_resid, R, cb, signs=kw["signs"]))
    ref = oracle.reference_decode(q, ek, ev, ek["n_quant"], ek["n_resid"], R, cb, signs=kw["signs"])
    oc = nsnq.KVCache(p, B, H, capacity(L, R), DEV)
    upload_half(oc, 0, ek)
    upload_half(oc, 1, ev)
    oc.n_quant, oc.n_resid = ek["n_quant"], ek["n_resid"]
    check_attention(nsnq.nsnq_decode_attention(p, cbt, q.to(DEV), oc).float().cpu().numpy(), ref)
    same = all(np.array_equal(half_np(cache, w)["codes"], e["codes"]) for w, e in ((0, ek), (1, ev)))
    if same and not dq:
        check_attention(o, ref)


def test_encode_candidate_list_spans(oracle_codebooks):
    """Every list-kernel variant: a constructed codebook whose lists hold 16
    entries (the 16 points {+-1}^4; the other 240 words lie far outside the
    region u can reach and are on no list) runs the 64-entry kernel; the
    k-means codebook runs with its own span and with the span forced to 96
    (searching repeated padding entries is still exact)."""
    R, B, H, L = 128, 1, 4, 3 * 128 + 17
    k, v = _kv(170, B, H, L)
    grid = np.array([[1.0 if (i >> e) & 1 else -1.0 for e in range(4)] for i in range(16)])
    far = 40.0 + np.arange(240)[:, None] * 0.25 + np.zeros((240, 4))
    cb_grid = np.concatenate([grid, far]).astype(np.float16).view(np.uint16)
    cases = [(cb_grid, None), (oracle_codebooks[2], None), (oracle_codebooks[2], 96)]
    for cb, force in cases:
        cbt = cb_tensor(cb)
        p = nsnq.with_candidates(nsnq.params(2, R), cbt)
        if cb is cb_grid:
            assert p.vq_span == 16
        if force is not None:
            p.vq_span = force
        cache = nsnq.KVCache(p, B, H, capacity(L, R), DEV)
        nsnq.nsnq_encode_kv(p, cbt, k.to(DEV), v.to(DEV), L, cache)
        torch.cuda.synchronize()
        ek, ev = oracle_encode_pair(k, v, R, cb)
        compare_encoded(cache, ek, ev)


def test_encode_candidate_lists_degenerate(oracle_codebooks):
    """A zero token, a constant block (n2 = 0: u = 0 on every box's faces) and
    a ragged prefill with a window flush, all through the candidate lists."""
    cb = oracle_codebooks[2]
    R = 64
    k, v = _kv(8, 1, 1, 3 * R + 5)
    k[0, 0, 10] = 0
    v[0, 0, R:2 * R] = v[0, 0, R]
    p, cbt, cache = gpu_encode(k, v, 2, R, cb, cand=True)
    ek, ev = oracle_encode_pair(k, v, R, cb)
    compare_encoded(cache, ek, ev)
    assert np.all(half_np(cache, 1)["scales"][0, 0, R:2 * R, 1] == 0)
    # R = 128: a constant block puts all 4096 sub-vectors in one box (128
    # column blocks), next to an ordinary block
    k2, v2 = _kv(9, 1, 1, 3 * 128 + 1)
    v2[0, 0, 128:256] = v2[0, 0, 128]
    p2, _, cache2 = gpu_encode(k2, v2, 2, 128, cb, cand=True)
    e2k, e2v = oracle_encode_pair(k2, v2, 128, cb)
    compare_encoded(cache2, e2k, e2v)
    assert np.all(half_np(cache2, 1)["scales"][0, 0, 128:256, 1] == 0)
    # ragged rows, then appends that flush a full window through the lists
    lengths = [0, R, 2 * R + 3]
    kk, vv = _kv(9, 3, 2, 3 * R + 2)
    pc = nsnq.with_candidates(nsnq.params(2, R), cbt)
    rc = nsnq.KVCache(pc, 3, 2, 4 * R, DEV, ragged=True)
    nsnq.nsnq_encode_kv_ragged(pc, cbt, kk.to(DEV), vv.to(DEV), torch.tensor(lengths, dtype=torch.int32, device=DEV),
                               max(lengths), rc)
    for i in range(2):
        idx = torch.tensor([Lb + i for Lb in lengths])
        nsnq.nsnq_append_kv(pc, cbt, kk[torch.arange(3), :, idx].contiguous().to(DEV),
                            vv[torch.arange(3), :, idx].contiguous().to(DEV), rc)
    torch.cuda.synchronize()
    flips = total = 0
    for b, Lb in enumerate(lengths):
        e_k = oracle_encode(kk[b:b + 1, :, :Lb + 2], R, cb)
        e_v = oracle_encode(vv[b:b + 1, :, :Lb + 2], R, cb)
        assert (rc.seq_quant[b].item(), rc.seq_resid[b].item()) == (e_k["n_quant"], e_k["n_resid"])
        f, t = _check_row(rc, b, e_k, e_v)
        flips, total = flips + f, total + t
    check_tie_rate(flips, total)


# ----------------------------------------------------------------- dequant --

@pytest.mark.parametrize("bits,R", [(2, 64), (1, 128)])
def test_dequant_same_cache(oracle_codebooks, bits, R):
    """GPU reconstruction of the oracle's own cache."""
    cb = oracle_codebooks[bits]
    B, H, L = 2, 2, 5 * R + 7
    k, v = _kv(200 + bits, B, H, L)
    ek, ev = oracle_encode_pair(k, v, R, cb)
    p = nsnq.params(bits, R)
    cache = nsnq.KVCache(p, B, H, capacity(L, R), DEV)
    upload_half(cache, 0, ek)
    upload_half(cache, 1, ev)
    cache.n_quant, cache.n_resid = ek["n_quant"], ek["n_resid"]
    cbt = cb_tensor(cb)
    nq = ek["n_quant"]
    for which, e, x in ((0, ek, k), (1, ev, v)):
        ref = oracle.dequant(e["codes"], e["scales"], e["mu"], R, cb)
        norms = token_norms(x[:, :, :nq].numpy())
        g32 = nsnq.nsnq_dequant(p, cbt, cache, which, 0, nq, torch.float32).cpu().numpy()
        assert check_dequant(g32, ref, norms) < 1e-5
        g16 = nsnq.nsnq_dequant(p, cbt, cache, which, 0, nq, torch.float16).cpu().numpy()
        check_dequant(g16, ref, norms)
        # a sub-range
        t0, nt = R + 3, 2 * R
        gs = nsnq.nsnq_dequant(p, cbt, cache, which, t0, nt, torch.float32).cpu().numpy()
        assert np.allclose(gs, g32[:, :, t0:t0 + nt], atol=0, rtol=0)


@pytest.mark.parametrize("bits,R", [(2, 128), (1, 64)])
def test_dequant_end_to_end(oracle_codebooks, bits, R):
    cb = oracle_codebooks[bits]
    B, H, L = 1, 3, 4 * R + 1
    k, v = _kv(300 + bits, B, H, L)
    p, cbt, cache = gpu_encode(k, v, bits, R, cb)
    ek, ev = oracle_encode_pair(k, v, R, cb)
    nq = ek["n_quant"]
    for which, e, x in ((0, ek, k), (1, ev, v)):
        g = nsnq.nsnq_dequant(p, cbt, cache, which, 0, nq, torch.float32).cpu().numpy()
        ref = oracle.dequant(e["codes"], e["scales"], e["mu"], R, cb)
        same = np.all(half_np(cache, which)["codes"] == e["codes"], axis=-1)
        check_dequant(g, ref, token_norms(x[:, :, :nq].numpy()), mask=same)


# --------------------------------------------------------------- attention --

def _decode_ref(q, ek, ev, cb, R):
    return oracle.reference_decode(q.cpu(), ek, ev, ek["n_quant"], ek["n_resid"], R, cb)


@pytest.mark.parametrize("bits,R,B,Hq,Hkv,L", [
    (2, 64, 1, 1, 1, 512),
    (2, 128, 2, 4, 4, 700),
    (1, 128, 1, 8, 2, 1000),   # grouped query heads, G = 4
    (2, 64, 1, 6, 3, 333),     # G = 2
    (2, 128, 1, 8, 1, 300),    # G = 8 (two head groups per KV head)
    (2, 64, 2, 2, 2, 40),      # residual tokens only
    (2, 128, 1, 16, 1, 300),   # G = 16: one matrix-core column per head
    (1, 64, 1, 32, 1, 200),    # G = 32: two 16-head groups
    (2, 64, 1, 12, 2, 333),    # G = 6: LUT kernel, 3 groups of 2
    (1, 128, 2, 8, 4, 129),    # G = 2, one residual token
    (2, 128, 1, 8, 2, 100),    # G = 4, residual tokens only (no wave has a chunk)
    (1, 64, 2, 4, 2, 50),      # G = 2, residual tokens only
    (1, 64, 1, 16, 4, 333),    # G = 4 at 1 bit: 8-channel codewords as two 4x4x4 slices
    (1, 128, 2, 3, 3, 700),    # G = 1 at 1 bit: the value sum on the matrix cores
])
def test_decode_same_cache_and_end_to_end(oracle_codebooks, bits, R, B, Hq, Hkv, L):
    cb = oracle_codebooks[bits]
    k, v = _kv(400 + bits, B, Hkv, L)
    q = synth.queries(400 + bits, 0, B, Hq, D)
    ek, ev = oracle_encode_pair(k, v, R, cb)
    ref = _decode_ref(q, ek, ev, cb, R)
    p = nsnq.params(bits, R)
    cbt = cb_tensor(cb)
    # same cache: the oracle's encoding, attended on the GPU
    cache = nsnq.KVCache(p, B, Hkv, capacity(L, R), DEV)
    upload_half(cache, 0, ek)
    upload_half(cache, 1, ev)
    cache.n_quant, cache.n_resid = ek["n_quant"], ek["n_resid"]
    qd = q.to(DEV)
    outs = []
    for ns in (0, 1, 3, 40):  # 40: more splits than blocks (one block each)
        o = nsnq.nsnq_decode_attention(p, cbt, qd, cache, num_splits=ns).float().cpu().numpy()
        check_attention(o, ref)
        outs.append(o)
    for o in outs[1:]:
        assert np.allclose(o, outs[0], atol=2e-3 * np.abs(outs[0]).max())
    # end to end: GPU encode, GPU decode
    _, _, gcache = gpu_encode(k, v, bits, R, cb)
    o = nsnq.nsnq_decode_attention(p, cbt, qd, gcache).float().cpu().numpy()
    check_attention(o, ref)


@pytest.mark.parametrize("bits,Hq,Hkv", [(2, 8, 2), (1, 8, 2), (2, 4, 2)])
def test_decode_late_maxima(oracle_codebooks, bits, Hq, Hkv):
    """Tokens far into each split whose keys point along one query head, with
    growing norms: that head's running maximum has to move several times after
    the first chunk, and the accumulated values be rescaled each time."""
    cb = oracle_codebooks[bits]
    R, B, L = 128, 1, 1700
    k, v = _kv(470 + bits, B, Hkv, L)
    q = synth.queries(470 + bits, 0, B, Hq, D)
    G = Hq // Hkv
    for hk in range(Hkv):
        d = q[0, hk * G].float()
        d = d / d.norm()
        for i, t in enumerate((300, 700, 1100, 1450)):
            k[0, hk, t] = (d * (4.0 * 2 ** i) * k[0, hk, t].float().norm()).half()
    ek, ev = oracle_encode_pair(k, v, R, cb)
    ref = _decode_ref(q, ek, ev, cb, R)
    p = nsnq.params(bits, R)
    cbt = cb_tensor(cb)
    cache = nsnq.KVCache(p, B, Hkv, capacity(L, R), DEV)
    upload_half(cache, 0, ek)
    upload_half(cache, 1, ev)
    cache.n_quant, cache.n_resid = ek["n_quant"], ek["n_resid"]
    qd = q.to(DEV)
    for ns in (0, 1, 2, 5):
        o = nsnq.nsnq_decode_attention(p, cbt, qd, cache, num_splits=ns).float().cpu().numpy()
        check_attention(o, ref)


@pytest.mark.parametrize("bits,Hq,Hkv", [(2, 2, 2), (2, 8, 2), (1, 4, 4)])
def test_decode_many_splits(oracle_codebooks, bits, Hq, Hkv):
    """More split partials than one combine batch holds (32): with one block per
    split the combine merges 63 partials in two batches, and keys late in the
    context pointing along a query head put that head's maximum in the second
    batch, so the sums of the first are rescaled between batches."""
    cb = oracle_codebooks[bits]
    R, B, L = 64, 1, 4000
    k, v = _kv(480 + bits, B, Hkv, L)
    q = synth.queries(480 + bits, 0, B, Hq, D)
    G = Hq // Hkv
    for hk in range(Hkv):
        d = q[0, hk * G].float()
        d = d / d.norm()
        for i, t in enumerate((2500, 3300, 3900)):
            k[0, hk, t] = (d * (4.0 * 2 ** i) * k[0, hk, t].float().norm()).half()
    ek, ev = oracle_encode_pair(k, v, R, cb)
    assert ek["n_quant"] // R == 62
    ref = _decode_ref(q, ek, ev, cb, R)
    p = nsnq.params(bits, R)
    cbt = cb_tensor(cb)
    cache = nsnq.KVCache(p, B, Hkv, capacity(L, R), DEV)
    upload_half(cache, 0, ek)
    upload_half(cache, 1, ev)
    cache.n_quant, cache.n_resid = ek["n_quant"], ek["n_resid"]
    qd = q.to(DEV)
    for ns in (62, 21, 0):  # 63, 22 and the planner's partials
        o = nsnq.nsnq_decode_attention(p, cbt, qd, cache, num_splits=ns).float().cpu().numpy()
        check_attention(o, ref)


@pytest.mark.parametrize("bits,Hq,Hkv", [(2, 1, 1), (2, 4, 1), (2, 8, 1), (1, 1, 1), (1, 4, 1), (2, 32, 1)])
@pytest.mark.parametrize("case", ["small_v_sink", "huge_v_token"])
def test_decode_weight_range(oracle_codebooks, bits, Hq, Hkv, case):
    """Value weights at both ends of the fp16 range, in every decode kernel
    (LUT with FMA values, LUT with matrix-core values at 1 bit, grouped heads
    with one token per lane and with 16-token tiles):
      small_v_sink: values of RMS 1e-2 and one key along every query, so one
        token takes nearly all the softmax weight and each other token of the
        2048-token split gets p ~ 1e-5; their p N1 N2 and p N1 fall below the
        fp16 subnormals unless scaled, and their mean term is ~1% of the output;
      huge_v_token: a value vector of norm 4e5 (N1 N2 above the fp16 maximum).
    One split holds all 2048 quantised tokens."""
    cb = oracle_codebooks[bits]
    R, B, L = 128, 1, 2049
    k, v = _kv(560 + bits, B, Hkv, L)
    q = synth.queries(560 + bits, 0, B, Hq, D)
    G = Hq // Hkv
    if case == "small_v_sink":
        vf = v.float()
        v = (vf * (1e-2 / vf.pow(2).mean().sqrt())).half()
        kf = k.float()
        k = (kf / kf.norm(dim=-1).mean()).half()  # key norms ~1: scores of order 1
        for hk in range(Hkv):
            qs = q[0, hk * G:(hk + 1) * G].float()
            dirn = qs.sum(0) / qs.sum(0).norm()
            k[0, hk, 700] = (dirn * 12.0 * G ** 0.5).half()  # score ~12 for each head
    else:
        sgn = torch.where(torch.arange(D) % 3 == 0, -1.0, 1.0)
        v[0, :, 900] = (sgn * 4e5 / np.sqrt(D)).half()
        assert float(v[0, 0, 900].float().norm()) > 3.7e5
    ek, ev = oracle_encode_pair(k, v, R, cb)
    assert ek["n_quant"] == 2048
    ref = _decode_ref(q, ek, ev, cb, R)
    assert np.all(np.isfinite(ref))
    p = nsnq.params(bits, R)
    cbt = cb_tensor(cb)
    cache = nsnq.KVCache(p, B, Hkv, capacity(L, R), DEV)
    upload_half(cache, 0, ek)
    upload_half(cache, 1, ev)
    cache.n_quant, cache.n_resid = ek["n_quant"], ek["n_resid"]
    o = nsnq.nsnq_decode_attention(p, cbt, q.to(DEV), cache, num_splits=1).float().cpu().numpy()
    assert np.all(np.isfinite(o))
    check_attention(o, ref)
    # end to end: the GPU's own encoding, attended, against the oracle's
    # attention over the same records
    _, _, gc = gpu_encode(k, v, bits, R, cb)
    o = nsnq.nsnq_decode_attention(p, cbt, q.to(DEV), gc, num_splits=1).float().cpu().numpy()
    check_attention(o, oracle.reference_decode(q, gpu_records(gc, 0), gpu_records(gc, 1), gc.n_quant,
                                               gc.n_resid, R, cb))


def test_decode_workspace_reuse(oracle_codebooks):
    """One workspace serves calls of different shapes, kernels (one KV head per
    query head, and grouped heads) and split counts in turn; every result
    matches the oracle's attention."""
    cases = []
    for bits, R, B, Hq, Hkv, L in ((2, 128, 2, 4, 4, 1500), (1, 64, 1, 8, 2, 700), (2, 64, 3, 3, 3, 900)):
        cb = oracle_codebooks[bits]
        k, v = _kv(480 + bits + B, B, Hkv, L)
        q = synth.queries(480 + bits + B, 0, B, Hq, D)
        ek, ev = oracle_encode_pair(k, v, R, cb)
        p = nsnq.params(bits, R)
        cache = nsnq.KVCache(p, B, Hkv, capacity(L, R), DEV)
        upload_half(cache, 0, ek)
        upload_half(cache, 1, ev)
        cache.n_quant, cache.n_resid = ek["n_quant"], ek["n_resid"]
        cases.append((p, cb_tensor(cb), q.to(DEV), cache, _decode_ref(q, ek, ev, cb, R)))
    need = max(nsnq.nsnq_decode_workspace_bytes(p, c, q.shape[1], ns)
               for p, _, q, c, _ in cases for ns in (0, 1, 7))
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    for ns in (0, 7, 1, 0):
        for p, cbt, qd, cache, ref in cases:
            o = nsnq.nsnq_decode_attention(p, cbt, qd, cache, num_splits=ns, ws=ws).float().cpu().numpy()
            check_attention(o, ref)


def test_flush_then_decode(oracle_codebooks):
    """Prefill leaves a full window; the next token flushes it, is appended,
    and attention covers all tokens."""
    cb = oracle_codebooks[2]
    R, B, H = 64, 1, 2
    L = 3 * R
    k, v = _kv(500, B, H, L + 1)
    p, cbt, cache = gpu_encode(k[:, :, :L], v[:, :, :L], 2, R, cb, cap=8 * R)
    assert (cache.n_quant, cache.n_resid) == (2 * R, R)
    nsnq.nsnq_flush_residual(p, cbt, cache)
    assert (cache.n_quant, cache.n_resid) == (3 * R, 0)
    nsnq.nsnq_append_kv(p, cbt, k[:, :, L].contiguous().to(DEV), v[:, :, L].contiguous().to(DEV), cache)
    torch.cuda.synchronize()
    ek, ev = oracle_encode_pair(k, v, R, cb)   # L + 1 tokens: 3R encoded, 1 residual
    assert ek["n_quant"] == 3 * R
    compare_encoded(cache, ek, ev)
    q = synth.queries(500, 0, B, H, D)
    o = nsnq.nsnq_decode_attention(p, cbt, q.to(DEV), cache).float().cpu().numpy()
    check_attention(o, _decode_ref(q, ek, ev, cb, R))


# ------------------------------------------- randomised Hadamard, Strategy 3 --

@pytest.mark.parametrize("bits,R,use_signs,adjust", [
    (2, 64, True, False),
    (2, 128, False, True),
    (2, 128, True, True),
    (1, 128, True, True),
])
def test_rht_and_scale_adjust(oracle_codebooks, bits, R, use_signs, adjust):
    """Encode, dequant and decode with a sign vector and/or Strategy 3."""
    cb = oracle_codebooks[bits]
    B, Hq, Hkv, L = 2, 4, 2, 5 * R + 9
    k, v = _kv(600 + bits, B, Hkv, L)
    q = synth.queries(600 + bits, 0, B, Hq, D)
    signs = synth.hadamard_signs(60 + bits) if use_signs else None
    flags = nsnq.NSNQ_SCALE_ADJUST if adjust else 0
    p, cbt, cache = gpu_encode(k, v, bits, R, cb, flags=flags, signs=signs)
    ek, ev = oracle_encode_pair(k, v, R, cb, signs=signs, scale_adjust=adjust)
    compare_encoded(cache, ek, ev, scale_adjust=adjust)
    nq = ek["n_quant"]
    for which, e, x in ((0, ek, k), (1, ev, v)):
        g = nsnq.nsnq_dequant(p, cbt, cache, which, 0, nq, torch.float32).cpu().numpy()
        ref = oracle.dequant(e["codes"], e["scales"], e["mu"], R, cb, signs=signs)
        same = np.all(half_np(cache, which)["codes"] == e["codes"], axis=-1)
        check_dequant(g, ref, token_norms(x[:, :, :nq].numpy()), mask=same)
    ref = oracle.reference_decode(q, ek, ev, nq, ek["n_resid"], R, cb, signs=signs)
    o = nsnq.nsnq_decode_attention(p, cbt, q.to(DEV), cache).float().cpu().numpy()
    check_attention(o, ref)
    # the oracle's own cache attended on the GPU
    oc = nsnq.KVCache(p, B, Hkv, capacity(L, R), DEV)
    upload_half(oc, 0, ek)
    upload_half(oc, 1, ev)
    oc.n_quant, oc.n_resid = nq, ek["n_resid"]
    o = nsnq.nsnq_decode_attention(p, cbt, q.to(DEV), oc, num_splits=3).float().cpu().numpy()
    check_attention(o, ref)


# ---------------------------------------------------- double quantisation --

@pytest.mark.parametrize("bits,R,Hq,Hkv,adjust", [
    (2, 64, 2, 2, False),
    (2, 128, 8, 2, True),    # G = 4: matrix-core decode
    (1, 128, 2, 2, False),
    (1, 64, 4, 2, False),    # G = 2
])
def test_double_quant_encode_dequant_decode(oracle_codebooks, bits, R, Hq, Hkv, adjust):
    cb = oracle_codebooks[bits]
    B, L = 2, 5 * R + 9
    k, v = _kv(900 + bits, B, Hkv, L + 1)
    q = synth.queries(900 + bits, 0, B, Hq, D)
    flags = nsnq.NSNQ_DOUBLE_QUANT | (nsnq.NSNQ_SCALE_ADJUST if adjust else 0)
    p, cbt, cache = gpu_encode(k[:, :, :L], v[:, :, :L], bits, R, cb, flags=flags)
    assert cache.dq
    kw = dict(dq=True, scale_adjust=adjust)
    ek, ev = oracle_encode(k[:, :, :L], R, cb, **kw), oracle_encode(v[:, :, :L], R, cb, **kw)
    masks = compare_encoded_dq(cache, ek, ev, R, scale_adjust=adjust)
    nq = ek["n_quant"]
    # dequant of the GPU's own records, on blocks and tokens that agree
    for which, e, x, full in ((0, ek, k, masks[0]), (1, ev, v, masks[1])):
        g = nsnq.nsnq_dequant(p, cbt, cache, which, 0, nq, torch.float32).cpu().numpy()
        ref = oracle.dequant(e["codes"], e["scales"], e["mu"], R, cb, dq=True)
        same = np.all(half_np(cache, which)["codes"] == e["codes"], axis=-1) & np.repeat(full, R, axis=-1)
        check_dequant(g, ref, token_norms(x[:, :, :nq].numpy()), mask=same)
    # decode: end to end, and on the oracle's own records
    ref = oracle.reference_decode(q, ek, ev, nq, ek["n_resid"], R, cb)
    o = nsnq.nsnq_decode_attention(p, cbt, q.to(DEV), cache).float().cpu().numpy()
    check_attention(o, ref)
    oc = nsnq.KVCache(p, B, Hkv, capacity(L, R), DEV)
    upload_half(oc, 0, ek)
    upload_half(oc, 1, ev)
    oc.n_quant, oc.n_resid = nq, ek["n_resid"]
    for ns in (0, 3):
        o = nsnq.nsnq_decode_attention(p, cbt, q.to(DEV), oc, num_splits=ns).float().cpu().numpy()
        check_attention(o, ref)
    # one more token: the full window is flushed in the double-quantised format
    if ek["n_resid"] == R:
        nsnq.nsnq_append_kv(p, cbt, k[:, :, L].contiguous().to(DEV), v[:, :, L].contiguous().to(DEV), cache)
        torch.cuda.synchronize()
        ek2, ev2 = oracle_encode(k, R, cb, **kw), oracle_encode(v, R, cb, **kw)
        compare_encoded_dq(cache, ek2, ev2, R, scale_adjust=adjust)


# --------------------------------------------- 4-bit codebook entries --

@pytest.mark.parametrize("bits,R,flags,cand,Hq,Hkv,dup", [
    (2, 128, 0, False, 2, 2, False),
    (2, 128, nsnq.NSNQ_DOUBLE_QUANT, True, 8, 2, False),   # the whole double-quantised format, G = 4
    (2, 64, nsnq.NSNQ_DOUBLE_QUANT | nsnq.NSNQ_SCALE_ADJUST, True, 2, 1, True),
    (2, 128, 0, True, 4, 4, True),                          # duplicated codewords through the lists
    (1, 64, nsnq.NSNQ_DOUBLE_QUANT, False, 2, 2, False),
    (1, 128, 0, False, 1, 1, True),
])
def test_codebook_4bit_entries(oracle_codebooks, bits, R, flags, cand, Hq, Hkv, dup):
    """Double quantisation of the codebook entries themselves: the library's
    4-bit read-back codebook (equal to the oracle's, checked on the CPU) drives
    encode, dequant and decode on the GPU, against the oracle running on the
    oracle's own read-back codebook; with duplicated codewords (the lowest
    index must win, through the candidate lists too)."""
    cb = oracle_codebooks[bits].copy()
    if dup:  # pairs inside one 32-entry group, so they stay equal in 4 bits
        cb[9] = cb[8]
        cb[18] = cb[17]
    o = oracle.codebook_dq(cb, 32)
    cbq = o["cb_hat"]
    p = nsnq.params(bits, R, flags=flags)
    _, hat = nsnq.nsnq_codebook_dq(p, cb_tensor(cb))
    assert np.array_equal(f16_bits(hat), cbq)
    if dup:
        assert np.array_equal(cbq[9], cbq[8]) and np.array_equal(cbq[18], cbq[17])
    B, L = 2, 4 * R + 5
    k, v = _kv(1100 + bits + R, B, Hkv, L)
    q = synth.queries(1100 + bits + R, 0, B, Hq, D)
    dq = bool(flags & nsnq.NSNQ_DOUBLE_QUANT)
    adjust = bool(flags & nsnq.NSNQ_SCALE_ADJUST)
    pe = nsnq.with_candidates(p, hat) if cand else p
    if cand:
        assert pe.vq_span in (64, 80, 96)
    cache = nsnq.KVCache(p, B, Hkv, capacity(L, R), DEV)
    nsnq.nsnq_encode_kv(pe, hat, k.to(DEV), v.to(DEV), L, cache)
    torch.cuda.synchronize()
    ek, ev = oracle_encode_pair(k, v, R, cbq, scale_adjust=adjust, dq=dq)
    if dq:
        compare_encoded_dq(cache, ek, ev, R, scale_adjust=adjust)
    else:
        compare_encoded(cache, ek, ev, scale_adjust=adjust)
    if dup:  # the higher index of a duplicated pair is never chosen
        for w in (0, 1):
            g = half_np(cache, w)["codes"]
            assert not np.any(g == 9) and not np.any(g == 18)
    nq = ek["n_quant"]
    if not dq:
        for which, e, x in ((0, ek, k), (1, ev, v)):
            g = nsnq.nsnq_dequant(p, hat, cache, which, 0, nq, torch.float32).cpu().numpy()
            ref = oracle.dequant(e["codes"], e["scales"], e["mu"], R, cbq)
            same = np.all(half_np(cache, which)["codes"] == e["codes"], axis=-1)
            check_dequant(g, ref, token_norms(x[:, :, :nq].numpy()), mask=same)
    o_gpu = nsnq.nsnq_decode_attention(p, hat, q.to(DEV), cache).float().cpu().numpy()
    check_attention(o_gpu, oracle.reference_decode(q, gpu_records(cache, 0), gpu_records(cache, 1), cache.n_quant,
                                                   cache.n_resid, R, cbq))
    oc = nsnq.KVCache(p, B, Hkv, capacity(L, R), DEV)
    upload_half(oc, 0, ek)
    upload_half(oc, 1, ev)
    oc.n_quant, oc.n_resid = nq, ek["n_resid"]
    check_attention(nsnq.nsnq_decode_attention(p, hat, q.to(DEV), oc, num_splits=2).float().cpu().numpy(),
                    oracle.reference_decode(q, ek, ev, nq, ek["n_resid"], R, cbq))


# ------------------------------------------------- keys stored before RoPE --

@pytest.mark.parametrize("bits,R,B,Hq,Hkv,L,flags,ragged", [
    (2, 64, 2, 2, 2, 333, 0, False),
    (2, 128, 1, 8, 2, 700, 0, False),                          # G = 4 (pre-RoPE always uses the LUT kernel)
    (1, 128, 2, 4, 4, 300, 0, False),
    (2, 64, 1, 2, 1, 200, 2, False),                           # double-quantised records
    (2, 64, 2, 4, 2, 40, 0, False),                            # residual tokens only
    (2, 64, 3, 2, 1, 0, 0, True),                              # ragged rows
])
def test_prerope_decode(oracle_codebooks, bits, R, B, Hq, Hkv, L, flags, ragged):
    cb = oracle_codebooks[bits]
    pos0 = 7
    lengths = [R + 3, 3 * R + 1, 1] if ragged else [L] * B
    Lmax = max(lengths)
    cos, sin = synth.rope_tables(pos0 + Lmax + 1, 10000.0 if bits == 2 else 500000.0, D)
    k, v = _kv(1000 + bits, B, Hkv, Lmax)
    q = synth.queries(1000 + bits, 0, B, Hq, D)
    p = nsnq.params(bits, R, flags=flags)
    cbt = cb_tensor(cb)
    dq = bool(flags & nsnq.NSNQ_DOUBLE_QUANT)
    if ragged:
        cache = nsnq.KVCache(p, B, Hkv, capacity(Lmax, R), DEV, ragged=True)
        nsnq.nsnq_encode_kv_ragged(p, cbt, k.to(DEV), v.to(DEV), torch.tensor(lengths, dtype=torch.int32,
                                   device=DEV), Lmax, cache)
    else:
        _, _, cache = gpu_encode(k, v, bits, R, cb, flags=flags)
    out = nsnq.nsnq_decode_attention_prerope(p, cbt, q.to(DEV), cache, cos.to(DEV), sin.to(DEV), pos0)
    out = out.float().cpu().numpy()
    for b, Lb in enumerate(lengths):
        ek = oracle.encode(k[b:b + 1, :, :Lb], R, cb, dq=dq)
        ev = oracle.encode(v[b:b + 1, :, :Lb], R, cb, dq=dq)
        ref = oracle.reference_decode(q[b:b + 1], ek, ev, ek["n_quant"], ek["n_resid"], R, cb,
                                      rope_tables=(cos, sin), pos0=pos0)
        check_attention(out[b:b + 1], ref)
    # the rotation matters: the plain decode of the same cache differs
    if not ragged and L > R:
        plain = nsnq.nsnq_decode_attention(p, cbt, q.to(DEV), cache).float().cpu().numpy()
        assert not np.allclose(plain, out, rtol=1e-2)


@pytest.mark.parametrize("bits,R,B,Hq,Hkv,L,use_signs,flags,ns", [
    (2, 128, 2, 4, 2, 5 * 128 + 9, True, 0, 3),                # randomised Hadamard, 3 splits
    (1, 64, 1, 2, 1, 700, True, 2, 0),                         # 1 bit, signs, double-quantised records
    (2, 128, 2, 8, 8, 2500, False, 0, 0),                      # one head per KV head, several splits
    (2, 64, 1, 8, 1, 500, False, 0, 0),                        # G = 8: four 2-head groups per KV head
    (1, 128, 1, 3, 1, 600, True, 0, 0),                        # G = 3: three one-head groups
])
def test_prerope_decode_signs_and_splits(oracle_codebooks, bits, R, B, Hq, Hkv, L, use_signs, flags, ns):
    """Keys stored before RoPE with a sign vector, double quantisation and
    several splits per row, against the oracle's rotated-key attention."""
    cb = oracle_codebooks[bits]
    pos0 = 3
    cos, sin = synth.rope_tables(pos0 + L + 1, 10000.0, D)
    k, v = _kv(1100 + bits, B, Hkv, L)
    q = synth.queries(1100 + bits, 0, B, Hq, D)
    signs = synth.hadamard_signs(110 + bits) if use_signs else None
    dq = bool(flags & nsnq.NSNQ_DOUBLE_QUANT)
    p, cbt, cache = gpu_encode(k, v, bits, R, cb, flags=flags, signs=signs)
    out = nsnq.nsnq_decode_attention_prerope(p, cbt, q.to(DEV), cache, cos.to(DEV), sin.to(DEV), pos0,
                                             num_splits=ns).float().cpu().numpy()
    sg = None if signs is None else signs.numpy()
    ek = oracle.encode(k, R, cb, dq=dq, signs=sg)
    ev = oracle.encode(v, R, cb, dq=dq, signs=sg)
    ref = oracle.reference_decode(q, ek, ev, ek["n_quant"], ek["n_resid"], R, cb, signs=sg,
                                  rope_tables=(cos, sin), pos0=pos0)
    check_attention(out, ref)


# ------------------------------------------------------------ ragged rows --

def _row_state(cache: nsnq.KVCache, which: int, b: int, nq: int, r: int) -> dict:
    h = cache.k if which == 0 else cache.v
    R = h.resid.shape[2]
    return dict(codes=h.codes[b:b + 1, :, :nq].cpu().numpy(), scales=f16_bits(h.scales[b:b + 1, :, :nq]),
                mu=f16_bits(h.mu[b:b + 1, :, :nq // R]), resid=f16_bits(h.resid[b:b + 1]))


def _check_row(cache, b, ek, ev):
    """Row b against the oracle; returns (near-tie flips, codes compared)."""
    nq, r = ek["n_quant"], ek["n_resid"]
    flips = total = 0
    for which, e in ((0, ek), (1, ev)):
        g = _row_state(cache, which, b, nq, r)
        flips += check_codes(g["codes"], e["codes"], e["gap"], e["u"], e["cb"], pooled=True)
        total += g["codes"].size
        check_f16_ulp(g["scales"], e["scales"], "scales")
        check_f16_ulp(g["mu"], e["mu"], "mu")
        assert np.array_equal(g["resid"][..., :r, :], e["resid"][..., :r, :])
    return flips, total


@pytest.mark.parametrize("bits,R,Hq,Hkv", [(2, 64, 2, 2), (1, 128, 8, 2), (2, 128, 4, 1)])
def test_ragged_prefill_append_decode(oracle_codebooks, bits, R, Hq, Hkv):
    """Rows of different lengths (one empty): prefill, decode, then appends that
    flush each row's window at its own step, and decode again; every row must
    match the oracle's encoding of its own prefix.  Attention is checked on the
    oracle's own per-row encodings placed in a ragged cache (the decode alone),
    and end to end on the rows whose codes all equal the oracle's: a single
    near-tie flip is a valid encoding, yet on a token that holds most of the
    softmax weight it moves the output by far more than the attention bar."""
    cb = oracle_codebooks[bits]
    lengths = [0, 1, R, R + 1, 3 * R + 7, 5 * R]
    B, T = len(lengths), R + 3
    Lmax = max(lengths)
    k, v = _kv(700 + bits, B, Hkv, Lmax + T)
    q = synth.queries(700 + bits, 0, B, Hq, D)
    p = nsnq.params(bits, R)
    cbt = cb_tensor(cb)
    cache = nsnq.KVCache(p, B, Hkv, capacity(Lmax + T, R), DEV, ragged=True)
    lens = torch.tensor(lengths, dtype=torch.int32, device=DEV)
    nsnq.nsnq_encode_kv_ragged(p, cbt, k.to(DEV), v.to(DEV), lens, Lmax, cache)
    torch.cuda.synchronize()

    def check_all(cur_len):
        sq, sr = cache.seq_quant.cpu().tolist(), cache.seq_resid.cpu().tolist()
        refs, row_flips = [], []
        flips = total = 0
        # the oracle's encodings in a ragged cache of the same bounds
        oc = nsnq.KVCache(p, B, Hkv, cache.cap_tokens, DEV, ragged=True)
        oc.n_quant, oc.n_resid, oc.max_len = cache.n_quant, cache.n_resid, cache.max_len
        for b, Lb in enumerate(cur_len):
            ek = oracle_encode(k[b:b + 1, :, :Lb], R, cb)
            ev = oracle_encode(v[b:b + 1, :, :Lb], R, cb)
            assert (sq[b], sr[b]) == (ek["n_quant"], ek["n_resid"]), (b, Lb)
            assert sq[b] <= cache.n_quant and sr[b] <= cache.n_resid
            f, t = _check_row(cache, b, ek, ev)
            flips, total = flips + f, total + t
            row_flips.append(f)
            refs.append((ek, ev))
            for h, e in ((oc.k, ek), (oc.v, ev)):
                nq = e["n_quant"]
                h.codes[b, :, :nq].copy_(torch.from_numpy(e["codes"][0]))
                h.scales[b, :, :nq].copy_(torch.from_numpy(e["scales"][0].view(np.float16)))
                h.mu[b, :, :nq // R].copy_(torch.from_numpy(e["mu"][0].view(np.float16)))
                h.resid[b].copy_(torch.from_numpy(e["resid"][0].view(np.float16)))
        oc.seq_quant.copy_(torch.tensor([e["n_quant"] for e, _ in refs], dtype=torch.int32))
        oc.seq_resid.copy_(torch.tensor([e["n_resid"] for e, _ in refs], dtype=torch.int32))
        check_tie_rate(flips, total)
        out = nsnq.nsnq_decode_attention(p, cbt, q.to(DEV), cache).float().cpu().numpy()
        out_oc = nsnq.nsnq_decode_attention(p, cbt, q.to(DEV), oc).float().cpu().numpy()
        for b, (ek, ev) in enumerate(refs):
            if ek["n_quant"] + ek["n_resid"] == 0:
                assert np.all(out[b] == 0) and np.all(out_oc[b] == 0)
                continue
            ref = oracle.reference_decode(q[b:b + 1], ek, ev, ek["n_quant"], ek["n_resid"], R, cb)
            check_attention(out_oc[b:b + 1], ref)
            if row_flips[b] == 0:
                check_attention(out[b:b + 1], ref)
        return refs

    check_all(lengths)
    # dequant over the bound range: rows past their own end read as zeros
    if cache.n_quant > 0:
        g = nsnq.nsnq_dequant(p, cbt, cache, 0, 0, cache.n_quant, torch.float32).cpu().numpy()
        for b, Lb in enumerate(lengths):
            nqb = cache.seq_quant[b].item()
            assert np.all(g[b, :, nqb:] == 0)
            if nqb:
                e = oracle.encode(k[b:b + 1, :, :Lb], R, cb)
                ref = oracle.dequant(e["codes"], e["scales"], e["mu"], R, cb)
                same = np.all(_row_state(cache, 0, b, nqb, 0)["codes"] == e["codes"], axis=-1)
                check_dequant(g[b:b + 1, :, :nqb], ref, token_norms(k[b:b + 1, :, :nqb].numpy()), mask=same)
    for i in range(T):
        idx = torch.tensor([Lb + i for Lb in lengths])
        kn = k[torch.arange(B), :, idx].contiguous().to(DEV)
        vn = v[torch.arange(B), :, idx].contiguous().to(DEV)
        nsnq.nsnq_append_kv(p, cbt, kn, vn, cache)
    torch.cuda.synchronize()
    check_all([Lb + T for Lb in lengths])


def test_uniform_append_flushes_full_window(oracle_codebooks):
    cb = oracle_codebooks[2]
    R, B, H = 64, 2, 2
    L = 3 * R
    k, v = _kv(800, B, H, L + 2)
    p, cbt, cache = gpu_encode(k[:, :, :L], v[:, :, :L], 2, R, cb, cap=8 * R)
    assert (cache.n_quant, cache.n_resid) == (2 * R, R)
    for t in (L, L + 1):
        nsnq.nsnq_append_kv(p, cbt, k[:, :, t].contiguous().to(DEV), v[:, :, t].contiguous().to(DEV), cache)
    torch.cuda.synchronize()
    assert (cache.n_quant, cache.n_resid) == (3 * R, 2)
    ek, ev = oracle_encode_pair(k, v, R, cb)
    compare_encoded(cache, ek, ev)


# ------------------------------------------------------------------ k-means --

@pytest.mark.parametrize("bits", [2, 1])
def test_kmeans_matches_oracle(bits):
    s = nsnq.sub_dim(bits)
    x = synth.randn_samples(900 + bits, 1 << 14, s)
    p = nsnq.params(bits, 128)
    xd = x.to(DEV)
    # one iteration from the same start
    cent1, cb1, dist1 = nsnq.nsnq_build_codebook(p, xd, 1)
    ocent1, ocb1, odist1 = oracle.kmeans(x.numpy(), 256, 1)
    assert dist1.item() == pytest.approx(odist1[0], rel=1e-5)
    dev = np.abs(cent1.cpu().numpy().astype(np.float64) - ocent1).max(axis=1)
    assert (dev > 1e-5).sum() <= 4, f"{(dev > 1e-5).sum()} centroids differ"
    # ten iterations: same distortion curve
    cent, cbk, dist = nsnq.nsnq_build_codebook(p, xd, 10)
    _, ocb, odist = oracle.kmeans(x.numpy(), 256, 10)
    assert np.allclose(dist.cpu().numpy(), odist, rtol=1e-3)
    assert np.all(np.diff(dist.cpu().numpy()) <= 1e-6)
    assert np.array_equal(f16_bits(cbk), f16_bits(cent.half()))
    # explicit init = the oracle's first-iteration centroids
    init = torch.from_numpy(ocent1.astype(np.float32)).to(DEV)
    cent2, _, d2 = nsnq.nsnq_build_codebook(p, xd, 1, init=init)
    _, _, od2 = oracle.kmeans(x.numpy(), 256, 1, init=ocent1.astype(np.float32).astype(np.float64))
    assert d2.item() == pytest.approx(od2[0], rel=1e-5)


@pytest.mark.parametrize("bits,n", [(2, 300), (1, 1000), (2, 64 * 517 + 13)])
def test_kmeans_sample_count_not_a_multiple_of_the_wave(bits, n):
    """The assignment takes 64 samples per wave step; a count that leaves a
    partial last step gives the oracle's iteration (the tail lanes add
    nothing)."""
    s = nsnq.sub_dim(bits)
    x = synth.randn_samples(970 + bits, n, s)
    p = nsnq.params(bits, 128)
    cent1, _, dist1 = nsnq.nsnq_build_codebook(p, x.to(DEV), 1)
    ocent1, _, odist1 = oracle.kmeans(x.numpy(), 256, 1)
    assert dist1.item() == pytest.approx(odist1[0], rel=1e-5)
    dev = np.abs(cent1.cpu().numpy().astype(np.float64) - ocent1).max(axis=1)
    assert (dev > 1e-5).sum() <= 2, f"{(dev > 1e-5).sum()} centroids differ"


@pytest.mark.parametrize("bits", [2, 1])
@pytest.mark.parametrize("case", ["some_wide", "all_wide"])
def test_kmeans_wide_samples(bits, case):
    """Samples the matrix-core assignment does not take (an element of
    magnitude >= 32 or a squared norm >= 1024) go through the per-sample fp32
    search; with such a centroid every sample does.  "some_wide": every 7th
    sample after the first 256 (the initial centroids) scaled by 40;
    "all_wide": every sample scaled by 40."""
    s = nsnq.sub_dim(bits)
    x = synth.randn_samples(960 + bits, 1 << 13, s).numpy().astype(np.float32)
    if case == "all_wide":
        x *= 40.0
    else:
        x[256::7] *= 40.0
    p = nsnq.params(bits, 128)
    cent1, _, dist1 = nsnq.nsnq_build_codebook(p, torch.from_numpy(x).to(DEV), 1)
    ocent1, _, odist1 = oracle.kmeans(x, 256, 1)
    assert dist1.item() == pytest.approx(odist1[0], rel=1e-5)
    scale = 40.0 if case == "all_wide" else 1.0
    dev = np.abs(cent1.cpu().numpy().astype(np.float64) - ocent1).max(axis=1) / scale
    assert (dev > 1e-5).sum() <= 4, f"{(dev > 1e-5).sum()} centroids differ"
    _, _, dist = nsnq.nsnq_build_codebook(p, torch.from_numpy(x).to(DEV), 5)
    _, _, odist = oracle.kmeans(x, 256, 5)
    assert np.allclose(dist.cpu().numpy(), odist, rtol=1e-3)


@pytest.mark.parametrize("bits", [2, 1])
def test_cosine_finetune_matches_oracle(bits):
    """Same start (the oracle's k-means centroids in fp32), same training head
    vectors: the loss curve and the refined centroids agree (assignments are
    fp32 argmins on the GPU, so a near-tie may move one vector's gradient)."""
    s = nsnq.sub_dim(bits)
    ocent, _, _ = oracle.kmeans(synth.randn_samples(bits, 1 << 13, s).numpy(), 256, 6)
    start = ocent.astype(np.float32)
    x = synth.randn_samples(950 + bits, 4096, D)
    p = nsnq.params(bits, 128)
    cent = torch.from_numpy(start.copy()).to(DEV)
    iters, lr = 6, 64.0
    cent, cbk, loss = nsnq.nsnq_finetune_codebook(p, x.to(DEV), iters, lr, cent)
    oc, ocb, oloss = oracle.finetune(x.numpy(), start.astype(np.float64), iters, lr)
    assert np.allclose(loss.cpu().numpy(), oloss, rtol=2e-5, atol=0)
    assert np.all(np.diff(oloss) < 0)
    dev = np.abs(cent.cpu().numpy().astype(np.float64) - oc).max()
    assert dev < 1e-4, dev
    assert np.array_equal(f16_bits(cbk), f16_bits(cent.half()))


# ---------------------------------------------------------- full-size cases --

@pytest.mark.parametrize("cand", [False, True])
def test_llama2_layer_2bit_full(oracle_codebooks, cand):
    """One LLaMA-2-7B-shaped layer: 32 heads, 4096 tokens, 2-bit, R = 128;
    every code of every head, and the decode step, post-RoPE and with the keys
    read as stored before RoPE (exhaustive search, and the candidate-list
    search the bench times)."""
    cb = oracle_codebooks[2]
    w = synth.WORKLOADS["llama2-7b-layer-b1-2bit"]
    B, H, L, R = w["B"], w["Hkv"], w["L"], w["R"]
    k, v = synth.kv_layer(w["config_id"], 0, B, H, L, D)
    p, cbt, cache = gpu_encode(k, v, 2, R, cb, cand=cand)
    assert (cache.n_quant, cache.n_resid) == (3968, 128)
    ek, ev = oracle_encode_pair(k, v, R, cb)
    compare_encoded(cache, ek, ev)
    q = synth.queries(w["config_id"], 0, B, w["Hq"], D)
    o = nsnq.nsnq_decode_attention(p, cbt, q.to(DEV), cache).float().cpu().numpy()
    check_attention(o, _decode_ref(q, ek, ev, cb, R))
    # the same cache read as keys stored before RoPE (positions 0 .. L - 1)
    cos, sin = synth.rope_tables(L + 1, 10000.0, D)
    o = nsnq.nsnq_decode_attention_prerope(p, cbt, q.to(DEV), cache, cos.to(DEV), sin.to(DEV), 0)
    check_attention(o.float().cpu().numpy(), oracle.reference_decode(q, ek, ev, ek["n_quant"], ek["n_resid"], R, cb,
                                                                     rope_tables=(cos, sin)))


def test_llama2_layer_1bit_b16_sampled(oracle_codebooks):
    """Batch 16 at 1 bit: the whole layer is encoded and attended on the GPU in
    the bench's launch configuration; sampled (b, h) streams are checked."""
    cb = oracle_codebooks[1]
    w = synth.WORKLOADS["llama2-7b-layer-b16-1bit"]
    B, H, L, R = w["B"], w["Hkv"], w["L"], w["R"]
    k, v = synth.kv_layer(w["config_id"], 0, B, H, L, D, device=DEV)
    p, cbt, cache = gpu_encode(k, v, 1, R, cb)
    q = synth.queries(w["config_id"], 0, B, w["Hq"], D, device=DEV)
    o = nsnq.nsnq_decode_attention(p, cbt, q, cache).float().cpu().numpy()
    units = [(0, 0), (5, 17), (15, 31)]
    ks = torch.stack([k[b, h] for b, h in units]).cpu()
    vs = torch.stack([v[b, h] for b, h in units]).cpu()
    ek, ev = oracle_encode(ks, R, cb), oracle_encode(vs, R, cb)
    compare_encoded(cache, ek, ev, units=units)
    for i, (b, h) in enumerate(units):
        eki = {key: (val[i:i + 1, None] if isinstance(val, np.ndarray) else val) for key, val in ek.items()}
        evi = {key: (val[i:i + 1, None] if isinstance(val, np.ndarray) else val) for key, val in ev.items()}
        ref = oracle.reference_decode(q[b:b + 1, h:h + 1].cpu(), eki, evi, ek["n_quant"], ek["n_resid"], R, cb)
        check_attention(o[b:b + 1, h:h + 1], ref)


def _sampled_layer_check(cb, w, layer, units, outlier):
    """Encode and attend one whole layer on the GPU (the bench's launch
    configuration), then check sampled (b, kv-head) streams and their query
    heads against the oracle, for the post-RoPE decode and for the decode
    that reads the same cache as keys stored before RoPE (positions 0 ..
    L - 1, standard tables)."""
    B, Hq, Hkv, L, R, bits = w["B"], w["Hq"], w["Hkv"], w["L"], w["R"], w["bits"]
    G = Hq // Hkv
    k, v = synth.kv_layer(w["config_id"], layer, B, Hkv, L, D, outlier_std=outlier, device=DEV)
    p, cbt, cache = gpu_encode(k, v, bits, R, cb)
    q = synth.queries(w["config_id"], layer, B, Hq, D, device=DEV)
    o = nsnq.nsnq_decode_attention(p, cbt, q, cache).float().cpu().numpy()
    cos, sin = synth.rope_tables(L + 8)
    o_pre = nsnq.nsnq_decode_attention_prerope(p, cbt, q, cache, cos.to(DEV), sin.to(DEV), 0).float().cpu().numpy()
    ks = torch.stack([k[b, h] for b, h in units]).cpu()
    vs = torch.stack([v[b, h] for b, h in units]).cpu()
    del k, v
    ek, ev = oracle_encode(ks, R, cb), oracle_encode(vs, R, cb)
    compare_encoded(cache, ek, ev, units=units)
    for i, (b, h) in enumerate(units):
        eki = {key: (val[i:i + 1, None] if isinstance(val, np.ndarray) else val) for key, val in ek.items()}
        evi = {key: (val[i:i + 1, None] if isinstance(val, np.ndarray) else val) for key, val in ev.items()}
        qh = q[b:b + 1, h * G:(h + 1) * G].cpu()
        ref = oracle.reference_decode(qh, eki, evi, ek["n_quant"], ek["n_resid"], R, cb)
        check_attention(o[b:b + 1, h * G:(h + 1) * G], ref)
        ref = oracle.reference_decode(qh, eki, evi, ek["n_quant"], ek["n_resid"], R, cb, rope_tables=(cos, sin))
        check_attention(o_pre[b:b + 1, h * G:(h + 1) * G], ref)


def test_llama31_gqa_32k_layer0_sampled(oracle_codebooks):
    """LLaMA-3.1-8B shape, layer 0 (30x outlier channels): batch 4, 32768
    tokens, 32 query heads over 8 KV heads (G = 4)."""
    w = synth.WORKLOADS["llama3.1-8b-gqa-b4-32k-2bit"]
    _sampled_layer_check(oracle_codebooks[2], w, 0, [(0, 0), (3, 7)],
                         synth.outlier_std_for("llama3.1-8b-gqa-b4-32k-2bit", 0))


def test_llama2_b256_layer_sampled(oracle_codebooks):
    """Batch-256 LLaMA-2-7B layer (the batch-scaling workload): the whole
    layer on the GPU, sampled streams against the oracle."""
    w = synth.WORKLOADS["llama2-7b-b256-2bit"]
    _sampled_layer_check(oracle_codebooks[2], w, 5, [(0, 0), (131, 16), (255, 31)], 10.0)


@pytest.mark.parametrize("B,Hq,Hkv", [(2100, 32, 32), (8200, 32, 8)])
def test_decode_more_units_than_grid_rows(oracle_codebooks, B, Hq, Hkv):
    """More than 65535 (row, head-group) units: the split must then be the
    slow grid dimension (the other one is limited to 65535).  Short contexts
    keep the caches small; sampled rows and heads, first and last included,
    are checked against the oracle's attention over the GPU's own records."""
    R, L = 64, 200
    G = Hq // Hkv
    cb = oracle_codebooks[2]
    k, v = synth.kv_layer(7, 0, B, Hkv, L, D, device=DEV)
    p, cbt, cache = gpu_encode(k, v, 2, R, cb)
    del k, v
    q = synth.queries(7, 0, B, Hq, D, device=DEV)
    o = nsnq.nsnq_decode_attention(p, cbt, q, cache).float().cpu().numpy()
    nq = cache.n_quant

    def rec(hv, b, h):  # one (row, KV head) of a half, in the oracle's layout
        return dict(codes=hv.codes[b:b + 1, h:h + 1, :nq].cpu().numpy(), scales=f16_bits(hv.scales[b:b + 1, h:h + 1, :nq]),
                    mu=f16_bits(hv.mu[b:b + 1, h:h + 1, :nq // R]), resid=f16_bits(hv.resid[b:b + 1, h:h + 1]))
    for b, h in [(0, 0), (B // 2, Hkv // 2), (B - 1, Hkv - 1)]:
        ref = oracle.reference_decode(q[b:b + 1, h * G:(h + 1) * G].cpu(), rec(cache.k, b, h), rec(cache.v, b, h),
                                      nq, cache.n_resid, R, cb)
        check_attention(o[b:b + 1, h * G:(h + 1) * G], ref)


# ------------------------------------------------- fp16-cache comparator --

@pytest.mark.parametrize("B,Hq,Hkv,T,ns", [
    (1, 4, 4, 4096, 0),
    (2, 8, 2, 1000, 0),     # G = 4, ragged last step
    (1, 16, 2, 777, 3),     # G = 8
    (3, 2, 1, 33, 0),       # G = 2, one full step and one token
    (1, 1, 1, 1, 0),        # a single token
    (2, 4, 4, 5000, 7),
])
def test_fp16_comparator_matches_oracle(B, Hq, Hkv, T, ns):
    """The uncompressed fp16-cache decode (the comparator of the benchmark)
    against the oracle's softmax attention over the same fp16 K/V."""
    k, v = _kv(1500 + T, B, Hkv, T)
    q = synth.queries(1500 + T, 0, B, Hq, D)
    o = nsnq.nsnq_fp16_decode_attention(q.to(DEV), k.to(DEV).contiguous(), v.to(DEV).contiguous(), num_splits=ns)
    ref = oracle.attention(q, oracle.f16_to_f64(f16_bits(k)), oracle.f16_to_f64(f16_bits(v)), 1.0 / math.sqrt(D))
    check_attention(o.float().cpu().numpy(), ref)
