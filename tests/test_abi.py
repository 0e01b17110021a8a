"""The C-ABI library loads on the CPU host, exports every function that
include/nsnq.h declares, and rejects bad arguments on the host before any
HIP call (no GPU is touched by these tests)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nsnq.h")


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(nsnq_[a-z0-9_]+)\s*\(", txt)))


@pytest.fixture(scope="module")
def nsnq():
    from kv_cache_bit_amd import nsnq as m
    m.lib()
    return m


def test_exports_every_declared_symbol(nsnq):
    names = _declared()
    assert len(names) == 19
    for n in names:
        assert hasattr(nsnq.lib(), n), n
    assert nsnq.nsnq_abi_version() == 7
    assert nsnq.lib().nsnq_status_str(1) == b"invalid argument"


def _cache_struct(nsnq, B=1, H=2, cap=256, nq=0, nr=0, ptr=0x1000, sq=None, sr=None, ml=0):
    kv = nsnq.nsnq_kv(ptr, ptr, ptr, ptr)
    return nsnq.nsnq_cache(kv, kv, B, H, cap, nq, nr, ml, sq, sr)


def test_host_validation_rejects_before_launch(nsnq):
    L = nsnq.lib()
    good = nsnq.params(2, 128)
    c = _cache_struct(nsnq)
    P = 0x1000  # aligned fake device pointer: never dereferenced on these paths
    EINVAL, EUNS, EWS = nsnq.NSNQ_EINVAL, nsnq.NSNQ_EUNSUPPORTED, nsnq.NSNQ_EWORKSPACE
    by = ctypes.byref
    # bad format parameters
    assert L.nsnq_encode_kv(by(nsnq.params(3, 128)), P, P, P, 0, 0, 128, 256, by(c), None) == EINVAL
    assert L.nsnq_encode_kv(by(nsnq.params(2, 128, head_dim=64)), P, P, P, 0, 0, 64, 256, by(c), None) == EUNS
    assert L.nsnq_encode_kv(by(nsnq.params(2, 96)), P, P, P, 0, 0, 128, 256, by(c), None) == EUNS
    assert L.nsnq_encode_kv(by(nsnq.params(2, 128, n_codewords=16)), P, P, P, 0, 0, 128, 256, by(c), None) == EINVAL
    # unknown flags; candidate-table fields that do not go together
    bad_flags = nsnq.params(2, 128, flags=4)
    assert L.nsnq_encode_kv(by(bad_flags), P, P, P, 0, 0, 128, 256, by(c), None) == EINVAL
    for bits, span, table in ((2, 16, None), (2, 0, P), (2, 144, P), (2, 72, P), (2, 96, P + 8), (1, 96, P)):
        bad = nsnq.params(bits, 128)
        bad.vq_span, bad.vq_candidates = span, table
        assert L.nsnq_encode_kv(by(bad), P, P, P, 0, 0, 128, 256, by(c), None) == EINVAL, (bits, span, table)
    ok = nsnq.params(2, 128)
    ok.vq_span, ok.vq_candidates = 80, P
    assert L.nsnq_encode_kv(by(ok), P, P, P, 0, 0, 128, 0, by(c), None) == nsnq.NSNQ_OK
    adj = nsnq.params(2, 128, flags=nsnq.NSNQ_SCALE_ADJUST)
    assert L.nsnq_encode_kv(by(adj), P, P, P, 0, 0, 128, 0, by(c), None) == nsnq.NSNQ_OK
    # misaligned or null pointers, bad strides, capacity, residual state
    assert L.nsnq_encode_kv(by(good), P + 2, P, P, 0, 0, 128, 256, by(c), None) == EINVAL
    assert L.nsnq_encode_kv(by(good), P, None, P, 0, 0, 128, 256, by(c), None) == EINVAL
    assert L.nsnq_encode_kv(by(good), P, P, P, 0, 0, 100, 256, by(c), None) == EINVAL
    assert L.nsnq_encode_kv(by(good), P, P, P, 0, 0, 128, 1000, by(c), None) == EINVAL  # 896 > cap 256
    c_res = _cache_struct(nsnq, nr=5)
    assert L.nsnq_encode_kv(by(good), P, P, P, 0, 0, 128, 256, by(c_res), None) == EINVAL
    c_badcap = _cache_struct(nsnq, cap=200)
    assert L.nsnq_encode_kv(by(good), P, P, P, 0, 0, 128, 256, by(c_badcap), None) == EINVAL
    c_mis = nsnq.nsnq_cache(nsnq.nsnq_kv(P + 4, P, P, P), nsnq.nsnq_kv(P, P, P, P), 1, 2, 256, 0, 0, 0, None, None)
    assert L.nsnq_encode_kv(by(good), P, P, P, 0, 0, 128, 256, by(c_mis), None) == EINVAL
    assert L.nsnq_encode_kv(by(good), P, P, P, 0, 0, 128, 0, by(c), None) == nsnq.NSNQ_OK  # L = 0: no work
    # flush needs a full window
    assert L.nsnq_flush_residual(by(good), P, by(_cache_struct(nsnq, nr=100)), None) == EINVAL
    assert L.nsnq_flush_residual(by(good), P, by(_cache_struct(nsnq, nq=256, nr=128)), None) == EINVAL
    # dequant range
    cq = _cache_struct(nsnq, nq=128)
    assert L.nsnq_dequant(by(good), P, by(cq), 0, 0, 129, 0, P, None) == EINVAL
    assert L.nsnq_dequant(by(good), P, by(cq), 2, 0, 1, 0, P, None) == EINVAL
    assert L.nsnq_dequant(by(good), P, by(cq), 0, 0, 0, 0, P, None) == nsnq.NSNQ_OK
    # decode: empty cache, head grouping, workspace
    assert L.nsnq_decode_attention(by(good), P, P, 4, by(c), 0.1, 0, P, P, 1 << 20, None) == EINVAL
    cd = _cache_struct(nsnq, nq=128, nr=3)
    assert L.nsnq_decode_attention(by(good), P, P, 3, by(cd), 0.1, 0, P, P, 1 << 20, None) == EINVAL
    need = L.nsnq_decode_workspace_bytes(by(good), by(cd), 4, 0)
    assert need > 0
    assert L.nsnq_decode_attention(by(good), P, P, 4, by(cd), 0.1, 0, P, P, need - 4, None) == EWS
    assert L.nsnq_decode_attention(by(good), P, P, 4, by(cd), 0.1, 0, P, None, need, None) == EWS
    # codebook fit
    ws = L.nsnq_build_codebook_workspace_bytes(by(good))
    assert ws > 0
    assert L.nsnq_build_codebook(by(good), P, 100, 5, None, P, P, None, P, ws, None) == EINVAL  # n < 256
    assert L.nsnq_build_codebook(by(good), P, 1000, 5, None, P, P, None, P, ws - 8, None) == EWS
    # ragged caches: both counter arrays or neither, aligned; the uniform
    # prefill refuses them and the ragged prefill needs one that is empty
    assert L.nsnq_encode_kv(by(good), P, P, P, 0, 0, 128, 256, by(_cache_struct(nsnq, sq=P)), None) == EINVAL
    assert L.nsnq_encode_kv(by(good), P, P, P, 0, 0, 128, 256,
                            by(_cache_struct(nsnq, sq=P + 2, sr=P)), None) == EINVAL
    cr = _cache_struct(nsnq, sq=P, sr=P + 64)
    assert L.nsnq_encode_kv(by(good), P, P, P, 0, 0, 128, 256, by(cr), None) == EINVAL
    assert L.nsnq_encode_kv_ragged(by(good), P, P, P, 0, 0, 128, P, 1000, by(cr), None) == EINVAL  # > cap
    assert L.nsnq_encode_kv_ragged(by(good), P, P, P, 0, 0, 128, P, 10, by(c), None) == EINVAL   # uniform
    assert L.nsnq_encode_kv_ragged(by(good), P, P, P, 0, 0, 128, P, 10,
                                   by(_cache_struct(nsnq, nq=128, sq=P, sr=P + 64)), None) == EINVAL  # not empty
    assert L.nsnq_encode_kv_ragged(by(good), P, P, P, 0, 0, 128, P + 1, 10, by(cr), None) == EINVAL  # misaligned
    # append: a full window needs room for its flush
    assert L.nsnq_append_kv(by(good), P, P, P, by(_cache_struct(nsnq, nq=256, nr=128)), None) == EINVAL
    assert L.nsnq_append_kv(by(good), P, P + 8, P, by(c), None) == EINVAL
    assert L.nsnq_append_kv(by(good), P, P, P, by(_cache_struct(nsnq, nq=256, nr=127, ml=383, sq=P, sr=P + 64)),
                            None) == EINVAL  # a 384-token row may need 384 quantised slots > cap 256
    cr_nofull = _cache_struct(nsnq, nq=128, nr=5, ml=133, sq=P, sr=P + 64)
    assert L.nsnq_flush_residual(by(good), P, by(cr_nofull), None) == nsnq.NSNQ_OK  # no row can be full
    # comparator
    assert L.nsnq_fp16_decode_attention(P, 3, P, P, 1, 1, 10, 0.1, 0, P, P, 1 << 20, None) == EUNS
    assert L.nsnq_fp16_decode_attention(P, 4, P, P, 1, 1, 0, 0.1, 0, P, P, 1 << 20, None) == EINVAL


def test_counters_untouched_on_error(nsnq):
    c = _cache_struct(nsnq, nq=128, nr=7)
    good = nsnq.params(2, 128)
    assert nsnq.lib().nsnq_flush_residual(ctypes.byref(good), 0x1000, ctypes.byref(c), None) == nsnq.NSNQ_EINVAL
    assert (c.n_quant, c.n_resid) == (128, 7)


def test_buffer_bytes(nsnq):
    """Plain format: codes S B, scales 4 B per token, mu 256 B per block;
    double-quantised: one padded scales record and one 80-byte mean record
    per block."""
    for bits, S in ((2, 32), (1, 16)):
        for R in (64, 128):
            c, sc, mu, rs = nsnq.nsnq_buffer_bytes(nsnq.params(bits, R), 4 * R)
            assert (c, sc, mu, rs) == (4 * R * S, 4 * R * 4, 4 * 256, R * 256)
            p = nsnq.params(bits, R, flags=nsnq.NSNQ_DOUBLE_QUANT)
            c, sc, mu, rs = nsnq.nsnq_buffer_bytes(p, 4 * R)
            rec = {64: 176, 128: 336}[R]
            assert (c, sc, mu, rs) == (4 * R * S, 4 * rec, 4 * 80, R * 256)
    with pytest.raises(nsnq.NsnqError):
        nsnq.nsnq_buffer_bytes(nsnq.params(2, 128), 100)
    with pytest.raises(nsnq.NsnqError):
        nsnq.nsnq_buffer_bytes(nsnq.params(2, 128, flags=8), 128)


def test_decode_split_plan(nsnq):
    """Split planning (host, read back through the workspace size, which holds
    one (d + 2)-float partial per row, query head and split): a requested split
    count is honoured between one block per split and 16 blocks per split, the
    residual window adds one split, and the default plan for one head keeps at
    least 512 tokens per split."""
    L = nsnq.lib()
    by = ctypes.byref
    p = nsnq.params(2, 128)

    def nsplit(nq, nr, ns, B=1, H=2):
        c = _cache_struct(nsnq, B=B, H=H, cap=nq + 128, nq=nq, nr=nr)
        per = 4 * (128 + 2) * B * H
        ws = L.nsnq_decode_workspace_bytes(by(p), by(c), H, ns)
        assert ws % per == 0
        return ws // per

    assert nsplit(31 * 128, 128, 7) == 8     # 7 splits of 4-5 blocks + the residual window
    assert nsplit(31 * 128, 128, 40) == 32   # one block each, no more
    assert nsplit(31 * 128, 0, 1) == 2       # 16 blocks at most: two splits
    assert nsplit(5 * 128, 3, 3) == 4
    assert nsplit(0, 5, 0) == 1              # residual tokens only
    assert nsplit(31 * 128, 128, 0, B=1, H=32) == 8   # default: 512 tokens or more per split
    assert nsplit(31 * 128, 128, 0, B=256, H=32) == 3  # default at batch 256: the 16-block cap


def test_noalloc_decode_rejects_oversize_on_the_host(nsnq):
    """The allocation-free decode refuses, before any HIP call, a call whose
    split partials would not fit the static scratch; it validates its
    arguments like the workspace call does."""
    L = nsnq.lib()
    by = ctypes.byref
    P = 0x1000
    p = nsnq.params(2, 128)
    big = _cache_struct(nsnq, B=4096, H=32, cap=4096, nq=3968, nr=128)
    need = L.nsnq_decode_workspace_bytes(by(p), by(big), 32, 0)
    assert need > nsnq.NSNQ_SCRATCH_BYTES
    assert L.nsnq_decode_attention_noalloc(by(p), P, P, 32, by(big), 0.088, 0, P, None) == nsnq.NSNQ_ESCRATCH
    assert b"static scratch" in L.nsnq_status_str(nsnq.NSNQ_ESCRATCH)
    small = _cache_struct(nsnq, B=1, H=2, cap=256, nq=128, nr=5)
    assert L.nsnq_decode_workspace_bytes(by(p), by(small), 2, 0) <= nsnq.NSNQ_SCRATCH_BYTES
    assert L.nsnq_decode_attention_noalloc(by(nsnq.params(3, 128)), P, P, 2, by(small), 0.088, 0, P, None) == \
        nsnq.NSNQ_EINVAL
    assert L.nsnq_decode_attention_noalloc(by(p), P, P, 3, by(small), 0.088, 0, P, None) == nsnq.NSNQ_EINVAL
    assert L.nsnq_decode_attention_noalloc(by(p), P, P, 2, by(small), 0.088, -1, P, None) == nsnq.NSNQ_EINVAL


@pytest.mark.parametrize("bits", [2, 1])
def test_codebook_dq_matches_oracle(nsnq, oracle_codebooks, bits):
    """The library's host quantisation of the codebook entries (4 bits) gives
    the oracle's record and read-back codebook byte for byte, on the k-means
    codebook and on one with duplicated codewords, a constant group and
    values near fp16 ties."""
    import numpy as np
    import torch

    import oracle
    cbs = [oracle_codebooks[bits]]
    c2 = oracle_codebooks[bits].copy()
    s = c2.shape[1]
    c2[5] = c2[4]
    c2[64:64 + 32 // s] = c2[64]           # a constant group
    c2[100] = np.float16(1.0 + 2.0 ** -10).view(np.uint16)
    cbs.append(c2)
    for cb in cbs:
        p = nsnq.params(bits, 128)
        rec, hat = nsnq.nsnq_codebook_dq(p, torch.from_numpy(cb.view(np.float16)))
        o = oracle.codebook_dq(cb, 32)
        assert np.array_equal(rec.numpy(), o["record"])
        assert np.array_equal(hat.numpy().view(np.uint16), o["cb_hat"])
    L = nsnq.lib()
    bad = cbs[0].copy()
    bad[7, 0] = 0x7c00  # inf
    out = np.zeros(4096, np.uint8)
    outh = np.zeros_like(bad)
    assert L.nsnq_codebook_dq(ctypes.byref(nsnq.params(bits, 128)), bad.ctypes.data, out.ctypes.data,
                              outh.ctypes.data) == nsnq.NSNQ_EINVAL
