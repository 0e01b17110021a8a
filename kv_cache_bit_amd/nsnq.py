"""ctypes binding of libnsnq (include/nsnq.h).

Argument marshalling only: tensors become device pointers, the current torch
stream becomes the hipStream_t, status codes become exceptions.  Every step of
the computation runs in the HIP library.  There is no fallback: if the library
is not built, loading it raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnsnq.so")

NSNQ_OK, NSNQ_EINVAL, NSNQ_EUNSUPPORTED, NSNQ_EHIP, NSNQ_EWORKSPACE, NSNQ_ESCRATCH = range(6)
NSNQ_SCRATCH_BYTES = 16 << 20  # static scratch of nsnq_decode_attention_noalloc, per device
NSNQ_SCALE_ADJUST = 1
NSNQ_DOUBLE_QUANT = 2

i32, i64, f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_float
P = ctypes.c_void_p
size_t = ctypes.c_size_t


class nsnq_params(ctypes.Structure):
    _fields_ = [("head_dim", i32), ("bits", i32), ("n_codewords", i32), ("block_tokens", i32),
                ("flags", i32), ("vq_span", i32), ("hadamard_signs", P), ("vq_candidates", P)]


class nsnq_rope(ctypes.Structure):
    _fields_ = [("cos", P), ("sin", P), ("max_pos", i32), ("pos0", i32)]


class nsnq_kv(ctypes.Structure):
    _fields_ = [("codes", P), ("scales", P), ("mu", P), ("resid", P)]


class nsnq_cache(ctypes.Structure):
    _fields_ = [("k", nsnq_kv), ("v", nsnq_kv), ("batch", i32), ("kv_heads", i32),
                ("cap_tokens", i32), ("n_quant", i32), ("n_resid", i32), ("max_len", i32),
                ("seq_quant", P), ("seq_resid", P)]


_PP, _PC = ctypes.POINTER(nsnq_params), ctypes.POINTER(nsnq_cache)

_SIGNATURES = {
    "nsnq_abi_version": (i32, []),
    "nsnq_status_str": (ctypes.c_char_p, [i32]),
    "nsnq_buffer_bytes": (i32, [_PP, i32, P, P, P, P]),
    "nsnq_build_codebook_workspace_bytes": (size_t, [_PP]),
    "nsnq_build_codebook": (i32, [_PP, P, i64, i32, P, P, P, P, P, size_t, P]),
    "nsnq_finetune_codebook": (i32, [_PP, P, i64, i32, f32, P, P, P, P, size_t, P]),
    "nsnq_vq_candidates": (i32, [_PP, P, P, P]),
    "nsnq_codebook_dq": (i32, [_PP, P, P, P]),
    "nsnq_encode_kv": (i32, [_PP, P, P, P, i64, i64, i64, i32, _PC, P]),
    "nsnq_encode_kv_ragged": (i32, [_PP, P, P, P, i64, i64, i64, P, i32, _PC, P]),
    "nsnq_flush_residual": (i32, [_PP, P, _PC, P]),
    "nsnq_append_kv": (i32, [_PP, P, P, P, _PC, P]),
    "nsnq_dequant": (i32, [_PP, P, _PC, i32, i32, i32, i32, P, P]),
    "nsnq_decode_workspace_bytes": (size_t, [_PP, _PC, i32, i32]),
    "nsnq_decode_attention": (i32, [_PP, P, P, i32, _PC, f32, i32, P, P, size_t, P]),
    "nsnq_decode_attention_prerope": (i32, [_PP, P, P, i32, _PC, f32, ctypes.POINTER(nsnq_rope), i32, P, P,
                                             size_t, P]),
    "nsnq_decode_attention_noalloc": (i32, [_PP, P, P, i32, _PC, f32, i32, P, P]),
    "nsnq_fp16_decode_workspace_bytes": (size_t, [i32, i32, i32, i32]),
    "nsnq_fp16_decode_attention": (i32, [P, i32, P, P, i32, i32, i32, f32, i32, P, P, size_t, P]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """Load libnsnq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m kv_cache_bit_amd.build`")
        _lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(_lib, name)
            fn.restype = res
            fn.argtypes = args
    return _lib


class NsnqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib().nsnq_status_str(status).decode()
        super().__init__(f"{where}: {msg} (status {status})")


def _check(status: int, where: str):
    if status != NSNQ_OK:
        raise NsnqError(status, where)


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        if torch.cuda.is_available() and torch.cuda.is_initialized():
            return torch.cuda.current_stream().cuda_stream
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def params(bits: int, block_tokens: int, head_dim: int = 128, n_codewords: int = 256, flags: int = 0,
           signs: torch.Tensor | None = None) -> nsnq_params:
    """Format parameters.  `signs`: device int8 [head_dim] of +-1 for the
    randomised Hadamard transform (kept referenced by the returned struct)."""
    p = nsnq_params(head_dim, bits, n_codewords, block_tokens, flags, 0, _ptr(signs), None)
    if signs is not None:
        assert signs.dtype == torch.int8 and signs.is_contiguous() and signs.numel() == head_dim
        p._signs_ref = signs
    return p


def with_candidates(p: nsnq_params, codebook: torch.Tensor) -> nsnq_params:
    """A copy of `p` whose encode calls search only the per-orthant candidate
    lists of `codebook` (2 bits; same codes as the exhaustive search).  The
    table is built on the host and copied next to the codebook."""
    table, span = nsnq_vq_candidates(p, codebook)
    dev = table.to(codebook.device)
    q = nsnq_params(p.head_dim, p.bits, p.n_codewords, p.block_tokens, p.flags, span, p.hadamard_signs,
                    dev.data_ptr())
    q._signs_ref = getattr(p, "_signs_ref", None)
    q._cand_ref = dev
    return q


def sub_dim(bits: int) -> int:
    """Sub-vector length: 4 elements at 2 bits, 8 at 1 bit (256 codewords)."""
    return {2: 4, 1: 8}[bits]


# --------------------------------------------------------------- raw calls --

def nsnq_abi_version() -> int:
    return lib().nsnq_abi_version()


def nsnq_vq_candidates(p: nsnq_params, codebook: torch.Tensor) -> tuple[torch.Tensor, int]:
    """Candidate table (uint8 [16][128], host) and the entries to search per
    list for a 2-bit fp16 codebook [256][4] (any device; read on the host)."""
    cb = codebook.detach().to("cpu").contiguous()
    assert cb.dtype == torch.float16 and cb.numel() == 256 * 4
    table = torch.empty(16, 128, dtype=torch.uint8)
    span = ctypes.c_int32()
    _check(lib().nsnq_vq_candidates(ctypes.byref(p), cb.data_ptr(), table.data_ptr(), ctypes.byref(span)),
           "nsnq_vq_candidates")
    return table, span.value


CODEBOOK_DQ_GROUP = 32


def nsnq_codebook_dq(p: nsnq_params, codebook: torch.Tensor) -> tuple[torch.Tensor, torch.Tensor]:
    """4-bit quantisation of the codebook entries (double quantisation):
    returns (record uint8 [bytes], read-back codebook fp16 [256, s]) on the
    codebook's device; the record layout is in include/nsnq.h."""
    cb = codebook.detach().to("cpu").contiguous()
    s = sub_dim(p.bits)
    assert cb.dtype == torch.float16 and cb.numel() == 256 * s
    rec = torch.zeros(128 * s + 4 * (256 * s // CODEBOOK_DQ_GROUP), dtype=torch.uint8)
    hat = torch.empty(256, s, dtype=torch.float16)
    _check(lib().nsnq_codebook_dq(ctypes.byref(p), cb.data_ptr(), rec.data_ptr(), hat.data_ptr()),
           "nsnq_codebook_dq")
    return rec.to(codebook.device), hat.to(codebook.device)


def nsnq_buffer_bytes(p: nsnq_params, cap_tokens: int) -> tuple[int, int, int, int]:
    """Bytes of (codes, scales, mu, resid) per (batch row, KV head) unit."""
    out = [ctypes.c_size_t() for _ in range(4)]
    _check(lib().nsnq_buffer_bytes(ctypes.byref(p), cap_tokens, *[ctypes.byref(o) for o in out]),
           "nsnq_buffer_bytes")
    return tuple(o.value for o in out)


def nsnq_build_codebook_workspace_bytes(p: nsnq_params) -> int:
    return lib().nsnq_build_codebook_workspace_bytes(ctypes.byref(p))


def nsnq_build_codebook(p: nsnq_params, samples: torch.Tensor, iters: int, init=None, centroids=None,
                        codebook=None, distortion=None, ws=None, stream=None):
    """k-means codebook fit on device samples fp32 [n, s].  Returns
    (centroids fp32 [256, s], codebook fp16 [256, s], distortion fp32 [iters])."""
    s = sub_dim(p.bits)
    dev = samples.device
    assert samples.dtype == torch.float32 and samples.is_contiguous() and samples.shape[1] == s
    if centroids is None:
        centroids = torch.empty(256, s, dtype=torch.float32, device=dev)
    if codebook is None:
        codebook = torch.empty(256, s, dtype=torch.float16, device=dev)
    if distortion is None and iters > 0:
        distortion = torch.empty(iters, dtype=torch.float32, device=dev)
    need = nsnq_build_codebook_workspace_bytes(p)
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    _check(lib().nsnq_build_codebook(ctypes.byref(p), _ptr(samples), samples.shape[0], iters, _ptr(init),
                                     _ptr(centroids), _ptr(codebook), _ptr(distortion), _ptr(ws),
                                     ws.numel() * ws.element_size(), _stream(stream)),
           "nsnq_build_codebook")
    return centroids, codebook, distortion


def nsnq_finetune_codebook(p: nsnq_params, samples: torch.Tensor, iters: int, lr: float, centroids: torch.Tensor,
                           codebook=None, loss=None, ws=None, stream=None):
    """Cosine refinement of `centroids` (fp32 [256, s], updated in place) on
    head vectors samples fp32 [n, 128].  Returns (centroids, codebook fp16, loss fp32 [iters])."""
    s = sub_dim(p.bits)
    dev = samples.device
    assert samples.dtype == torch.float32 and samples.is_contiguous() and samples.shape[1] == p.head_dim
    assert centroids.dtype == torch.float32 and centroids.is_contiguous() and tuple(centroids.shape) == (256, s)
    if codebook is None:
        codebook = torch.empty(256, s, dtype=torch.float16, device=dev)
    if loss is None and iters > 0:
        loss = torch.empty(iters, dtype=torch.float32, device=dev)
    if ws is None:
        ws = torch.empty(nsnq_build_codebook_workspace_bytes(p), dtype=torch.uint8, device=dev)
    _check(lib().nsnq_finetune_codebook(ctypes.byref(p), _ptr(samples), samples.shape[0], iters, float(lr),
                                        _ptr(centroids), _ptr(codebook), _ptr(loss), _ptr(ws),
                                        ws.numel() * ws.element_size(), _stream(stream)),
           "nsnq_finetune_codebook")
    return centroids, codebook, loss


def nsnq_encode_kv(p: nsnq_params, codebook, k, v, L: int, cache: "KVCache", stream=None):
    """Prefill encode of k, v fp16 [B, H, >=L, d] (any strides with d contiguous)."""
    assert k.dtype == torch.float16 and v.dtype == torch.float16
    assert k.stride() == v.stride() and k.shape == v.shape and k.stride(3) == 1
    sb, sh, st, _ = k.stride()
    c = cache.c_struct()
    _check(lib().nsnq_encode_kv(ctypes.byref(p), _ptr(codebook), _ptr(k), _ptr(v), sb, sh, st, L,
                                ctypes.byref(c), _stream(stream)), "nsnq_encode_kv")
    cache.n_quant, cache.n_resid, cache.max_len = c.n_quant, c.n_resid, c.max_len


def nsnq_encode_kv_ragged(p: nsnq_params, codebook, k, v, lengths: torch.Tensor, max_len: int,
                          cache: "KVCache", stream=None):
    """Ragged prefill: row b encodes its first lengths[b] tokens (lengths: device
    int32 [B]); the cache must be ragged and empty."""
    assert k.dtype == torch.float16 and v.dtype == torch.float16
    assert k.stride() == v.stride() and k.shape == v.shape and k.stride(3) == 1
    assert lengths.dtype == torch.int32 and lengths.is_contiguous() and lengths.numel() == cache.batch
    sb, sh, st, _ = k.stride()
    c = cache.c_struct()
    _check(lib().nsnq_encode_kv_ragged(ctypes.byref(p), _ptr(codebook), _ptr(k), _ptr(v), sb, sh, st,
                                       _ptr(lengths), max_len, ctypes.byref(c), _stream(stream)),
           "nsnq_encode_kv_ragged")
    cache.n_quant, cache.n_resid, cache.max_len = c.n_quant, c.n_resid, c.max_len


def nsnq_append_kv(p: nsnq_params, codebook, k_new, v_new, cache: "KVCache", stream=None):
    """Append one token per row (k_new, v_new fp16 [B, H, d]), flushing full windows first."""
    assert k_new.dtype == torch.float16 and v_new.dtype == torch.float16
    assert k_new.is_contiguous() and v_new.is_contiguous()
    assert tuple(k_new.shape) == (cache.batch, cache.kv_heads, p.head_dim) and k_new.shape == v_new.shape
    c = cache.c_struct()
    _check(lib().nsnq_append_kv(ctypes.byref(p), _ptr(codebook), _ptr(k_new), _ptr(v_new), ctypes.byref(c),
                                _stream(stream)), "nsnq_append_kv")
    cache.n_quant, cache.n_resid, cache.max_len = c.n_quant, c.n_resid, c.max_len


def nsnq_flush_residual(p: nsnq_params, codebook, cache: "KVCache", stream=None):
    c = cache.c_struct()
    _check(lib().nsnq_flush_residual(ctypes.byref(p), _ptr(codebook), ctypes.byref(c), _stream(stream)),
           "nsnq_flush_residual")
    cache.n_quant, cache.n_resid, cache.max_len = c.n_quant, c.n_resid, c.max_len


def nsnq_dequant(p: nsnq_params, codebook, cache: "KVCache", which: int, tok0: int, ntok: int,
                 out_dtype=torch.float32, out=None, stream=None):
    if out is None:
        out = torch.empty(cache.batch, cache.kv_heads, ntok, p.head_dim, dtype=out_dtype, device=cache.device)
    c = cache.c_struct()
    _check(lib().nsnq_dequant(ctypes.byref(p), _ptr(codebook), ctypes.byref(c), which, tok0, ntok,
                              1 if out.dtype == torch.float16 else 0, _ptr(out), _stream(stream)),
           "nsnq_dequant")
    return out


def nsnq_decode_workspace_bytes(p: nsnq_params, cache: "KVCache", q_heads: int, num_splits: int = 0) -> int:
    c = cache.c_struct()
    return lib().nsnq_decode_workspace_bytes(ctypes.byref(p), ctypes.byref(c), q_heads, num_splits)


def nsnq_decode_attention(p: nsnq_params, codebook, q, cache: "KVCache", softmax_scale: float | None = None,
                          num_splits: int = 0, out=None, ws=None, stream=None):
    """One decode step: q fp16 [B, Hq, d] -> out fp16 [B, Hq, d]."""
    B, Hq, d = q.shape
    assert q.dtype == torch.float16 and q.is_contiguous()
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if ws is None:  # (the library checks a caller's workspace size itself)
        need = nsnq_decode_workspace_bytes(p, cache, Hq, num_splits)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    c = cache.c_struct()
    _check(lib().nsnq_decode_attention(ctypes.byref(p), _ptr(codebook), _ptr(q), Hq, ctypes.byref(c),
                                       float(softmax_scale), num_splits, _ptr(out), _ptr(ws),
                                       ws.numel() * ws.element_size(), _stream(stream)),
           "nsnq_decode_attention")
    return out


def nsnq_decode_attention_noalloc(p: nsnq_params, codebook, q, cache: "KVCache", out,
                                  softmax_scale: float | None = None, num_splits: int = 0, stream=None):
    """One decode step into the caller's `out` (fp16 [B, Hq, d]) with the split
    partials in the library's static device scratch: no allocation here or in
    the library."""
    B, Hq, d = q.shape
    assert q.dtype == torch.float16 and q.is_contiguous()
    assert out.dtype == torch.float16 and out.is_contiguous() and out.shape == q.shape
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    c = cache.c_struct()
    _check(lib().nsnq_decode_attention_noalloc(ctypes.byref(p), _ptr(codebook), _ptr(q), Hq, ctypes.byref(c),
                                               float(softmax_scale), num_splits, _ptr(out), _stream(stream)),
           "nsnq_decode_attention_noalloc")
    return out


def nsnq_decode_attention_prerope(p: nsnq_params, codebook, q, cache: "KVCache", rope_cos: torch.Tensor,
                                  rope_sin: torch.Tensor, pos0: int = 0, softmax_scale: float | None = None,
                                  num_splits: int = 0, out=None, ws=None, stream=None):
    """Decode step over a cache whose keys were stored before RoPE; rope_cos /
    rope_sin: device fp32 [max_pos, 64]; q is the rotated query."""
    B, Hq, d = q.shape
    assert q.dtype == torch.float16 and q.is_contiguous()
    assert rope_cos.dtype == torch.float32 and rope_cos.is_contiguous() and rope_cos.shape == rope_sin.shape
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if ws is None:  # (the library checks a caller's workspace size itself)
        need = nsnq_decode_workspace_bytes(p, cache, Hq, num_splits)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    c = cache.c_struct()
    r = nsnq_rope(_ptr(rope_cos), _ptr(rope_sin), rope_cos.shape[0], pos0)
    _check(lib().nsnq_decode_attention_prerope(ctypes.byref(p), _ptr(codebook), _ptr(q), Hq, ctypes.byref(c),
                                               float(softmax_scale), ctypes.byref(r), num_splits, _ptr(out),
                                               _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "nsnq_decode_attention_prerope")
    return out


def nsnq_fp16_decode_workspace_bytes(batch: int, q_heads: int, n_tokens: int, num_splits: int = 0) -> int:
    return lib().nsnq_fp16_decode_workspace_bytes(batch, q_heads, n_tokens, num_splits)


def nsnq_fp16_decode_attention(q, k, v, softmax_scale: float | None = None, num_splits: int = 0, out=None,
                               ws=None, stream=None):
    """Comparator over an fp16 cache k, v [B, Hkv, T, d] (contiguous)."""
    B, Hq, d = q.shape
    _, Hkv, T, _ = k.shape
    assert k.is_contiguous() and v.is_contiguous() and q.is_contiguous()
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    need = nsnq_fp16_decode_workspace_bytes(B, Hq, T, num_splits)
    if ws is None:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check(lib().nsnq_fp16_decode_attention(_ptr(q), Hq, _ptr(k), _ptr(v), B, Hkv, T, float(softmax_scale),
                                            num_splits, _ptr(out), _ptr(ws), ws.numel() * ws.element_size(),
                                            _stream(stream)), "nsnq_fp16_decode_attention")
    return out


# ------------------------------------------------------------------ cache --

@dataclass
class KVHalf:
    codes: torch.Tensor   # uint8 [B, H, cap, S]
    scales: torch.Tensor  # fp16 [B, H, cap, 2]; double-quantised: uint8 [B, H, cap/R, record bytes]
    mu: torch.Tensor      # fp16 [B, H, cap/R, d]; double-quantised: uint8 [B, H, cap/R, 80]
    resid: torch.Tensor   # fp16 [B, H, R, d]


class KVCache:
    """Caller-owned buffers of one layer's compressed cache plus the two host
    counters (n_quant, n_resid) the library reads and updates.  A ragged cache
    also owns per-row device counters seq_quant / seq_resid (int32 [B]); its
    host counters are then upper bounds."""

    def __init__(self, p: nsnq_params, batch: int, kv_heads: int, cap_tokens: int, device="cuda",
                 ragged: bool = False):
        R, d = p.block_tokens, p.head_dim
        S = d // sub_dim(p.bits)
        assert cap_tokens % R == 0
        self.batch, self.kv_heads, self.cap_tokens = batch, kv_heads, cap_tokens
        self.device = torch.device(device)
        self.n_quant = 0
        self.n_resid = 0
        self.max_len = 0
        self.seq_quant = torch.zeros(batch, dtype=torch.int32, device=device) if ragged else None
        self.seq_resid = torch.zeros(batch, dtype=torch.int32, device=device) if ragged else None

        self.dq = bool(p.flags & NSNQ_DOUBLE_QUANT)
        _, sc_bytes, mu_bytes, _ = nsnq_buffer_bytes(p, cap_tokens)
        nb = cap_tokens // R

        def half():
            if self.dq:
                scales = torch.zeros(batch, kv_heads, nb, sc_bytes // max(nb, 1), dtype=torch.uint8, device=device)
                mu = torch.zeros(batch, kv_heads, nb, mu_bytes // max(nb, 1), dtype=torch.uint8, device=device)
            else:
                scales = torch.zeros(batch, kv_heads, cap_tokens, 2, dtype=torch.float16, device=device)
                mu = torch.zeros(batch, kv_heads, nb, d, dtype=torch.float16, device=device)
            return KVHalf(
                codes=torch.zeros(batch, kv_heads, cap_tokens, S, dtype=torch.uint8, device=device),
                scales=scales, mu=mu,
                resid=torch.zeros(batch, kv_heads, R, d, dtype=torch.float16, device=device))

        self.k = half()
        self.v = half()

    def c_struct(self) -> nsnq_cache:
        def kv(h: KVHalf):
            return nsnq_kv(h.codes.data_ptr(), h.scales.data_ptr(), h.mu.data_ptr(), h.resid.data_ptr())
        return nsnq_cache(kv(self.k), kv(self.v), self.batch, self.kv_heads, self.cap_tokens,
                          self.n_quant, self.n_resid, self.max_len, _ptr(self.seq_quant), _ptr(self.seq_resid))

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for h in (self.k, self.v)
                   for t in (h.codes, h.scales, h.mu, h.resid))
