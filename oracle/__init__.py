"""ctypes front end of the CPU oracle (``nsnq_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
CPU-baseline leg of the benchmark.  The product library never imports it.

Every function takes and returns numpy arrays; fp16 values travel as their
uint16 bit patterns so that the oracle's own fp16 conversion is the one used.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nsnq_oracle.c")
_LIB = os.path.join(_HERE, "libnsnq_oracle.so")


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        _lib = ctypes.CDLL(build())
        P = ctypes.c_void_p
        i32, i64, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_double
        sig = {
            "orc_h2d": (f64, [ctypes.c_uint16]),
            "orc_d2h": (ctypes.c_uint16, [f64]),
            "orc_d2h_array": (None, [P, P, i64]),
            "orc_h2d_array": (None, [P, P, i64]),
            "orc_hadamard_matrix": (None, [i32, P]),
            "orc_hadamard": (None, [P, P, i32]),
            "orc_nsn_block": (None, [P, i32, i32, P, P, P, P, P, P]),
            "orc_vq": (i32, [P, i32, P, i32, P, P]),
            "orc_resid_count": (i32, [i32, i32]),
            "orc_encode": (i32, [P, i64, i32, i32, i32, i32, P, i32, P, i32, P, P, P, P, P, P]),
            "orc_dequant": (None, [P, P, P, i64, i32, i32, i32, i32, i32, i32, P, P, P]),
            "orc_attention": (None, [P, i32, i32, i32, i32, P, P, i32, f64, P]),
            "orc_kmeans": (None, [P, i64, i32, i32, i32, P, P, P, P]),
            "orc_num_threads": (i32, []),
            "orc_set_num_threads": (None, [i32]),
            "orc_rtn4": (None, [P, i32, P, P, P, P, P]),
            "orc_cos_loss_grad": (f64, [P, i64, i32, i32, P, i32, P]),
            "orc_rope": (None, [P, i64, i32, i32, P, P, i32]),
            "orc_finetune": (None, [P, i64, i32, i32, i32, i32, f64, P, P, P]),
            "orc_dq_scales_bytes": (i32, [i32]),
            "orc_encode_dq": (i32, [P, i64, i32, i32, i32, i32, P, i32, P, i32, P, P, P, P, P, P, P, P, P, P, P]),
            "orc_dequant_dq": (None, [P, P, P, i64, i32, i32, i32, i32, i32, i32, P, P, P]),
            "orc_codebook_dq": (None, [P, i32, i32, P, P, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(_lib, name)
            fn.restype = res
            fn.argtypes = args
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def as_f16_bits(a) -> np.ndarray:
    """fp16 array (numpy or torch) -> contiguous uint16 bit patterns."""
    if hasattr(a, "detach"):
        a = a.detach().cpu().contiguous().numpy()
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        return a.view(np.uint16)
    assert a.dtype == np.uint16, a.dtype
    return a


def f16_to_f64(bits: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, np.float64)
    lib().orc_h2d_array(_p(bits), _p(out), bits.size)
    return out


def f64_to_f16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, np.uint16)
    lib().orc_d2h_array(_p(x), _p(out), x.size)
    return out


def hadamard_matrix(d: int) -> np.ndarray:
    H = np.empty((d, d), np.float64)
    lib().orc_hadamard_matrix(d, _p(H))
    return H


def hadamard(w: np.ndarray) -> np.ndarray:
    w = np.ascontiguousarray(w, dtype=np.float64)
    u = np.empty_like(w)
    lib().orc_hadamard(_p(w), _p(u), w.shape[-1])
    return u


def nsn_block(x) -> dict:
    """Intermediates of Normalize-Shift-Normalize on one block x fp16 [R, d]."""
    xb = as_f16_bits(x)
    R, d = xb.shape
    out = {k: np.empty(shape, np.float64) for k, shape in
           dict(n1=(R,), y=(R, d), mu=(d,), z=(R, d), n2=(R,), w=(R, d)).items()}
    lib().orc_nsn_block(_p(xb), R, d, _p(out["n1"]), _p(out["y"]), _p(out["mu"]),
                        _p(out["z"]), _p(out["n2"]), _p(out["w"]))
    return out


def vq(v: np.ndarray, codebook) -> tuple[int, float, float]:
    """(code, D1, gap_rel) of one sub-vector against an fp16 codebook [ncw, s]."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    cb = as_f16_bits(codebook)
    dmin = ctypes.c_double()
    gap = ctypes.c_double()
    code = lib().orc_vq(_p(v), v.shape[0], _p(cb), cb.shape[0], ctypes.byref(dmin), ctypes.byref(gap))
    return code, dmin.value, gap.value


def resid_count(L: int, R: int) -> int:
    return lib().orc_resid_count(L, R)


def _signs(signs):
    if signs is None:
        return None
    if hasattr(signs, "detach"):
        signs = signs.detach().cpu().numpy()
    return np.ascontiguousarray(signs, dtype=np.float64)


DQ_MU_BYTES = 80


def dq_scales_bytes(R: int) -> int:
    """Bytes of one block's scales record in the double-quantised format."""
    return lib().orc_dq_scales_bytes(R)


def rtn4(v) -> dict:
    """4-bit round-to-nearest of one group: Z, S (fp16 bits), q, v_hat, margin."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    Z, S = ctypes.c_uint16(), ctypes.c_uint16()
    q = np.empty(v.size, np.uint8)
    vh = np.empty(v.size, np.float64)
    m = np.empty(v.size, np.float64)
    lib().orc_rtn4(_p(v), v.size, ctypes.byref(Z), ctypes.byref(S), _p(q), _p(vh), _p(m))
    return dict(Z=Z.value, S=S.value, q=q, vhat=vh, margin=m)


def codebook_dq(codebook, group: int = 32) -> dict:
    """4-bit double quantisation of the codebook entries (groups of `group`
    consecutive entries in storage order).  Returns record (uint8: n/2 bytes
    of codes, then (S, Z) fp16 per group), cb_hat (fp16 bits, the read-back
    codebook, same shape as the input) and margin (per entry)."""
    cb = as_f16_bits(codebook)
    n = cb.size
    assert n % group == 0 and group % 2 == 0
    rec = np.zeros(n // 2 + 4 * (n // group), np.uint8)
    hat = np.zeros(cb.shape, np.uint16)
    margin = np.zeros(cb.shape, np.float64)
    lib().orc_codebook_dq(_p(np.ascontiguousarray(cb)), n, group, _p(rec), _p(hat), _p(margin))
    return dict(record=rec, cb_hat=hat, margin=margin)


def encode(x, R: int, codebook, with_u: bool = False, signs=None, scale_adjust: bool = False,
           dq: bool = False, force_records=None) -> dict:
    """Encode streams x fp16 [..., L, d] (leading dims are independent units).
    signs: +-1 [d] for the randomised Hadamard transform (None: plain);
    scale_adjust: Strategy-3 scale folded into n2; dq: double-quantised format
    (scales [..., nq/R, dq_scales_bytes(R)] and mu [..., nq/R, 80] uint8
    records, plus n1hat / m1 per token and mmu per block channel).
    force_records (dq only): (scales, mu) records of the same layout whose
    4-bit decisions, (S, Z) and codes, every block takes instead of rounding
    its own; n2, codes, gap and u then follow from those read-back values.

    Returns codes [..., nq, S] uint8, scales [..., nq, 2] (fp16 bits),
    mu [..., nq/R, d] (fp16 bits), resid [..., R, d] (fp16 bits, rows >= r
    zero), gap [..., nq, S] float64, and optionally u [..., nq, d]."""
    xb = as_f16_bits(x)
    *lead, L, d = xb.shape
    n_units = int(np.prod(lead)) if lead else 1
    cb = as_f16_bits(codebook)
    ncw, s = cb.shape
    S = d // s
    r = resid_count(L, R)
    nq = L - r
    codes = np.zeros((n_units, nq, S), np.uint8)
    scales = np.zeros((n_units, nq, 2), np.uint16)
    mu = np.zeros((n_units, nq // R, d), np.uint16)
    resid = np.zeros((n_units, R, d), np.uint16)
    gap = np.zeros((n_units, nq, S), np.float64)
    u = np.zeros((n_units, nq, d), np.float64) if with_u else None
    sg = _signs(signs)
    if dq:
        SR = dq_scales_bytes(R)
        scales = np.zeros((n_units, nq // R, SR), np.uint8)
        mu = np.zeros((n_units, nq // R, DQ_MU_BYTES), np.uint8)
        n1hat = np.zeros((n_units, nq), np.float64)
        m1 = np.zeros((n_units, nq), np.float64)
        mmu = np.zeros((n_units, nq // R, d), np.float64)
        fs = fm = None
        if force_records is not None:
            fs = np.ascontiguousarray(force_records[0], dtype=np.uint8).reshape(n_units, nq // R, SR)
            fm = np.ascontiguousarray(force_records[1], dtype=np.uint8).reshape(n_units, nq // R, DQ_MU_BYTES)
        lib().orc_encode_dq(_p(xb), n_units, L, d, R, s, _p(cb), ncw, _p(sg) if sg is not None else None,
                            int(scale_adjust), _p(codes), _p(scales), _p(mu), _p(resid), _p(gap),
                            _p(u) if with_u else None, _p(n1hat), _p(m1), _p(mmu),
                            _p(fs) if fs is not None else None, _p(fm) if fm is not None else None)
        out = dict(codes=codes.reshape(*lead, nq, S), scales=scales.reshape(*lead, nq // R, SR),
                   mu=mu.reshape(*lead, nq // R, DQ_MU_BYTES), resid=resid.reshape(*lead, R, d),
                   gap=gap.reshape(*lead, nq, S), n1hat=n1hat.reshape(*lead, nq), m1=m1.reshape(*lead, nq),
                   mmu=mmu.reshape(*lead, nq // R, d), n_quant=nq, n_resid=r, dq=True)
        if with_u:
            out["u"] = u.reshape(*lead, nq, d)
        return out
    lib().orc_encode(_p(xb), n_units, L, d, R, s, _p(cb), ncw, _p(sg) if sg is not None else None,
                     int(scale_adjust), _p(codes), _p(scales), _p(mu), _p(resid), _p(gap),
                     _p(u) if with_u else None)
    out = dict(codes=codes.reshape(*lead, nq, S), scales=scales.reshape(*lead, nq, 2),
               mu=mu.reshape(*lead, nq // R, d), resid=resid.reshape(*lead, R, d),
               gap=gap.reshape(*lead, nq, S), n_quant=nq, n_resid=r)
    if with_u:
        out["u"] = u.reshape(*lead, nq, d)
    return out


def dequant(codes, scales, mu, R: int, codebook, tok0: int = 0, ntok: int | None = None,
            signs=None, dq: bool = False) -> np.ndarray:
    """Reconstruct tokens [tok0, tok0+ntok) of streams with codes [..., cap, S],
    scales [..., cap, 2] (fp16 bits), mu [..., cap/R, d] (fp16 bits); with
    dq, scales and mu are the uint8 records of the double-quantised format."""
    if dq:
        codes = np.ascontiguousarray(codes, dtype=np.uint8)
        scales = np.ascontiguousarray(scales, dtype=np.uint8)
        mu = np.ascontiguousarray(mu, dtype=np.uint8)
        cb = as_f16_bits(codebook)
        *lead, cap, S = codes.shape
        s = cb.shape[1]
        d = S * s
        n_units = int(np.prod(lead)) if lead else 1
        if ntok is None:
            ntok = cap - tok0
        out = np.empty((n_units, ntok, d), np.float64)
        sg = _signs(signs)
        lib().orc_dequant_dq(_p(codes), _p(scales), _p(mu), n_units, cap, tok0, ntok, d, R, s, _p(cb),
                             _p(sg) if sg is not None else None, _p(out))
        return out.reshape(*lead, ntok, d)
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = as_f16_bits(scales)
    mu = as_f16_bits(mu)
    cb = as_f16_bits(codebook)
    *lead, cap, S = codes.shape
    d = mu.shape[-1]
    s = cb.shape[1]
    assert S * s == d
    n_units = int(np.prod(lead)) if lead else 1
    if ntok is None:
        ntok = cap - tok0
    out = np.empty((n_units, ntok, d), np.float64)
    sg = _signs(signs)
    lib().orc_dequant(_p(codes), _p(scales), _p(mu), n_units, cap, tok0, ntok, d, R, s, _p(cb),
                      _p(sg) if sg is not None else None, _p(out))
    return out.reshape(*lead, ntok, d)


def attention(q, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """Softmax attention of q fp16 [B, Hq, d] over k, v float64 [B, Hkv, T, d]."""
    qb = as_f16_bits(q)
    B, Hq, d = qb.shape
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    _, Hkv, T, _ = k.shape
    out = np.empty((B, Hq, d), np.float64)
    lib().orc_attention(_p(qb), B, Hq, Hkv, d, _p(k), _p(v), T, float(scale), _p(out))
    return out


def kmeans(samples, ncw: int, iters: int, init: np.ndarray | None = None):
    """Lloyd k-means; returns (centroids float64 [ncw, s], codebook fp16 bits
    [ncw, s], distortion float64 [iters])."""
    if hasattr(samples, "detach"):
        samples = samples.detach().cpu().numpy()
    x = np.ascontiguousarray(samples, dtype=np.float32)
    n, s = x.shape
    cent = np.empty((ncw, s), np.float64)
    cb = np.empty((ncw, s), np.uint16)
    dist = np.empty((max(iters, 1),), np.float64)
    ini = None if init is None else np.ascontiguousarray(init, dtype=np.float64)
    lib().orc_kmeans(_p(x), n, s, ncw, iters, _p(ini) if ini is not None else None,
                     _p(cent), _p(cb), _p(dist))
    return cent, cb, dist[:iters]


def cos_loss_grad(x, centroids) -> tuple[float, np.ndarray]:
    """Cosine objective of the codebook refinement and its gradient, for head
    vectors x fp32 [n, d] and centroids float64 [ncw, s]."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    c = np.ascontiguousarray(centroids, dtype=np.float64)
    ncw, s = c.shape
    g = np.empty_like(c)
    loss = lib().orc_cos_loss_grad(_p(x), x.shape[0], x.shape[1], s, _p(c), ncw, _p(g))
    return loss, g


def finetune(x, centroids, iters: int, lr: float):
    """Gradient descent on the cosine objective; returns (centroids float64,
    codebook fp16 bits, loss per step)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    c = np.array(centroids, dtype=np.float64, copy=True, order="C")
    ncw, s = c.shape
    cb = np.empty((ncw, s), np.uint16)
    loss = np.empty(max(iters, 1), np.float64)
    lib().orc_finetune(_p(x), x.shape[0], x.shape[1], s, ncw, iters, float(lr), _p(c), _p(cb), _p(loss))
    return c, cb, loss[:iters]


def num_threads() -> int:
    return lib().orc_num_threads()


def set_num_threads(n: int) -> None:
    """Threads of the batched routines from now on (OpenMP)."""
    lib().orc_set_num_threads(int(n))


def rope(k: np.ndarray, cos, sin, pos0: int = 0) -> np.ndarray:
    """Rotate keys k float64 [..., T, d] (token t at position pos0 + t) with the
    tables cos, sin fp32 [max_pos, d/2]; returns a new array."""
    k = np.array(k, dtype=np.float64, copy=True, order="C")
    *lead, T, d = k.shape
    n = int(np.prod(lead)) if lead else 1
    cs = np.ascontiguousarray(cos, dtype=np.float32)
    sn = np.ascontiguousarray(sin, dtype=np.float32)
    assert cs.shape == sn.shape and cs.shape[1] == d // 2 and pos0 + T <= cs.shape[0]
    lib().orc_rope(_p(k), n, T, d, _p(cs), _p(sn), int(pos0))
    return k


def reference_decode(q, k_cache: dict, v_cache: dict, n_quant: int, n_resid: int,
                     R: int, codebook, scale: float | None = None, signs=None, rope_tables=None,
                     pos0: int = 0) -> np.ndarray:
    """Attention over a compressed cache, by its plain definition: reconstruct
    the n_quant quantised tokens, append the n_resid fp16 residual tokens, and
    run textbook softmax attention.  Caches are dicts with codes [B,H,cap,S],
    scales, mu (fp16 bits) and resid [B,H,R,d] (fp16 bits).  rope_tables =
    (cos, sin): the keys are stored before RoPE and are rotated to positions
    pos0 + t before the dot products."""
    qb = as_f16_bits(q)
    d = qb.shape[-1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    parts_k, parts_v = [], []
    if n_quant > 0:
        dq = bool(k_cache.get("dq", False))
        parts_k.append(dequant(k_cache["codes"], k_cache["scales"], k_cache["mu"], R, codebook, 0, n_quant,
                               signs=signs, dq=dq))
        parts_v.append(dequant(v_cache["codes"], v_cache["scales"], v_cache["mu"], R, codebook, 0, n_quant,
                               signs=signs, dq=dq))
    if n_resid > 0:
        parts_k.append(f16_to_f64(as_f16_bits(k_cache["resid"])[..., :n_resid, :]))
        parts_v.append(f16_to_f64(as_f16_bits(v_cache["resid"])[..., :n_resid, :]))
    K = np.concatenate(parts_k, axis=-2)
    V = np.concatenate(parts_v, axis=-2)
    if rope_tables is not None:
        K = rope(K, rope_tables[0], rope_tables[1], pos0)
    return attention(qb, K, V, scale)
