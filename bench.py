"""Benchmark of the NSNQuant hot path on one MI355X.

Headline: decode-attention tokens/s of the batch-scaling workload, the
LLaMA-2-7B shape with 32 layers, 32 MHA heads, batch 256, a 4096-token
context and 2-bit codes.  One step = one generated token per sequence: the
decode attention of every layer over its compressed cache (3968 quantised +
128 fp16 residual tokens per sequence).  `value` = batch / step time.  The
compressed caches of all 32 layers are resident in HBM before the timed
region (98.8 GB; the fp16 cache of the same batch, 550 GB, would not fit).

Beside it, on the same line:
  encode      the prefill encode of one batch-256 layer (NSN, Hadamard, VQ
              through the candidate lists, residual window) and the flush of
              a full residual window, tokens/s and HBM fraction;
  fp16        the uncompressed comparator at the largest batch whose fp16
              K/V of all 32 layers fits the same HBM, and the gain;
  roofline    the decode call (split kernel + combine) against 8 TB/s, timed
              with HIP events per call in a loop of its own after the timed
              region; traffic from the committed rocprofv3 counter summary;
  workloads   the LLaMA-2-7B single layer at batch 1 (2 bits) and batch 16
              (1 bit), and the LLaMA-3.1-8B GQA 32k decode step, each with its
              own fp16 comparator; the format options on the batch-1 layer;
  cpu_baseline  the CPU oracle on a bounded sample of the headline workload
              (layer 0, the first batch rows, all heads), extrapolated.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode-attn tokens/s & HBM GB/s (% roofline) + KV encode tokens/s, 2b/1b"
HEADLINE = "llama2-7b-b256-2bit"
HBM_PEAK_GBS = 8000.0
FP16_MFMA_PEAK_TFLOPS = 2500.0
# Vector ALU: 256 CUs x 4 SIMD x 16 lanes x 2.4 GHz (32-bit ops, unpacked)
VALU_PEAK_TOPS = 256 * 64 * 2.4e9 / 1e12
MALL_BYTES = 256e6  # Infinity Cache: rotated working sets must exceed it well


def progress(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def encode_bytes_per_vector(bits: int, R: int, d: int = 128) -> float:
    """HBM bytes the encode must move per head vector: fp16 input, codes,
    (n1, n2) fp16, and its share of the block mean."""
    S = d // (4 if bits == 2 else 8)
    return 2 * d + S + 4 + 2 * d / R


def dequant_bytes_per_vector(bits: int, R: int, d: int = 128) -> float:
    """Dequant, per head vector: codes S + (n1, n2) 4 + the block mean's share
    2d/R read, 2d written (fp16)."""
    return d // (4 if bits == 2 else 8) + 4 + 2 * d / R + 2 * d


def decode_bytes(bits: int, R: int, n_quant: int, n_resid: int, units: int, d: int = 128) -> float:
    """Algorithmic bytes of one decode call: K and V codes + scalars + means of
    the compressed tokens, and the fp16 residual tokens, for `units` (b, h)."""
    S = d // (4 if bits == 2 else 8)
    per_tok = 2 * (S + 4) + 2 * (2 * d / R)
    return units * (n_quant * per_tok + n_resid * 2 * 2 * d)


def decode_bytes_dq(bits: int, R: int, n_quant: int, n_resid: int, units: int, d: int = 128) -> float:
    """Algorithmic decode bytes with double-quantised records: codes, the padded
    scales record and the 80-byte mean record per block, fp16 residual."""
    S = d // (4 if bits == 2 else 8)
    rec = ((2 * R + R // 2 + 4) + 15) // 16 * 16
    per_tok = 2 * (S + (rec + 80) / R)
    return units * (n_quant * per_tok + n_resid * 2 * 2 * d)


def event_time(stream, f, n: int, warm: int = 2) -> float:
    """Mean seconds of f() over n calls, HIP events on `stream` around the loop."""
    import torch
    for _ in range(warm):
        f()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(n):
        f()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n / 1e3


def per_call_times(stream, calls, reps: int):
    """HIP-event duration of every call of `calls` (a list of callables run in
    order), over `reps` passes; returns the list of durations in seconds."""
    import torch
    evs = []
    torch.cuda.synchronize()
    for _ in range(reps):
        for f in calls:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            f()
            e1.record(stream)
            evs.append((e0, e1))
    torch.cuda.synchronize()
    return [a.elapsed_time(b) / 1e3 for a, b in evs]


def build_codebook(nsnq, synth, bits: int, R: int, dev, iters: int = 50):
    p = nsnq.params(bits, R)
    s = nsnq.sub_dim(bits)
    t0 = time.perf_counter()
    _, cb, dist = nsnq.nsnq_build_codebook(p, synth.randn_samples(0, 1 << 20, s).to(dev), iters)
    import torch
    torch.cuda.synchronize()
    return cb, dict(build_s=time.perf_counter() - t0, iters=iters, n=1 << 20,
                    final_mse_per_elem=float(dist[-1].item()))


def kernel_traffic(name: str):
    """HBM bytes per launch of a kernel from its committed rocprofv3 counter
    summary (profiles/<name>_traffic.json), or None when the kernel's sources
    have changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", name + "_traffic.json")
    try:
        rec = json.load(open(path))
        h = hashlib.sha256()
        for n in rec["sources"]:
            h.update(open(os.path.join(ROOT, "kv_cache_bit_amd", "csrc", n), "rb").read())
    except (OSError, ValueError, KeyError):
        return None
    if rec.get("sources_sha256") != h.hexdigest():
        return None
    return rec.get("bytes_per_launch")


# ------------------------------------------------------------ decode step --

def decode_step(nsnq, synth, workload: str, steps: int, warmup: int, dev, with_fp16: bool = True,
                distinct_layers: int = 2, max_layers: int = 0, keep_inputs_rows: int = 0, encode_reps: int = 0):
    """Whole-model decode step of a multi-layer workload: one new token per
    sequence, the decode attention of every layer over its own compressed
    cache.  Setup encodes `distinct_layers` layers from the generator and
    copies their caches to the other layers (every layer keeps its own
    buffers).  The timed region is exactly `steps` steps after `warmup`,
    bracketed by synchronisations, with no events inside; per-call HIP events
    follow in a loop of their own.  Optionally times the encode of layer 0
    (`encode_reps` > 0) and returns the first `keep_inputs_rows` rows of layer
    0's K/V on the host (for the CPU baseline)."""
    import numpy as np
    import torch
    w = synth.WORKLOADS[workload]
    NL, B, Hq, Hkv, L, d, bits, R = (w["layers"], w["B"], w["Hq"], w["Hkv"], w["L"], w["d"], w["bits"], w["R"])
    if max_layers > 0:
        NL = min(NL, max_layers)
    distinct_layers = min(distinct_layers, NL)
    stream = torch.cuda.current_stream()
    p = nsnq.params(bits, R)
    cb, cb_info = build_codebook(nsnq, synth, bits, R, dev)
    p_enc = nsnq.with_candidates(p, cb) if bits == 2 else p
    r = ((L - 1) % R) + 1
    nq = L - r
    units = B * Hkv
    caches, qs = [], []
    enc = None
    host_kv = None
    for layer in range(NL):
        c = nsnq.KVCache(p, B, Hkv, nq + R, dev)
        if layer < distinct_layers:
            progress(f"{workload}: generating and encoding layer {layer}")
            k, v = synth.kv_layer(w["config_id"], layer, B, Hkv, L, d,
                                  outlier_std=synth.outlier_std_for(workload, layer), device=dev)
            nsnq.nsnq_encode_kv(p_enc, cb, k, v, L, c, stream=stream)
            if layer == 0 and encode_reps > 0:
                enc = encode_layer_timing(nsnq, p_enc, p, cb, k, v, L, B, Hkv, bits, R, dev, encode_reps)
            if layer == 0 and keep_inputs_rows > 0:
                host_kv = (k[:keep_inputs_rows].cpu(), v[:keep_inputs_rows].cpu())
            del k, v
        else:
            src = caches[layer % distinct_layers]
            for dst_h, src_h in ((c.k, src.k), (c.v, src.v)):
                for name in ("codes", "scales", "mu", "resid"):
                    getattr(dst_h, name).copy_(getattr(src_h, name))
            c.n_quant, c.n_resid = src.n_quant, src.n_resid
        caches.append(c)
        qs.append(synth.queries(w["config_id"], layer, B, Hq, d, device=dev))
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    ws = torch.empty(nsnq.nsnq_decode_workspace_bytes(p, caches[0], Hq), dtype=torch.uint8, device=dev)
    outs = [torch.empty_like(q) for q in qs]

    def call(layer):
        return lambda: nsnq.nsnq_decode_attention(p, cb, qs[layer], caches[layer], out=outs[layer], ws=ws,
                                                  stream=stream)
    calls = [call(layer) for layer in range(NL)]

    def step():
        for f in calls:
            f()

    progress(f"{workload}: timing {steps} decode steps over {NL} layers")
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_step = wall / steps
    # per-call HIP events (their own loop, >= 20 passes)
    reps = max(20, steps)
    durs = np.array(per_call_times(stream, calls, reps))
    t_call = float(durs.mean())
    step_s = durs.reshape(reps, NL).sum(axis=1)
    cache_bytes = sum(c.nbytes() for c in caches)
    call_b = decode_bytes(bits, R, nq, r, units, d)
    dec_b = NL * call_b
    # the same step with the keys read as stored before RoPE (the pages' key
    # order): standard RoPE tables, positions 0 .. L - 1
    cos, sin = (t.to(dev).contiguous() for t in synth.rope_tables(L + 8))

    def call_pre(layer):
        return lambda: nsnq.nsnq_decode_attention_prerope(p, cb, qs[layer], caches[layer], cos, sin, 0,
                                                          out=outs[layer], ws=ws, stream=stream)
    calls_pre = [call_pre(layer) for layer in range(NL)]
    progress(f"{workload}: timing {min(steps, 5)} decode steps with keys stored before RoPE")
    for f in calls_pre:
        f()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(min(steps, 5)):
        for f in calls_pre:
            f()
    torch.cuda.synchronize()
    t_pre = (time.perf_counter() - t0) / min(steps, 5)
    prerope = {"step_ms": t_pre * 1e3, "tokens_per_s": B / t_pre, "hbm_gbs": dec_b / t_pre / 1e9,
               "hbm_frac": dec_b / t_pre / 1e9 / HBM_PEAK_GBS, "vs_post_rope": t_pre / t_step,
               "steps": min(steps, 5),
               "note": "keys rebuilt per token (codewords, Hadamard on the matrix cores, scale, mean) and rotated "
                       "with fp32 tables before the product; values as in the post-RoPE step"}
    del caches, ws, outs, cos, sin
    torch.cuda.empty_cache()
    res = {"workload": workload, "layers": NL, "batch": B, "q_heads": Hq, "kv_heads": Hkv, "context": L,
           "bits": bits, "residual": R, "encoded_tokens": nq, "residual_tokens": r,
           "step_ms": t_step * 1e3, "tokens_per_s": B / t_step,
           "kv_tokens_per_s": NL * units * L / t_step,
           "hbm_gbs": dec_b / t_step / 1e9, "hbm_frac": dec_b / t_step / 1e9 / HBM_PEAK_GBS,
           "bytes_per_step": dec_b, "compressed_cache_gb": cache_bytes / 1e9,
           "call": {"us_mean": t_call * 1e6, "us_p10": float(np.percentile(durs, 10)) * 1e6,
                    "us_p90": float(np.percentile(durs, 90)) * 1e6, "samples": int(durs.size),
                    "bytes": call_b, "hbm_gbs": call_b / t_call / 1e9,
                    "hbm_frac": call_b / t_call / 1e9 / HBM_PEAK_GBS,
                    "step_ms_events_median": float(np.median(step_s)) * 1e3},
           "codebook": cb_info, "prerope": prerope,
           "setup": f"{distinct_layers} distinct layers encoded, caches copied to the other {NL - distinct_layers}"}
    if enc is not None:
        res["encode"] = enc
    if with_fp16:
        res["fp16"] = fp16_comparator(nsnq, synth, w, NL, qs[0], dev, steps, B, t_step)
    del qs
    torch.cuda.empty_cache()
    return res, host_kv, cb


def encode_layer_timing(nsnq, p_enc, p, cb, k, v, L, B, Hkv, bits, R, dev, reps):
    """Prefill encode of one whole layer (the candidate-list search at 2 bits)
    into a cache of its own, and the flush of a full residual window."""
    import torch
    stream = torch.cuda.current_stream()
    r = ((L - 1) % R) + 1
    nq = L - r
    c = nsnq.KVCache(p, B, Hkv, nq + R, dev)

    def enc():
        c.n_quant = c.n_resid = 0
        nsnq.nsnq_encode_kv(p_enc, cb, k, v, L, c, stream=stream)
    t = event_time(stream, enc, reps, warm=1)
    units = B * Hkv
    n_vec = 2 * units * nq
    byts = n_vec * encode_bytes_per_vector(bits, R) + 2 * units * r * 2 * 128 * 2
    # flush: the window of every (row, head) is full after the prefill
    c.n_quant, c.n_resid = nq - R, R

    def flush():
        c.n_quant, c.n_resid = nq - R, R
        nsnq.nsnq_flush_residual(p_enc, cb, c, stream=stream)
    tf = event_time(stream, flush, reps, warm=1)
    fl_vec = 2 * units * R
    fl_b = fl_vec * (encode_bytes_per_vector(bits, R) + 0.0)
    s = 128 // nsnq.sub_dim(bits)
    span = p_enc.vq_span if p_enc is not p else 256
    del c
    return {"us": t * 1e6, "tokens_per_s": B * L / t, "vectors_per_s": n_vec / t,
            "hbm_gbs": byts / t / 1e9, "hbm_frac": byts / t / 1e9 / HBM_PEAK_GBS, "bytes": byts,
            "search": (f"orthant candidate lists, {span} of 256 codewords per sub-vector" if span < 256
                       else "exhaustive, 256 codewords per sub-vector"),
            "distance_gemm_tflops_alg": n_vec * 65536 / t / 1e12,
            "distance_gemm_frac_alg": n_vec * 65536 / t / 1e12 / FP16_MFMA_PEAK_TFLOPS,
            "compared_per_s": n_vec * s * span / t,
            "flush": {"us": tf * 1e6, "tokens": B * R, "tokens_per_s": B * R / tf,
                      "hbm_frac": fl_b / tf / 1e9 / HBM_PEAK_GBS}}


def encode_bench(nsnq, synth, workload: str, dev, reps: int = 5):
    """Prefill encode of layer 0 of `workload` alone (for profiling)."""
    import torch
    w = synth.WORKLOADS[workload]
    B, Hkv, L, d, bits, R = w["B"], w["Hkv"], w["L"], w["d"], w["bits"], w["R"]
    p = nsnq.params(bits, R)
    cb, _ = build_codebook(nsnq, synth, bits, R, dev)
    p_enc = nsnq.with_candidates(p, cb) if bits == 2 else p
    k, v = synth.kv_layer(w["config_id"], 0, B, Hkv, L, d, outlier_std=synth.outlier_std_for(workload, 0),
                          device=dev)
    res = encode_layer_timing(nsnq, p_enc, p, cb, k, v, L, B, Hkv, bits, R, dev, reps)
    res["workload"] = workload
    return res


def fp16_comparator(nsnq, synth, w, NL, q, dev, steps, B, t_step):
    """The fp16-cache decode at the largest batch whose K/V of all layers fits
    the HBM left free (less an 8 GB reserve).  Two layers' caches are held and
    alternate across the layer loop (each far larger than the Infinity Cache)."""
    import torch
    stream = torch.cuda.current_stream()
    Hkv, L, d, Hq = w["Hkv"], w["L"], w["d"], w["Hq"]
    free, _ = torch.cuda.mem_get_info()
    budget = free - 8e9
    per_seq = NL * 2 * Hkv * L * d * 2
    B16 = int(max(1, min(B, budget // per_seq)))
    progress(f"fp16 comparator: batch {B16}")
    g = torch.Generator(device=dev)
    g.manual_seed(12345)
    kf = [torch.randn(B16, Hkv, L, d, device=dev, dtype=torch.float16, generator=g) for _ in range(2)]
    vf = [torch.randn(B16, Hkv, L, d, device=dev, dtype=torch.float16, generator=g) for _ in range(2)]
    q16 = q[:B16].contiguous()
    ws16 = torch.empty(nsnq.nsnq_fp16_decode_workspace_bytes(B16, Hq, L), dtype=torch.uint8, device=dev)
    o16 = torch.empty_like(q16)

    def step16():
        for layer in range(NL):
            nsnq.nsnq_fp16_decode_attention(q16, kf[layer % 2], vf[layer % 2], out=o16, ws=ws16, stream=stream)
    n = max(3, min(steps, 10))
    t16 = event_time(stream, step16, n)
    b16 = NL * B16 * Hkv * L * 2 * 2 * d
    del kf, vf, ws16
    torch.cuda.empty_cache()
    return {"batch": B16, "step_ms": t16 * 1e3, "tokens_per_s": B16 / t16, "hbm_gbs": b16 / t16 / 1e9,
            "hbm_frac": b16 / t16 / 1e9 / HBM_PEAK_GBS, "cache_gb": per_seq * B16 / 1e9,
            "budget_gb": budget / 1e9, "gain_tokens_per_s": (B / t_step) / (B16 / t16)}


# ------------------------------------------------------ single-layer case --

def layer_bench(nsnq, synth, workload: str, dev, reps: int = 20, options: bool = False, keep_rows: int = 0):
    """One layer: prefill encode (candidate lists at 2 bits; the exhaustive
    search beside it), decode, and the fp16 comparator on the same layer.
    Inputs and caches rotate over enough copies that each rotated set exceeds
    1 GB (the 256 MB Infinity Cache cannot serve it)."""
    import torch
    w = synth.WORKLOADS[workload]
    B, Hq, Hkv, L, d, bits, R = w["B"], w["Hq"], w["Hkv"], w["L"], w["d"], w["bits"], w["R"]
    stream = torch.cuda.current_stream()
    p = nsnq.params(bits, R)
    cb, cb_info = build_codebook(nsnq, synth, bits, R, dev)
    p_enc = nsnq.with_candidates(p, cb) if bits == 2 else p
    k, v = synth.kv_layer(w["config_id"], 0, B, Hkv, L, d, device=dev)
    q = synth.queries(w["config_id"], 0, B, Hq, d, device=dev)
    r = ((L - 1) % R) + 1
    nq = L - r
    units = B * Hkv
    progress(f"{workload}: encode")
    in_bytes = 2 * k.numel() * 2
    n_in = max(4, math.ceil(1e9 / in_bytes))
    ks = [k] + [k.clone() for _ in range(n_in - 1)]
    vs = [v] + [v.clone() for _ in range(n_in - 1)]
    enc_cache = nsnq.KVCache(p, B, Hkv, nq + R, dev)
    it = [0]

    def enc(pp):
        def f():
            i = it[0] % n_in
            it[0] += 1
            enc_cache.n_quant = enc_cache.n_resid = 0
            nsnq.nsnq_encode_kv(pp, cb, ks[i], vs[i], L, enc_cache, stream=stream)
        return f
    t_enc = event_time(stream, enc(p_enc), reps)
    t_exh = event_time(stream, enc(p), reps) if p_enc is not p else None
    n_vec = 2 * units * nq
    enc_b = n_vec * encode_bytes_per_vector(bits, R, d) + 2 * units * r * 2 * d * 2
    del ks, vs
    # decode over rotated copies of the encoded cache
    progress(f"{workload}: decode")
    enc_cache.n_quant = enc_cache.n_resid = 0
    nsnq.nsnq_encode_kv(p_enc, cb, k, v, L, enc_cache, stream=stream)
    n_c = max(4, math.ceil(1e9 / enc_cache.nbytes()))
    caches = [enc_cache]
    for _ in range(n_c - 1):
        c = nsnq.KVCache(p, B, Hkv, nq + R, dev)
        for dst_h, src_h in ((c.k, enc_cache.k), (c.v, enc_cache.v)):
            for name in ("codes", "scales", "mu", "resid"):
                getattr(dst_h, name).copy_(getattr(src_h, name))
        c.n_quant, c.n_resid = enc_cache.n_quant, enc_cache.n_resid
        caches.append(c)
    ws = torch.empty(nsnq.nsnq_decode_workspace_bytes(p, enc_cache, Hq), dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)
    it[0] = 0

    def dec():
        c = caches[it[0] % n_c]
        it[0] += 1
        nsnq.nsnq_decode_attention(p, cb, q, c, out=out, ws=ws, stream=stream)
    t_dec = event_time(stream, dec, max(reps, 2 * n_c))
    dec_b = decode_bytes(bits, R, nq, r, units, d)
    # dequant of every compressed token, K and V, to fp16, over the rotated
    # caches and rotated output buffers
    progress(f"{workload}: dequant")
    out_b = units * nq * d * 2
    n_o = max(4, math.ceil(1e9 / out_b))
    outs = [torch.empty(B, Hkv, nq, d, dtype=torch.float16, device=dev) for _ in range(n_o)]
    it[0] = 0

    def deq():
        c, o = caches[it[0] % n_c], outs[it[0] % n_o]
        it[0] += 1
        nsnq.nsnq_dequant(p, cb, c, 0, 0, nq, out=o, stream=stream)
        nsnq.nsnq_dequant(p, cb, c, 1, 0, nq, out=o, stream=stream)
    t_deq = event_time(stream, deq, max(reps, 2 * max(n_c, n_o)))
    deq_b = 2 * units * nq * dequant_bytes_per_vector(bits, R, d)
    del caches, ws, outs
    torch.cuda.empty_cache()
    # fp16 comparator over rotated copies of the layer's K/V
    kf, vf = k.contiguous(), v.contiguous()
    n16 = max(4, math.ceil(1e9 / (2 * kf.numel() * 2)))
    kfs = [kf] + [kf.clone() for _ in range(n16 - 1)]
    vfs = [vf] + [vf.clone() for _ in range(n16 - 1)]
    ws16 = torch.empty(nsnq.nsnq_fp16_decode_workspace_bytes(B, Hq, L), dtype=torch.uint8, device=dev)
    o16 = torch.empty_like(q)
    it[0] = 0

    def dec16():
        i = it[0] % n16
        it[0] += 1
        nsnq.nsnq_fp16_decode_attention(q, kfs[i], vfs[i], out=o16, ws=ws16, stream=stream)
    t16 = event_time(stream, dec16, max(reps, 2 * n16))
    b16 = units * L * 2 * 2 * d
    del kfs, vfs, ws16
    s = d // nsnq.sub_dim(bits)
    span = p_enc.vq_span if p_enc is not p else 256
    res = {"workload": workload, "bits": bits, "batch": B, "q_heads": Hq, "kv_heads": Hkv, "context": L,
           "encode": {"us": t_enc * 1e6, "tokens_per_s": B * L / t_enc, "vectors_per_s": n_vec / t_enc,
                      "hbm_gbs": enc_b / t_enc / 1e9, "hbm_frac": enc_b / t_enc / 1e9 / HBM_PEAK_GBS,
                      "bytes": enc_b, "rotated_copies": n_in,
                      "search": (f"orthant candidate lists, {span} of 256 codewords per sub-vector"
                                 if span < 256 else "exhaustive, 256 codewords per sub-vector"),
                      "compared_per_s": n_vec * s * span / t_enc,
                      "valu_frac_of_compares": n_vec * s * span * 1.5 / t_enc / 1e12 / VALU_PEAK_TOPS,
                      "exhaustive_us": None if t_exh is None else t_exh * 1e6},
           "decode": {"us": t_dec * 1e6, "tokens_per_s": B / t_dec, "kv_tokens_per_s": units * L / t_dec,
                      "hbm_gbs": dec_b / t_dec / 1e9, "hbm_frac": dec_b / t_dec / 1e9 / HBM_PEAK_GBS,
                      "bytes": dec_b, "rotated_copies": n_c},
           "dequant": {"us": t_deq * 1e6, "vectors_per_s": 2 * units * nq / t_deq, "hbm_gbs": deq_b / t_deq / 1e9,
                       "hbm_frac": deq_b / t_deq / 1e9 / HBM_PEAK_GBS, "bytes": deq_b,
                       "note": "K and V of every compressed token to fp16, one call each"},
           "fp16_decode": {"us": t16 * 1e6, "tokens_per_s": B / t16, "hbm_gbs": b16 / t16 / 1e9,
                           "hbm_frac": b16 / t16 / 1e9 / HBM_PEAK_GBS, "bytes": b16, "rotated_copies": n16,
                           "compressed_speedup": t16 / t_dec},
           "codebook": cb_info}
    if options:
        res["options"] = measure_options(nsnq, synth, w, k, v, q, cb, dev)
    host_kv = (k[:keep_rows].cpu(), v[:keep_rows].cpu()) if keep_rows > 0 else None
    del k, v
    torch.cuda.empty_cache()
    return res, host_kv


def measure_options(nsnq, synth, w: dict, k, v, q, codebook, dev, reps: int = 20):
    """The format options on one layer, each against the same inputs: double
    quantisation, randomised Hadamard + Strategy 3, decode over keys stored
    before RoPE, and the cosine refinement of the codebook."""
    import torch
    B, Hq, Hkv, L, d, bits, R = w["B"], w["Hq"], w["Hkv"], w["L"], w["d"], w["bits"], w["R"]
    r = ((L - 1) % R) + 1
    nq = L - r
    units = B * Hkv
    stream = torch.cuda.current_stream()

    def layer(p):
        if bits == 2:  # the same nearest-codeword search as the headline encode
            p = nsnq.with_candidates(p, codebook)
        cache = nsnq.KVCache(p, B, Hkv, nq + R, dev)

        def enc():
            cache.n_quant = cache.n_resid = 0
            nsnq.nsnq_encode_kv(p, codebook, k, v, L, cache, stream=stream)
        t_enc = event_time(stream, enc, reps)
        cache.n_quant, cache.n_resid = nq, r
        ws = torch.empty(max(16, nsnq.nsnq_decode_workspace_bytes(p, cache, Hq)), dtype=torch.uint8, device=dev)
        out = torch.empty_like(q)
        t_dec = event_time(stream, lambda: nsnq.nsnq_decode_attention(p, codebook, q, cache, out=out, ws=ws,
                                                                      stream=stream), reps)
        return cache, ws, out, t_enc, t_dec

    res = {"note": "single layer, inputs not rotated: times are cache-warm"}
    p = nsnq.params(bits, R, flags=nsnq.NSNQ_DOUBLE_QUANT)
    _, _, _, te, td = layer(p)
    db = decode_bytes_dq(bits, R, nq, r, units, d)
    res["double_quant"] = {"encode_us": te * 1e6, "decode_us": td * 1e6, "decode_bytes": db,
                           "bytes_vs_plain": db / decode_bytes(bits, R, nq, r, units, d)}
    signs = synth.hadamard_signs(1, d).to(dev)
    p = nsnq.params(bits, R, flags=nsnq.NSNQ_SCALE_ADJUST, signs=signs)
    _, _, _, te, td = layer(p)
    res["rht_scale_adjust"] = {"encode_us": te * 1e6, "decode_us": td * 1e6}
    p = nsnq.params(bits, R)
    cache, ws, out, _, td_plain = layer(p)
    cos, sin = synth.rope_tables(L + 1, 10000.0, d)
    cos, sin = cos.to(dev), sin.to(dev)
    tr = event_time(stream, lambda: nsnq.nsnq_decode_attention_prerope(p, codebook, q, cache, cos, sin, 0, out=out,
                                                                        ws=ws, stream=stream), reps)
    res["prerope_decode"] = {"us": tr * 1e6, "vs_post_rope": tr / td_plain}
    s = nsnq.sub_dim(bits)
    cent, _, _ = nsnq.nsnq_build_codebook(p, synth.randn_samples(0, 1 << 18, s).to(dev), 20)
    x = synth.randn_samples(5, 1 << 16, d).to(dev)
    xt = synth.randn_samples(6, 1 << 14, d).to(dev)
    c0 = cent.clone()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    cent, _, loss = nsnq.nsnq_finetune_codebook(p, x, 20, 64.0, cent)
    torch.cuda.synchronize()
    tf = time.perf_counter() - t0
    _, _, l0 = nsnq.nsnq_finetune_codebook(p, xt, 1, 0.0, c0.clone())
    _, _, l1 = nsnq.nsnq_finetune_codebook(p, xt, 1, 0.0, cent.clone())
    res["cosine_finetune"] = {"s": tf, "iters": 20, "n": 1 << 16, "lr": 64.0,
                              "train_loss": [float(loss[0]), float(loss[-1])],
                              "held_out_loss": [float(l0[0]), float(l1[0])]}
    return res


# ------------------------------------------------------------ CPU oracle --

def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w: dict, host_kv, rows: int, layers: int, single_thread: bool = True):
    """The CPU oracle on layer 0's first `rows` batch rows, all heads: their
    prefill encode and one decode step, timed; scaled linearly by the units of
    the whole workload (batch x layers) and labelled as extrapolated when that
    scale is above 1.  The codebook is the oracle's own k-means fit (its values
    do not change the oracle's work)."""
    import numpy as np
    import oracle
    from kv_cache_bit_amd import synth
    R, d, bits, L = w["R"], w["d"], w["bits"], w["L"]
    B, Hq, Hkv = w["B"], w["Hq"], w["Hkv"]
    s = 4 if bits == 2 else 8
    _, cb, _ = oracle.kmeans(synth.randn_samples(0, 1 << 14, s).numpy(), 256, 10)
    k, v = host_kv
    k, v = k[:rows].contiguous(), v[:rows].contiguous()
    q = synth.queries(w["config_id"], 0, rows, Hq, d)
    t0 = time.perf_counter()
    ek, ev = oracle.encode(k, R, cb), oracle.encode(v, R, cb)
    t1 = time.perf_counter()
    oracle.reference_decode(q, ek, ev, ek["n_quant"], ek["n_resid"], R, cb)
    t2 = time.perf_counter()
    cores = oracle.num_threads()
    scale = (B / rows) * layers
    dec_step = (t2 - t1) * scale
    enc_layer = (t1 - t0) * B / rows
    try:
        nproc = len(os.sched_getaffinity(0))
    except AttributeError:
        nproc = os.cpu_count()
    res = {"value": B / dec_step, "unit": "tokens/s", "cores": cores, "kind": "oracle",
           "sample": (f"layer 0, batch rows 0..{rows - 1} of {B}, all {Hkv} KV heads: prefill encode "
                      f"{t1 - t0:.1f} s and one decode step {t2 - t1:.1f} s measured"
                      + (f"; extrapolated x{scale:g} to the {layers}-layer batch-{B} step" if scale > 1 else "")),
           "extrapolated": scale > 1, "measured_s": t2 - t0,
           "encode_tokens_per_s": B * L / enc_layer,
           "encode_layer_s": enc_layer,
           "decode_step_s": dec_step,
           "nproc": nproc, "cpu_model": cpu_model()}
    if single_thread:
        # one KV head of one row on one thread
        oracle.set_num_threads(1)
        try:
            t3 = time.perf_counter()
            e1k = oracle.encode(k[:1, :1].contiguous(), R, cb)
            e1v = oracle.encode(v[:1, :1].contiguous(), R, cb)
            t4 = time.perf_counter()
            oracle.reference_decode(q[:1, :Hq // Hkv].contiguous(), e1k, e1v, e1k["n_quant"], e1k["n_resid"], R,
                                    cb)
            t5 = time.perf_counter()
        finally:
            oracle.set_num_threads(cores)
        dec_1t = (t5 - t4) * B * Hkv * layers
        res["single_thread"] = {"value": B / dec_1t, "unit": "tokens/s", "cores": 1,
                                "sample": (f"layer 0, row 0, one KV head on one thread ({t5 - t4:.2f} s decode); "
                                           f"extrapolated x{B * Hkv * layers}")}
    return res


def copy_calibration(nbytes: int, reps: int):
    """Plain device-to-device copy of `nbytes`, for scaling FETCH_SIZE /
    WRITE_SIZE counters to bytes."""
    import torch
    dev = torch.device("cuda:0")
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "reps": reps}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=HEADLINE, help="multi-layer workload of the headline decode step")
    ap.add_argument("--cpu-rows", type=int, default=24,
                    help="batch rows of layer 0 in the CPU-baseline sample (0: skip)")
    ap.add_argument("--no-fp16", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="headline only: skip the other workloads")
    ap.add_argument("--only", default="", help="run one part for profiling: headline, layer:<workload>, "
                                                "step:<workload>, encode:<workload>")
    ap.add_argument("--copy-bytes", type=int, default=0, help="only run a device copy of this size")
    ap.add_argument("--decode-layers", type=int, default=0, help="time the decode of only this many layers")
    args = ap.parse_args()
    if args.copy_bytes:
        copy_calibration(args.copy_bytes, max(args.steps, 1))
        return
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(this path has no multi-GPU code).", file=sys.stderr)
        sys.exit(2)

    import torch
    from kv_cache_bit_amd import nsnq, synth

    nsnq.lib()  # fail loudly if the HIP library is missing
    assert torch.cuda.is_available(), "bench needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.only.startswith("layer:"):
        print(json.dumps(layer_bench(nsnq, synth, args.only[6:], dev, reps=max(args.steps, 4))[0]), flush=True)
        return
    if args.only.startswith("encode:"):
        print(json.dumps(encode_bench(nsnq, synth, args.only[7:], dev, reps=max(args.steps, 3))), flush=True)
        return
    if args.only.startswith("step:"):
        r, _, _ = decode_step(nsnq, synth, args.only[5:], args.steps, args.warmup, dev,
                              with_fp16=not args.no_fp16, max_layers=args.decode_layers)
        print(json.dumps(r), flush=True)
        return

    w = synth.WORKLOADS[args.workload]
    head, host_kv, _ = decode_step(nsnq, synth, args.workload, args.steps, args.warmup, dev,
                                   with_fp16=not args.no_fp16 and args.only != "headline",
                                   max_layers=args.decode_layers,
                                   keep_inputs_rows=args.cpu_rows if args.only != "headline" else 0,
                                   encode_reps=5 if args.only != "headline" else 0)
    call = head["call"]
    traffic = kernel_traffic(f"decode_{args.workload}")
    res = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["step_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "layers": head["layers"], "batch": head["batch"],
                   "q_heads": head["q_heads"], "kv_heads": head["kv_heads"], "context": head["context"],
                   "head_dim": 128, "bits": head["bits"], "residual": head["residual"],
                   "encoded_tokens": head["encoded_tokens"], "residual_tokens": head["residual_tokens"]},
        "hbm_gbs": head["hbm_gbs"],
        "hbm_frac": head["hbm_frac"],
        "roofline": {"kernel": "decode attention call: decode_split_kernel<4, 1, false, false> + combine_kernel",
                     "bound": "hbm", "achieved": call["hbm_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": call["hbm_frac"], "traffic": traffic,
                     "bytes_per_launch": call["bytes"], "launch_us": call["us_mean"],
                     "note": ("achieved = algorithmic bytes of one layer's decode call (K and V codes 32 B + "
                              "(n1, n2) 4 B each per compressed token-head, the block means' share, fp16 residual "
                              "tokens) / the call's mean HIP-event duration over 20 passes of all layers")},
        "decode_step": {k: head[k] for k in ("step_ms", "tokens_per_s", "kv_tokens_per_s", "hbm_gbs",
                                             "hbm_frac", "bytes_per_step", "compressed_cache_gb", "call",
                                             "prerope", "setup")},
        "codebook": head["codebook"],
    }
    if "encode" in head:
        res["encode"] = head["encode"]
    if "fp16" in head:
        res["fp16"] = head["fp16"]
    cpu_samples = []  # (workload, host K/V rows, rows, layers)
    if not args.no_extra and args.only != "headline":
        res["workloads"] = {}
        for wl, opts in (("llama2-7b-layer-b1-2bit", True), ("llama2-7b-layer-b16-1bit", False)):
            res["workloads"][wl], hkv = layer_bench(nsnq, synth, wl, dev, options=opts,
                                                    keep_rows=1 if args.cpu_rows > 0 else 0)
            cpu_samples.append((wl, hkv, 1, 1))
        wl = "llama3.1-8b-gqa-b4-32k-2bit"
        r4, hkv, _ = decode_step(nsnq, synth, wl, args.steps, args.warmup, dev, with_fp16=not args.no_fp16,
                                 keep_inputs_rows=1 if args.cpu_rows > 0 else 0)
        res["workloads"][wl] = r4
        cpu_samples.append((wl, hkv, 1, synth.WORKLOADS[wl]["layers"]))
    if args.cpu_rows > 0 and host_kv is not None:
        progress("CPU oracle baseline")
        res["cpu_baseline"] = cpu_baseline(w, host_kv, min(args.cpu_rows, w["B"]), head["layers"])
        res["cpu_baseline"]["workloads"] = {}
        for wl, hkv, rows, layers in cpu_samples:
            if hkv is not None:
                cb_ = cpu_baseline(synth.WORKLOADS[wl], hkv, rows, layers, single_thread=False)
                res["cpu_baseline"]["workloads"][wl] = {key: cb_[key] for key in (
                    "value", "unit", "sample", "extrapolated", "encode_tokens_per_s", "decode_step_s")}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
