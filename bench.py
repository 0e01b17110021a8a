"""Benchmark of the NSNQuant hot path on one MI355X.

One step = prefill encode of a whole layer's K/V context (NSN, Hadamard, VQ,
residual window) followed by one decode-attention step over the compressed
cache, on synthetic K/V shaped like the named LLaMA layer.  Inputs are resident
in HBM before the timed region; input and cache buffers rotate over several
copies so the 256 MB Infinity Cache cannot serve them.

Prints one JSON line.  `value` is context tokens (batch x context length)
taken through encode + decode per second.
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
HBM_PEAK_GBS = 8000.0
# Vector ALU: 256 CUs x 4 SIMD x 16 lanes x 2.4 GHz (32-bit ops, unpacked)
VALU_PEAK_TOPS = 256 * 64 * 2.4e9 / 1e12


def encode_bytes_per_vector(bits: int, R: int, d: int = 128) -> float:
    """HBM bytes the encode must move per head vector: fp16 input, codes,
    (n1, n2) fp16, and its share of the block mean."""
    S = d // (4 if bits == 2 else 8)
    return 2 * d + S + 4 + 2 * d / R


def decode_bytes(bits: int, R: int, n_quant: int, n_resid: int, units: int, d: int = 128) -> float:
    """Algorithmic bytes of one decode step: K and V codes + scalars + means of
    the compressed tokens, and the fp16 residual tokens, for `units` (b, h)."""
    S = d // (4 if bits == 2 else 8)
    per_tok = 2 * (S + 4) + 2 * (2 * d / R)
    return units * (n_quant * per_tok + n_resid * 2 * 2 * d)


def measure_layer(nsnq, synth, workload: str, reps: int, dev):
    """Encode and decode timing of one layer of `workload` (no CPU baseline):
    mean HIP-event times over `reps` calls on rotating buffers."""
    import numpy as np
    import torch
    w = synth.WORKLOADS[workload]
    B, Hq, Hkv, L, d, bits, R = w["B"], w["Hq"], w["Hkv"], w["L"], w["d"], w["bits"], w["R"]
    p = nsnq.params(bits, R)
    s = nsnq.sub_dim(bits)
    _, cb, _ = nsnq.nsnq_build_codebook(p, synth.randn_samples(0, 1 << 18, s).to(dev), 20)
    k, v = synth.kv_layer(w["config_id"], 0, B, Hkv, L, d, device=dev)
    q = synth.queries(w["config_id"], 0, B, Hq, d, device=dev)
    nbuf = max(1, min(4, math.ceil(512e6 / (4 * k.numel()))))
    ks = [k] + [k.clone() for _ in range(nbuf - 1)]
    vs = [v] + [v.clone() for _ in range(nbuf - 1)]
    r = ((L - 1) % R) + 1
    nq = L - r
    caches = [nsnq.KVCache(p, B, Hkv, nq + R, dev) for _ in range(nbuf)]
    for i in range(nbuf):
        nsnq.nsnq_encode_kv(p, cb, ks[i], vs[i], L, caches[i])
    ws = torch.empty(nsnq.nsnq_decode_workspace_bytes(p, caches[0], Hq), dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()

    def enc(i):
        c = caches[i % nbuf]
        c.n_quant = c.n_resid = 0
        nsnq.nsnq_encode_kv(p, cb, ks[i % nbuf], vs[i % nbuf], L, c, stream=stream)

    def dec(i):
        nsnq.nsnq_decode_attention(p, cb, q, caches[i % nbuf], out=out, ws=ws, stream=stream)

    res = {}
    for name, f in (("encode", enc), ("decode", dec)):
        for i in range(3):
            f(i)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(reps):
            f(i)
        e1.record(stream)
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) / reps / 1e3
    units = B * Hkv
    n_vec = 2 * units * nq
    enc_b = n_vec * encode_bytes_per_vector(bits, R, d) + 2 * units * r * 2 * d * 2
    dec_b = decode_bytes(bits, R, nq, r, units, d)
    del ks, vs, caches
    return {"workload": workload, "bits": bits, "batch": B, "context": L,
            "encode": {"us": res["encode"] * 1e6, "tokens_per_s": B * L / res["encode"],
                       "hbm_gbs": enc_b / res["encode"] / 1e9,
                       "hbm_frac": enc_b / res["encode"] / 1e9 / HBM_PEAK_GBS},
            "decode": {"us": res["decode"] * 1e6, "tokens_per_s": B / res["decode"],
                       "hbm_gbs": dec_b / res["decode"] / 1e9,
                       "hbm_frac": dec_b / res["decode"] / 1e9 / HBM_PEAK_GBS, "bytes": dec_b}}


def decode_bytes_dq(bits: int, R: int, n_quant: int, n_resid: int, units: int, d: int = 128) -> float:
    """Algorithmic decode bytes with double-quantised records: codes, the padded
    scales record and the 80-byte mean record per block, fp16 residual."""
    S = d // (4 if bits == 2 else 8)
    rec = ((2 * R + R // 2 + 4) + 15) // 16 * 16
    per_tok = 2 * (S + (rec + 80) / R)
    return units * (n_quant * per_tok + n_resid * 2 * 2 * d)


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

    def timed(f, n=reps):
        for _ in range(3):
            f()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(n):
            f()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n / 1e3

    def layer(p):
        if bits == 2:  # the same nearest-codeword search as the headline encode
            p = nsnq.with_candidates(p, codebook)
        cache = nsnq.KVCache(p, B, Hkv, nq + R, dev)
        ws = torch.empty(max(16, nsnq.nsnq_decode_workspace_bytes(p, cache, Hq)), dtype=torch.uint8, device=dev)

        def enc():
            cache.n_quant = cache.n_resid = 0
            nsnq.nsnq_encode_kv(p, codebook, k, v, L, cache, stream=stream)
        t_enc = timed(enc)
        cache.n_quant, cache.n_resid = nq, r
        ws = torch.empty(max(16, nsnq.nsnq_decode_workspace_bytes(p, cache, Hq)), dtype=torch.uint8, device=dev)
        out = torch.empty_like(q)
        t_dec = timed(lambda: nsnq.nsnq_decode_attention(p, codebook, q, cache, out=out, ws=ws, stream=stream))
        return cache, ws, out, t_enc, t_dec

    res = {}
    p = nsnq.params(bits, R, flags=nsnq.NSNQ_DOUBLE_QUANT)
    _, _, _, te, td = layer(p)
    db = decode_bytes_dq(bits, R, nq, r, units, d)
    res["double_quant"] = {"encode_us": te * 1e6, "decode_us": td * 1e6, "decode_bytes": db,
                           "decode_hbm_frac": db / td / 1e9 / HBM_PEAK_GBS,
                           "bytes_vs_plain": db / decode_bytes(bits, R, nq, r, units, d)}
    signs = synth.hadamard_signs(1, d).to(dev)
    p = nsnq.params(bits, R, flags=nsnq.NSNQ_SCALE_ADJUST, signs=signs)
    _, _, _, te, td = layer(p)
    res["rht_scale_adjust"] = {"encode_us": te * 1e6, "decode_us": td * 1e6}
    p = nsnq.params(bits, R)
    cache, ws, out, _, td_plain = layer(p)
    p = nsnq.params(bits, R)
    cos, sin = synth.rope_tables(L + 1, 10000.0, d)
    cos, sin = cos.to(dev), sin.to(dev)
    tr = timed(lambda: nsnq.nsnq_decode_attention_prerope(p, codebook, q, cache, cos, sin, 0, out=out, ws=ws,
                                                          stream=stream))
    res["prerope_decode"] = {"us": tr * 1e6, "vs_post_rope": tr / td_plain,
                             "hbm_frac": decode_bytes(bits, R, nq, r, units, d) / tr / 1e9 / HBM_PEAK_GBS}
    # cosine refinement from the k-means centroids: 20 steps on 2^16 head vectors
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


def decode_step_bench(nsnq, synth, workload: str, steps: int, dev, distinct_layers: int = 2,
                      max_layers: int = 0, with_fp16: bool = True):
    """Whole-model decode step (every layer's decode attention, one new token
    per sequence) on a multi-layer workload, against the fp16-cache comparator
    at the largest batch whose fp16 cache fits the same HBM budget.

    Setup encodes `distinct_layers` layers from the generator and copies their
    compressed caches to the remaining layers, so every layer has its own
    buffers (no cache reuse across layers) without generating hundreds of GB
    of fp16 input.  The fp16 side holds two layers' caches and alternates
    between them across the layer loop (each is far larger than the 256 MB
    Infinity Cache)."""
    import numpy as np
    import torch
    w = synth.WORKLOADS[workload]
    NL, B, Hq, Hkv, L, d, bits, R = (w["layers"], w["B"], w["Hq"], w["Hkv"], w["L"], w["d"], w["bits"], w["R"])
    if max_layers > 0:
        NL = min(NL, max_layers)
        distinct_layers = min(distinct_layers, NL)
    p = nsnq.params(bits, R)
    s = nsnq.sub_dim(bits)
    _, cb, _ = nsnq.nsnq_build_codebook(p, synth.randn_samples(0, 1 << 20, s).to(dev), 50)
    r = ((L - 1) % R) + 1
    nq = L - r
    caches, qs = [], []
    for layer in range(NL):
        c = nsnq.KVCache(p, B, Hkv, nq + R, dev)
        if layer < distinct_layers:
            k, v = synth.kv_layer(w["config_id"], layer, B, Hkv, L, d,
                                  outlier_std=synth.outlier_std_for(workload, layer), device=dev)
            nsnq.nsnq_encode_kv(p, cb, k, v, L, c)
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
    ws = torch.empty(nsnq.nsnq_decode_workspace_bytes(p, caches[0], Hq), dtype=torch.uint8, device=dev)
    outs = [torch.empty_like(q) for q in qs]
    stream = torch.cuda.current_stream()

    def step():
        for layer in range(NL):
            nsnq.nsnq_decode_attention(p, cb, qs[layer], caches[layer], out=outs[layer], ws=ws, stream=stream)

    def timed(f, n):
        for _ in range(2):
            f()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(n):
            f()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n / 1e3

    t_c = timed(step, steps)
    cache_bytes = sum(c.nbytes() for c in caches)
    dec_b = NL * decode_bytes(bits, R, nq, r, B * Hkv, d)
    del caches
    torch.cuda.empty_cache()
    res = {"metric": "decode-attn tokens/s", "workload": workload, "layers": NL, "batch": B, "context": L,
           "bits": bits, "step_ms": t_c * 1e3, "tokens_per_s": B / t_c,
           "hbm_gbs": dec_b / t_c / 1e9, "hbm_frac": dec_b / t_c / 1e9 / HBM_PEAK_GBS,
           "compressed_cache_gb": cache_bytes / 1e9,
           "setup": f"{distinct_layers} distinct layers encoded, caches copied to the other {NL - distinct_layers}"}
    if not with_fp16:
        return res
    # fp16 comparator: largest batch whose fp16 K/V for all layers fits the budget
    free, total = torch.cuda.mem_get_info()
    budget = free - 8e9
    per_seq = NL * 2 * Hkv * L * d * 2
    B16 = int(max(1, min(B, budget // per_seq)))
    kf = [torch.randn(B16, Hkv, L, d, device=dev, dtype=torch.float16) for _ in range(2)]
    vf = [torch.randn(B16, Hkv, L, d, device=dev, dtype=torch.float16) for _ in range(2)]
    q16 = qs[0][:B16].contiguous()
    ws16 = torch.empty(nsnq.nsnq_fp16_decode_workspace_bytes(B16, Hq, L), dtype=torch.uint8, device=dev)
    o16 = torch.empty_like(q16)

    def step16():
        for layer in range(NL):
            nsnq.nsnq_fp16_decode_attention(q16, kf[layer % 2], vf[layer % 2], out=o16, ws=ws16, stream=stream)

    t_16 = timed(step16, steps)
    b16 = NL * B16 * Hkv * L * 2 * 2 * d
    res["fp16"] = {"batch": B16, "step_ms": t_16 * 1e3, "tokens_per_s": B16 / t_16,
                   "hbm_gbs": b16 / t_16 / 1e9, "cache_gb": per_seq * B16 / 1e9, "budget_gb": budget / 1e9}
    res["gain_tokens_per_s"] = (B / t_c) / (B16 / t_16)
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


ENCODE_SOURCES = ("encode.hip", "nsnq_device.hpp", "nsnq_launch.hpp")  # what the encode kernel compiles from


def sources_sha256(names) -> str:
    """sha256 over the named files of the kernel source folder, in order."""
    import hashlib
    h = hashlib.sha256()
    for n in names:
        h.update(open(os.path.join(ROOT, "kv_cache_bit_amd", "csrc", n), "rb").read())
    return h.hexdigest()


def encode_traffic():
    """HBM bytes per encode launch from the committed rocprofv3 counter
    summary, or None when the kernel's sources have changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "encode_kernel_llama2-7b-layer-b1-2bit_traffic.json")
    try:
        rec = json.load(open(path))
        sha = sources_sha256(ENCODE_SOURCES)
    except (OSError, ValueError):
        return None
    if rec.get("sources") != list(ENCODE_SOURCES) or rec.get("sources_sha256") != sha:
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(w: dict, cb_bits, k, v, q, heads: int):
    """Time the CPU oracle on `heads` of the layer's KV heads (encode of those
    heads' K and V, then their decode step); scale to the whole layer."""
    import numpy as np
    import oracle
    from kv_cache_bit_amd import nsnq
    R = w["R"]
    G = w["Hq"] // w["Hkv"]
    kk = k[:, :heads].cpu().contiguous()
    vv = v[:, :heads].cpu().contiguous()
    qq = q[:, :heads * G].cpu().contiguous()
    t0 = time.perf_counter()
    ek, ev = oracle.encode(kk, R, cb_bits), oracle.encode(vv, R, cb_bits)
    t1 = time.perf_counter()
    oracle.reference_decode(qq, ek, ev, ek["n_quant"], ek["n_resid"], R, cb_bits)
    t2 = time.perf_counter()
    scale = w["Hkv"] / heads
    step = (t2 - t0) * scale
    cores = oracle.num_threads()
    # the same work on one thread, for one KV head
    oracle.set_num_threads(1)
    try:
        t3 = time.perf_counter()
        e1k, e1v = oracle.encode(kk[:, :1].contiguous(), R, cb_bits), oracle.encode(vv[:, :1].contiguous(), R, cb_bits)
        oracle.reference_decode(qq[:, :G].contiguous(), e1k, e1v, e1k["n_quant"], e1k["n_resid"], R, cb_bits)
        step1 = (time.perf_counter() - t3) * w["Hkv"]
    finally:
        oracle.set_num_threads(cores)
    return dict(step_s=step, encode_s=(t1 - t0) * scale, decode_s=(t2 - t1) * scale, cores=cores,
                sample=f"{heads} of {w['Hkv']} KV heads x batch {w['B']}, full context; time scaled x{scale:g}",
                step_1t_s=step1, sample_1t=f"1 of {w['Hkv']} KV heads on one thread; time scaled x{w['Hkv']}")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama2-7b-layer-b1-2bit")
    ap.add_argument("--cpu-heads", type=int, default=4, help="KV heads in the CPU-baseline sample (0: skip)")
    ap.add_argument("--codebook-iters", type=int, default=50)
    ap.add_argument("--no-fp16", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the 1-bit layer measurement")
    ap.add_argument("--copy-bytes", type=int, default=0, help="only run a device copy of this size")
    ap.add_argument("--decode-layers", type=int, default=0,
                    help="multi-layer workloads: time the decode of only this many layers (profiling)")
    args = ap.parse_args()
    if args.copy_bytes:
        copy_calibration(args.copy_bytes, max(args.steps, 1))
        return
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(this path has no multi-GPU code).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from kv_cache_bit_amd import nsnq, synth

    nsnq.lib()  # fail loudly if the HIP library is missing
    assert torch.cuda.is_available(), "bench needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = dict(synth.WORKLOADS[args.workload])
    if w["layers"] > 1:
        print(json.dumps(decode_step_bench(nsnq, synth, args.workload, max(args.steps // 5, 3), dev,
                                           max_layers=args.decode_layers, with_fp16=not args.no_fp16)), flush=True)
        return
    B, Hq, Hkv, L, d, bits, R = w["B"], w["Hq"], w["Hkv"], w["L"], w["d"], w["bits"], w["R"]
    s = nsnq.sub_dim(bits)
    p = nsnq.params(bits, R)

    # ---- setup (untimed) ----------------------------------------------------
    t_cb = time.perf_counter()
    samples = synth.randn_samples(0, 1 << 20, s).to(dev)
    _, codebook, dist = nsnq.nsnq_build_codebook(p, samples, args.codebook_iters)
    torch.cuda.synchronize()
    t_cb = time.perf_counter() - t_cb
    # 2 bits: the encoder searches each sub-vector's orthant candidate list
    # (same codes as the exhaustive search); the table is built once per codebook
    t_tab = time.perf_counter()
    p_enc = nsnq.with_candidates(p, codebook) if bits == 2 else p
    t_tab = time.perf_counter() - t_tab
    search_cols = p_enc.vq_span if p_enc.vq_span else 256  # codewords compared per sub-vector
    k, v = synth.kv_layer(w["config_id"], 0, B, Hkv, L, d, outlier_std=synth.outlier_std_for(args.workload, 0),
                          device=dev)
    q = synth.queries(w["config_id"], 0, B, Hq, d, device=dev)
    set_bytes = 2 * k.numel() * 2
    nbuf = max(1, min(8, math.ceil(512e6 / set_bytes)))
    ks = [k] + [k.clone() for _ in range(nbuf - 1)]
    vs = [v] + [v.clone() for _ in range(nbuf - 1)]
    r = ((L - 1) % R) + 1
    nq = L - r
    caches = [nsnq.KVCache(p, B, Hkv, nq + R, dev) for _ in range(nbuf)]
    outs = [torch.empty_like(q) for _ in range(nbuf)]
    # workspace sized for a filled cache
    caches[0].n_quant, caches[0].n_resid = nq, r
    ws_bytes = nsnq.nsnq_decode_workspace_bytes(p, caches[0], Hq)
    caches[0].n_quant = caches[0].n_resid = 0
    wss = [torch.empty(ws_bytes, dtype=torch.uint8, device=dev) for _ in range(nbuf)]
    stream = torch.cuda.current_stream()

    def step(i, ev=None):
        c = caches[i % nbuf]
        c.n_quant = c.n_resid = 0
        if ev is not None:
            ev[0].record(stream)
        nsnq.nsnq_encode_kv(p_enc, codebook, ks[i % nbuf], vs[i % nbuf], L, c, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        nsnq.nsnq_decode_attention(p, codebook, q, c, out=outs[i % nbuf], ws=wss[i % nbuf], stream=stream)
        if ev is not None:
            ev[2].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # per-phase HIP events on every 8th timed step (events between the phases
    # cost ~10 us of wall time per step they bracket)
    every = 8
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(0, args.steps, every)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, evs[i // every] if i % every == 0 else None)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    enc_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    dec_ms = np.array([e[1].elapsed_time(e[2]) for e in evs])
    step_ms = np.array([e[0].elapsed_time(e[2]) for e in evs])
    ms_per_step = wall * 1e3 / args.steps

    units = B * Hkv
    n_vec = 2 * units * nq
    enc_bytes = n_vec * encode_bytes_per_vector(bits, R, d) + 2 * units * r * 2 * d * 2  # + residual copy
    dec_bytes = decode_bytes(bits, R, nq, r, units, d)
    enc_s = float(np.mean(enc_ms)) / 1e3
    dec_s = float(np.mean(dec_ms)) / 1e3
    cand = n_vec * (d // s) * 256  # algorithmic argmin candidates per launch (nearest of 256 codewords)
    cand_run = n_vec * (d // s) * search_cols  # distances the search actually compares
    enc_gbs = enc_bytes / enc_s / 1e9
    dec_gbs = dec_bytes / dec_s / 1e9
    enc_alu_tops = cand / enc_s / 1e12

    # the exhaustive search on the same inputs, for comparison
    enc_full_s = None
    if p_enc is not p:
        c = caches[0]
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        nfull = 20
        for j in range(nfull + 3):
            if j == 3:
                e0.record(stream)
            c.n_quant = c.n_resid = 0
            nsnq.nsnq_encode_kv(p, codebook, ks[j % nbuf], vs[j % nbuf], L, c, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        enc_full_s = e0.elapsed_time(e1) / nfull / 1e3

    # fp16 comparator on the same layer
    fp16 = None
    if not args.no_fp16:
        kf, vf = k[:, :, :L].contiguous(), v[:, :, :L].contiguous()
        o16 = nsnq.nsnq_fp16_decode_attention(q, kf, vf)
        for _ in range(5):
            nsnq.nsnq_fp16_decode_attention(q, kf, vf, out=o16)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n16 = 50
        e0.record(stream)
        for _ in range(n16):
            nsnq.nsnq_fp16_decode_attention(q, kf, vf, out=o16)
        e1.record(stream)
        torch.cuda.synchronize()
        t16 = e0.elapsed_time(e1) / n16 / 1e3
        b16 = units * L * 2 * 2 * d
        fp16 = dict(us=t16 * 1e6, tokens_per_s=B / t16, gbs=b16 / t16 / 1e9,
                    compressed_speedup=t16 / dec_s, bytes=b16)

    value = B * L / (ms_per_step / 1e3)
    res = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": B, "q_heads": Hq, "kv_heads": Hkv, "context": L,
                   "head_dim": d, "bits": bits, "residual": R, "encoded_tokens": nq, "residual_tokens": r},
        "encode": {"us": enc_s * 1e6, "tokens_per_s": B * L / enc_s, "vectors_per_s": n_vec / enc_s,
                   "hbm_gbs": enc_gbs, "hbm_frac": enc_gbs / HBM_PEAK_GBS,
                   "search": (f"orthant candidate lists, {search_cols} of 256 codewords per sub-vector"
                              if p_enc is not p else "exhaustive, 256 codewords per sub-vector"),
                   "candidate_table_s": t_tab if p_enc is not p else None,
                   "argmin_candidates_per_s": cand / enc_s, "compared_per_s": cand_run / enc_s,
                   "bytes": enc_bytes,
                   "exhaustive_us": None if enc_full_s is None else enc_full_s * 1e6},
        "decode": {"us": dec_s * 1e6, "tokens_per_s": B / dec_s, "kv_tokens_per_s": units * L / dec_s,
                   "hbm_gbs": dec_gbs, "hbm_frac": dec_gbs / HBM_PEAK_GBS, "bytes": dec_bytes},
        "fp16_decode": fp16,
        "codebook": {"build_s": t_cb, "iters": args.codebook_iters, "n": 1 << 20,
                     "final_mse_per_elem": float(dist[-1].item())},
        "roofline": {"kernel": (f"encode_kernel<4, {R}, false, {(search_cols + 31) // 32}, "
                                f"{'true' if search_cols % 32 else 'false'}>" if p_enc is not p
                                else f"encode_kernel<{s}, {R}, false, 0, false>"),
                     "bound": "alu", "achieved": enc_alu_tops,
                     "peak": VALU_PEAK_TOPS, "unit": "Tops/s", "frac": enc_alu_tops / VALU_PEAK_TOPS,
                     "traffic": encode_traffic(),
                     "note": ("achieved = algorithmic argmin candidates per second: the nearest of 256 "
                              "codewords per sub-vector (8192 per vector at 2 bits), one 32-bit compare "
                              "each; the candidate-list search compares " + str(search_cols) +
                              " of them per sub-vector")},
        "timing": {"step_ms_median": float(np.median(step_ms)), "step_ms_p10": float(np.percentile(step_ms, 10)),
                   "step_ms_p90": float(np.percentile(step_ms, 90)), "buffer_sets": nbuf},
    }
    if not args.no_extra:
        res["options"] = measure_options(nsnq, synth, w, k, v, q, codebook, dev)
    if not args.no_extra and args.workload != "llama2-7b-layer-b16-1bit":
        del ks, vs, caches
        torch.cuda.empty_cache()
        res["one_bit"] = measure_layer(nsnq, synth, "llama2-7b-layer-b16-1bit", 10, dev)
    if args.cpu_heads > 0:
        cb_bits = codebook.cpu().numpy().view(np.uint16)
        cb_ = cpu_baseline(w, cb_bits, k, v, q, min(args.cpu_heads, Hkv))
        res["cpu_baseline"] = {"value": B * L / cb_["step_s"], "unit": "tokens/s", "cores": cb_["cores"],
                               "kind": "oracle", "sample": cb_["sample"],
                               "encode_s": cb_["encode_s"], "decode_s": cb_["decode_s"],
                               "single_thread": {"value": B * L / cb_["step_1t_s"], "unit": "tokens/s",
                                                 "cores": 1, "sample": cb_["sample_1t"]}}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
