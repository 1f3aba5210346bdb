"""Benchmark of the KQV KV-cache hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input:
quantize-on-write of K and V for the whole context (kvq_quantize_k/v), an
Infinity-Cache flush (so the decode reads HBM, not the 256 MB last-level
cache), then one decode-attention step over the compressed cache
(kvq_decode_attention: query prep, split scan, merge).  Inputs are resident in
HBM before timing starts.  Every duration is taken with HIP events recorded on
the stream the library launches on; each reported figure is the median (with
p10 / p90) over `--steps` repetitions (at least 30).

Prints ONE JSON line.  `value` is decode-attention HBM GB/s of the default
workload (algorithmic bytes of one decode call / its median duration).  Along
with it: quantize GB/s, KV tokens/s, the decode stages (prep / scan / merge),
the roofline of the dominant kernel (the scan), the device's streaming-read
ceiling, the other workloads (one-layer cold/warm decode, the nine-run
bit-budget sweep, long-context chunked quantize / one-token append / decode)
and the CPU oracle baseline.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "4-bit KQV decode-attn HBM GB/s (% of peak) + KV tokens/s; quantize GB/s"
HBM_PEAK_GBPS = 8000.0
FP32_MFMA_PEAK = 157.3  # TFLOP/s, dense fp32 matrix (MI355X)
FP16_MFMA_PEAK = 2500.0  # TFLOP/s, dense fp16 matrix (MI355X)


def record_bytes(d, kb, vb, kq, vq):
    """Bytes of one (token, KV head) record: codes + sign bits + fp16 norms."""
    return d * kb // 8 + d * vb // 8 + (d // 8) * (kq + vq) + 2 * (2 + kq + vq)


class Timer:
    """HIP-event timing on the launch stream; cold runs zero a 512 MiB buffer
    first so the measured call reads HBM, not the last-level cache."""

    def __init__(self, torch, dev):
        self.torch, self.dev = torch, dev
        self.stream = torch.cuda.current_stream(dev)
        self.flush = torch.empty(512 * 1024 * 1024 // 4, dtype=torch.float32, device=dev)

    def run(self, fn, reps, cold=True, marks=1):
        """fn(ev) calls ev(k) after its k-th part (k = 1..marks); returns an
        array [reps][marks] of microseconds per part."""
        torch = self.torch
        import numpy as np
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(marks + 1)] for _ in range(reps)]
        for r in range(reps):
            if cold:
                self.flush.zero_()
            e = evs[r]
            e[0].record(self.stream)
            fn(lambda k, e=e: e[k].record(self.stream))
        torch.cuda.synchronize(self.dev)
        return np.array([[e[k].elapsed_time(e[k + 1]) * 1e3 for k in range(marks)] for e in evs])


def stats(us):
    """median / p10 / p90 of a 1-D array of microseconds."""
    import numpy as np
    return {"median": round(float(np.median(us)), 2), "p10": round(float(np.percentile(us, 10)), 2),
            "p90": round(float(np.percentile(us, 90)), 2)}


def build_cache(torch, KVQCache, synth, w, scheme, n_bits, dev, rotation="wht", cap=None):
    S = synth.bits_u16(synth.sketch_bf16(w.d, w.d, 7))
    rot_param = {"wht": None, "rht": synth.rotation_signs(w.d, 19),
                 "qr": synth.rotation_qr(w.d, 19)}[rotation]
    cache = KVQCache(scheme, n_bits, w.d, w.B, w.Hkv, cap or w.N, S_bf16=S, device=dev,
                     rotation=rotation, rot_signs=rot_param if rotation == "rht" else None,
                     rot_Q=rot_param if rotation == "qr" else None)
    return cache, S, rot_param


def quant_bytes(c, T, B, H, d, in_b):
    """Algorithmic bytes of quantizing T tokens of K and of V (inputs read,
    records written)."""
    qk = B * H * T * (d * in_b + d * c.k_bits // 8 + (d // 8) * c.k_qjl + 2 * (1 + c.k_qjl))
    qv = B * H * T * (d * in_b + d * c.v_bits // 8 + (d // 8) * c.v_qjl + 2 * (1 + c.v_qjl))
    return qk, qv


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama_gqa_decode")
    ap.add_argument("--scheme", default=None, help="override the workload's scheme")
    ap.add_argument("--bits", type=int, default=None, help="override n bits/coordinate")
    ap.add_argument("--rotation", default="wht", choices=["wht", "rht", "qr"],
                    help="rotation of the rotated schemes (Walsh-Hadamard, randomized "
                         "Hadamard, dense SO(d))")
    ap.add_argument("--prefill-chunk", type=int, default=256,
                    help="also time multi-query attention of a chunk of this many query tokens "
                         "at the end of the context (causal); 0 skips it")
    ap.add_argument("--no-suite", action="store_true",
                    help="skip the other workloads (one-layer, bit-budget sweep, long context)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-units", type=int, default=32,
                    help="(b, KV head) units in the CPU sample (about 20 s of oracle work "
                         "on 16 host threads)")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "traffic_gqa_decode_kqv4.md"),
                    help="profiles/*.md summary holding measured HBM bytes per launch (json block)")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="run one plain device copy of this many MiB first (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build measures one GPU only; run with --gpus 1"}))
        sys.exit(2)
    reps = max(30, args.steps)

    import numpy as np
    import torch

    from kv_cache_quantization_kqv_amd import synth
    from kv_cache_quantization_kqv_amd import kvq as K_
    from kv_cache_quantization_kqv_amd.kvq import KVQCache

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    T_ = Timer(torch, dev)
    w = synth.WORKLOADS[args.workload]
    scheme = args.scheme or w.scheme
    n_bits = args.bits or w.n_bits
    B, Hq, Hkv, d, N = w.B, w.Hq, w.Hkv, w.d, w.N
    log = lambda m: print(f"[bench] {m}", file=sys.stderr, flush=True)
    log(f"workload {w.name} {scheme}{n_bits} B={B} Hq={Hq} Hkv={Hkv} d={d} N={N}")

    K, V, q = synth.make_kvq(w, device=dev)
    cache, S, rot_param = build_cache(torch, KVQCache, synth, w, scheme, n_bits, dev, args.rotation)
    c = cache.c
    rec = record_bytes(d, c.k_bits, c.v_bits, c.k_qjl, c.v_qjl)
    in_b = 2 if w.dtype == torch.bfloat16 else 4
    q_bytes = B * Hq * d * (in_b + 4)
    dec_bytes = B * Hkv * N * rec + q_bytes
    qk_bytes, qv_bytes = quant_bytes(c, N, B, Hkv, d, in_b)
    splits = K_.kvq_decode_auto_splits(c, Hq, N)
    ws = torch.zeros(cache.workspace_bytes(Hq, N), dtype=torch.uint8, device=dev)
    out = torch.empty(B, Hq, d, dtype=torch.float32, device=dev)
    if args.copy_probe_mb:
        n = args.copy_probe_mb * 1024 * 1024 // 4
        a_src = torch.ones(n, dtype=torch.float32, device=dev)
        a_dst = torch.empty_like(a_src)
        a_dst.copy_(a_src)
        torch.cuda.synchronize(dev)
        del a_src, a_dst

    def step(ev):
        cache.quantize_k(K, 0)
        ev(1)
        cache.quantize_v(V, 0)
        ev(2)
        T_.flush.zero_()
        ev(3)
        cache.decode_attention(q, N, out=out, workspace=ws)
        ev(4)

    for _ in range(args.warmup):
        step(lambda k: None)
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    tm = T_.run(step, args.steps, cold=False, marks=4)
    wall = time.perf_counter() - t0
    log(f"timed {args.steps} steps in {wall:.3f}s")

    # per-call statistics over `reps` repetitions (decode cold: LLC flushed first)
    tq = T_.run(lambda ev: (cache.quantize_k(K, 0), ev(1), cache.quantize_v(V, 0), ev(2)),
                reps, cold=True, marks=2)
    td = T_.run(lambda ev: (cache.decode_attention(q, N, out=out, workspace=ws), ev(1)),
                reps, cold=True)[:, 0]
    st = T_.run(lambda ev: (cache.decode_attention(q, N, out=out, workspace=ws, stages=K_.KVQ_STAGE_PREP), ev(1),
                            cache.decode_attention(q, N, out=out, workspace=ws, stages=K_.KVQ_STAGE_SCAN), ev(2),
                            cache.decode_attention(q, N, out=out, workspace=ws, stages=K_.KVQ_STAGE_MERGE), ev(3)),
                reps, cold=True, marks=3)
    tw = T_.run(lambda ev: (cache.decode_attention(q, N, out=out, workspace=ws), ev(1)),
                reps, cold=False)[:, 0]
    dec_t = float(np.median(td)) * 1e-6
    dec_gbps = dec_bytes / dec_t / 1e9
    tk, tv = tq[:, 0], tq[:, 1]
    quant_t = float(np.median(tk + tv)) * 1e-6
    quant_gbps = (qk_bytes + qv_bytes) / quant_t / 1e9

    # the scan kernel alone: cache records + queries read, split partials written;
    # at d = 128 with a Hadamard rotation (or none) and no key sketch the scan
    # prepares q' from q itself (no prep launch), else it reads q' (and S q') in fp32
    prep_fused = d == 128 and not c.k_qjl and args.rotation != "qr"
    q_bytes = B * Hq * d * (q.element_size() if prep_fused else 4 * (1 + c.k_qjl))
    scan_bytes = B * Hkv * N * rec + q_bytes + B * Hq * splits * (2 + 2 * d) * 4
    scan_t = float(np.median(st[:, 1])) * 1e-6
    roof = {"kernel": "scan_kernel (kvq_decode_attention_stages KVQ_STAGE_SCAN: split scan on fp16 MFMA"
                      + (", query prepared in its prologue)" if prep_fused else ")"),
            "bound": "hbm",
            "achieved": round(scan_bytes / scan_t / 1e9, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(scan_bytes / scan_t / 1e9 / HBM_PEAK_GBPS, 4), "traffic": None,
            "bytes_per_launch": scan_bytes, "launch_us": round(scan_t * 1e6, 2),
            "per_record_bytes": rec}
    if args.traffic and os.path.exists(args.traffic) and args.rotation == "wht":
        roof["traffic"] = read_traffic(args.traffic, scheme, n_bits, w.name)

    # the device's streaming-read ceiling (simplest access pattern, 1 GiB)
    probe = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
    pw = torch.zeros(4, dtype=torch.int32, device=dev)
    sr = T_.run(lambda ev: (K_.kvq_probe_stream_read(probe.data_ptr(), probe.numel(), pw.data_ptr(),
                                                      T_.stream.cuda_stream), ev(1)),
                reps, cold=True)[:, 0]
    stream_gbps = probe.numel() / float(np.median(sr)) / 1e3
    del probe

    prefill = None
    if args.prefill_chunk > 0:
        C = min(args.prefill_chunk, N)
        qp = synth.gaussian((B, C, Hq, d), 31, w.dtype, device=dev)
        wsp = torch.empty(K_.kvq_prefill_workspace(c, Hq, C), dtype=torch.uint8, device=dev)
        outp = torch.empty(B, C, Hq, d, dtype=torch.float32, device=dev)
        cache.prefill_attention(qp, N - C, N, causal=True, out=outp, workspace=wsp)
        tp = T_.run(lambda ev: (cache.prefill_attention(qp, N - C, N, causal=True, out=outp, workspace=wsp),
                                ev(1)), 3, cold=False)[:, 0]
        pt = float(np.median(tp)) * 1e-6
        # MFMA work per (row, visible token): q'.k (d), the K sketch (m, QKQV),
        # P V (d) and the V sketch (m)
        per = 2 * (d + d + d * c.k_qjl + d * c.v_qjl)
        vis = sum(N - C + i + 1 for i in range(C))
        flops = B * Hq * vis * per
        tf = flops / pt / 1e12
        if d == 128:
            # fp16 matrix cores; every fp32 operand is split into two fp16 parts,
            # so one algorithmic product costs two MFMA products
            prefill = {"chunk": C, "q_pos0": N - C, "causal": True, "us": round(pt * 1e6, 2),
                       "TFLOPs": round(tf, 2), "peak_TFLOPs": FP16_MFMA_PEAK,
                       "pct_fp16_mfma_peak": round(100 * tf / FP16_MFMA_PEAK, 2),
                       "pct_split_operand_peak": round(100 * tf / (FP16_MFMA_PEAK / 2), 2),
                       "x_fp32_mfma_peak": round(tf / FP32_MFMA_PEAK, 3),
                       "kernel": "prep_kernel + prefill16_kernel (fp16 MFMA 16x16x32, split operands) + finish_kernel"}
        else:
            prefill = {"chunk": C, "q_pos0": N - C, "causal": True, "us": round(pt * 1e6, 2),
                       "TFLOPs": round(tf, 2), "peak_TFLOPs": FP32_MFMA_PEAK,
                       "pct_fp32_mfma_peak": round(100 * tf / FP32_MFMA_PEAK, 2),
                       "kernel": "prep_kernel + prefill_kernel (fp32 MFMA 16x16x4) + finish_kernel"}
        del qp, wsp, outp

    result = {
        "metric": METRIC, "value": round(dec_gbps, 1), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "scheme": scheme, "n_bits": n_bits, "batch": B,
                   "q_heads": Hq, "kv_heads": Hkv, "head_dim": d, "context": N,
                   "input_dtype": str(w.dtype).replace("torch.", ""), "keys": w.keys,
                   "splits": splits, "rotation": args.rotation, "reps": reps},
        "decode": {"us": stats(td), "GBps": round(dec_gbps, 1),
                   "pct_hbm_peak": round(100 * dec_gbps / HBM_PEAK_GBPS, 2),
                   "kv_tokens_per_s": round(B * N / dec_t, 1),
                   "records_per_s": round(B * Hkv * N / dec_t, 1),
                   "stages_us": {"prep": "in scan prologue" if prep_fused else stats(st[:, 0]),
                                 "scan": stats(st[:, 1]), "merge": stats(st[:, 2])},
                   "warm_us": stats(tw),
                   "warm_GBps": round(dec_bytes / float(np.median(tw)) / 1e3, 1)},
        "quantize": {"us_k": stats(tk), "us_v": stats(tv),
                     "GBps": round(quant_gbps, 1),
                     "pct_hbm_peak": round(100 * quant_gbps / HBM_PEAK_GBPS, 2),
                     "GBps_k": round(qk_bytes / float(np.median(tk)) / 1e3, 1),
                     "GBps_v": round(qv_bytes / float(np.median(tv)) / 1e3, 1)},
        "roofline": roof,
        "stream_read_GBps": round(stream_gbps, 1),
    }
    if prefill is not None:
        result["prefill"] = prefill
    del K, V, cache, ws
    torch.cuda.empty_cache()

    if not args.no_suite:
        result["workloads"] = suite(torch, np, synth, K_, KVQCache, T_, dev, reps, log)

    if not args.no_cpu_baseline:
        Kc, Vc, qc = synth.make_kvq(w, device=dev)
        result["cpu_baseline"] = cpu_baseline(w, scheme, n_bits, Kc, Vc, qc, S, args.cpu_units, rec,
                                              args.rotation, rot_param)
    print(json.dumps(result), flush=True)


def decode_cold_warm(torch, np, T_, cache, q, n_ctx, reps, ws, out, nbytes):
    td = T_.run(lambda ev: (cache.decode_attention(q, n_ctx, out=out, workspace=ws), ev(1)),
                reps, cold=True)[:, 0]
    tw = T_.run(lambda ev: (cache.decode_attention(q, n_ctx, out=out, workspace=ws), ev(1)),
                reps, cold=False)[:, 0]
    return {"cold_us": stats(td), "cold_GBps": round(nbytes / float(np.median(td)) / 1e3, 1),
            "warm_us": stats(tw), "warm_GBps": round(nbytes / float(np.median(tw)) / 1e3, 1)}


def suite(torch, np, synth, K_, KVQCache, T_, dev, reps, log):
    """The other workloads, each on its own shapes."""
    res = {}
    # one layer, batch 1, 32 heads, N = 4096: quantize all tokens + one decode step
    w = synth.WORKLOADS["one_layer_decode"]
    log(f"suite: {w.name}")
    K, V, q = synth.make_kvq(w, device=dev)
    cache, _, _ = build_cache(torch, KVQCache, synth, w, w.scheme, w.n_bits, dev)
    c = cache.c
    rec = record_bytes(w.d, c.k_bits, c.v_bits, c.k_qjl, c.v_qjl)
    in_b = 2 if w.dtype == torch.bfloat16 else 4
    qk, qv = quant_bytes(c, w.N, w.B, w.Hkv, w.d, in_b)
    tq = T_.run(lambda ev: (cache.quantize_k(K, 0), cache.quantize_v(V, 0), ev(1)), reps, cold=True)[:, 0]
    ws = torch.zeros(cache.workspace_bytes(w.Hq, w.N), dtype=torch.uint8, device=dev)
    out = torch.empty(w.B, w.Hq, w.d, dtype=torch.float32, device=dev)
    nbytes = w.B * w.Hkv * w.N * rec + w.B * w.Hq * w.d * (in_b + 4)
    res[w.name] = {"quantize_us": stats(tq), "quantize_GBps": round((qk + qv) / float(np.median(tq)) / 1e3, 1),
                   "decode": decode_cold_warm(torch, np, T_, cache, q, w.N, reps, ws, out, nbytes),
                   "decode_bytes": nbytes}
    del K, V, q, cache, ws, out

    # bit-budget sweep: KV, KQV, QKQV at n = 2, 3, 4 over the same inputs
    w = synth.WORKLOADS["bit_budget_sweep"]
    log(f"suite: {w.name}")
    K, V, q = synth.make_kvq(w, device=dev)
    in_b = 2 if w.dtype == torch.bfloat16 else 4
    runs = []
    for scheme in ("KV", "KQV", "QKQV"):
        for n in (2, 3, 4):
            cache, _, _ = build_cache(torch, KVQCache, synth, w, scheme, n, dev)
            c = cache.c
            rec = record_bytes(w.d, c.k_bits, c.v_bits, c.k_qjl, c.v_qjl)
            qk, qv = quant_bytes(c, w.N, w.B, w.Hkv, w.d, in_b)
            tq = T_.run(lambda ev: (cache.quantize_k(K, 0), cache.quantize_v(V, 0), ev(1)), reps,
                        cold=True)[:, 0]
            ws = torch.zeros(cache.workspace_bytes(w.Hq, w.N), dtype=torch.uint8, device=dev)
            out = torch.empty(w.B, w.Hq, w.d, dtype=torch.float32, device=dev)
            nbytes = w.B * w.Hkv * w.N * rec + w.B * w.Hq * w.d * (in_b + 4)
            runs.append({"scheme": scheme, "n_bits": n, "record_bytes": rec,
                         "quantize_GBps": round((qk + qv) / float(np.median(tq)) / 1e3, 1),
                         **decode_cold_warm(torch, np, T_, cache, q, w.N, reps, ws, out, nbytes)})
            del cache, ws, out
    res[w.name] = runs
    del K, V, q

    # long context: 8192-token prefill chunks, then 64 decode steps that each
    # append one token and decode over the grown context
    w = synth.WORKLOADS["long_context"]
    log(f"suite: {w.name}")
    steps = 64
    K, V, q = synth.make_kvq(w, device=dev, N=w.N + steps)
    cap = (w.N + steps + 15) // 16 * 16
    cache, _, _ = build_cache(torch, KVQCache, synth, w, w.scheme, w.n_bits, dev, cap=cap)
    c = cache.c
    rec = record_bytes(w.d, c.k_bits, c.v_bits, c.k_qjl, c.v_qjl)
    in_b = 2 if w.dtype == torch.bfloat16 else 4
    CH = 8192
    qk, qv = quant_bytes(c, CH, w.B, w.Hkv, w.d, in_b)

    def chunks(ev):
        for i in range(w.N // CH):
            cache.quantize_k(K[:, :, i * CH:(i + 1) * CH], i * CH)
            cache.quantize_v(V[:, :, i * CH:(i + 1) * CH], i * CH)
            ev(i + 1)
    tc = T_.run(chunks, 3, cold=True, marks=w.N // CH).reshape(-1)
    ws = torch.zeros(cache.workspace_bytes(w.Hq, w.N + steps), dtype=torch.uint8, device=dev)
    out = torch.empty(w.B, w.Hq, w.d, dtype=torch.float32, device=dev)
    nbytes = w.B * w.Hkv * w.N * rec + w.B * w.Hq * w.d * (in_b + 4)
    dec = decode_cold_warm(torch, np, T_, cache, q, w.N, reps, ws, out, nbytes)

    def decode_steps(ev):
        for s in range(steps):
            p = w.N + s
            cache.quantize_k(K[:, :, p:p + 1], p)
            cache.quantize_v(V[:, :, p:p + 1], p)
            ev(2 * s + 1)
            cache.decode_attention(q, p + 1, out=out, workspace=ws)
            ev(2 * s + 2)
    ts = T_.run(decode_steps, 1, cold=False, marks=2 * steps)[0]

    # the last step (append + decode) captured as a HIP graph and replayed back
    # to back: the step's device time without the host's per-call issue
    p = w.N + steps - 1
    kt, vt = K[:, :, p:p + 1].contiguous(), V[:, :, p:p + 1].contiguous()

    def one_step():
        cache.quantize_k(kt, p)
        cache.quantize_v(vt, p)
        cache.decode_attention(q, p + 1, out=out, workspace=ws)
    one_step()
    torch.cuda.synchronize(dev)
    try:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            one_step()
        tg = stats(T_.run(lambda ev: (graph.replay(), ev(1)), reps, cold=False)[:, 0])
        del graph
    except RuntimeError as e:                  # capture unsupported here: report, go on
        log(f"graph capture failed: {e}")
        tg = None
    res[w.name] = {"chunk_tokens": CH,
                   "chunk_quantize_us": stats(tc),
                   "chunk_quantize_GBps": round((qk + qv) / float(np.median(tc)) / 1e3, 1),
                   "decode_131k": dec, "decode_bytes": nbytes,
                   "step_append_us": stats(ts[0::2]), "step_decode_us": stats(ts[1::2]),
                   "step_graph_us": tg}
    del K, V, q, cache, ws, out
    torch.cuda.empty_cache()
    return res


def kernel_source_digest():
    """sha256 over the device and host sources of libkvq (counter summaries are
    only valid for the code they were taken on)."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "kv_cache_quantization_kqv_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def read_traffic(path, scheme, n_bits, workload):
    """Measured HBM bytes per scan launch from a profile summary's json block;
    None unless it was taken on this workload and on the current sources."""
    text = open(path).read()
    if "```json" not in text:
        return None
    blk = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
    if blk.get("workload") != workload or blk.get("scheme") != f"{scheme}{n_bits}":
        return None
    if blk.get("source_sha256") != kernel_source_digest():
        return None
    return blk.get("scan_bytes_per_launch")


def cpu_baseline(w, scheme, n_bits, K, V, q, S, units, rec, rotation="wht", rot_param=None):
    """The CPU oracle as it stands, on a bounded sample of the same workload:
    `units` (b=0, KV head h) units, full context, all their query heads."""
    import numpy as np
    import torch

    from oracle import ref

    cores = len(os.sched_getaffinity(0))
    units = max(1, min(units, w.B * w.Hkv))
    G = w.Hq // w.Hkv
    # the first `units` (b, KV head) units in batch-major order, as whole batch
    # rows of KV heads (nb rows x hk heads)
    hk = min(units, w.Hkv)
    nb = max(1, units // hk)
    units = nb * hk
    Ks = K[0:nb, :hk].detach().cpu()
    Vs = V[0:nb, :hk].detach().cpu()
    qs = q[0:nb, : hk * G].detach().cpu()

    def host(x):
        return synth_bits(x) if x.dtype == torch.bfloat16 else x.numpy()

    ks, vs = ref.scheme_sides(scheme, n_bits)
    rot = ref.Rot(rotation, rot_param)
    ok = ref.OracleCache(nb, hk, w.N, w.d, ks, w.d, rot)
    ov = ref.OracleCache(nb, hk, w.N, w.d, vs, w.d, rot, values=True)
    t0 = time.perf_counter()
    ok.quantize(host(Ks), 0, S, cores)
    ov.quantize(host(Vs), 0, S, cores)
    tq = time.perf_counter() - t0
    t0 = time.perf_counter()
    ref.attention(ok, ov, host(qs), w.N, S, nthreads=cores)
    ta = time.perf_counter() - t0
    in_b = 2 if w.dtype == torch.bfloat16 else 4
    dec_bytes = units * w.N * rec + units * G * w.d * (in_b + 4)
    q_bytes = units * w.N * (2 * w.d * in_b + rec)
    # the first unit again on one thread (the per-core rate)
    ok1 = ref.OracleCache(1, 1, w.N, w.d, ks, w.d, rot)
    ov1 = ref.OracleCache(1, 1, w.N, w.d, vs, w.d, rot, values=True)
    t0 = time.perf_counter()
    ok1.quantize(host(Ks[:1, :1]), 0, S, 1)
    ov1.quantize(host(Vs[:1, :1]), 0, S, 1)
    tq1 = time.perf_counter() - t0
    t0 = time.perf_counter()
    ref.attention(ok1, ov1, host(qs[:1, :G]), w.N, S, nthreads=1)
    ta1 = time.perf_counter() - t0
    del np
    return {"value": round(dec_bytes / ta / 1e9, 4), "unit": "GB/s", "cores": cores,
            "kind": "oracle",
            "sample": f"b < {nb}, {hk} of {w.Hkv} KV heads x {G} query heads ({units} units), "
                      f"full context {w.N}: "
                      f"oracle quantize {tq:.2f}s, fp64 decode attention {ta:.2f}s",
            "quantize_GBps": round(q_bytes / tq / 1e9, 4),
            "decode_kv_tokens_per_s": round(w.N * units / w.Hkv / ta, 1),
            "single_thread": {"sample": f"b = 0, KV head 0 x {G} query heads, full context "
                                        f"{w.N}: quantize {tq1:.2f}s, decode {ta1:.2f}s",
                              "decode_GBps": round(dec_bytes / units / ta1 / 1e9, 5),
                              "quantize_GBps": round(q_bytes / units / tq1 / 1e9, 5)}}


def synth_bits(x):
    from kv_cache_quantization_kqv_amd import synth
    return synth.bits_u16(x)


if __name__ == "__main__":
    main()
