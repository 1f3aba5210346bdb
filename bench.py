"""Benchmark of the KQV KV-cache hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input:
quantize-on-write of K and V for the whole context (kvq_quantize_k/v), an
Infinity-Cache flush (so the decode reads HBM, not the 256 MB last-level
cache), then one decode-attention step over the compressed cache
(kvq_decode_attention: query prep, split scan, merge).  Inputs are resident in
HBM before timing starts.  Per-call durations come from HIP events recorded on
the stream the library launches on.

Prints ONE JSON line.  `value` is decode-attention HBM GB/s (algorithmic bytes
of one decode call / its mean duration); quantize GB/s, KV tokens/s, the
roofline of the dominant kernel and the CPU oracle baseline ride along.
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


def record_bytes(d, kb, vb, kq, vq):
    """Bytes of one (token, KV head) record: codes + sign bits + fp16 norms."""
    return d * kb // 8 + d * vb // 8 + (d // 8) * (kq + vq) + 2 * (2 + kq + vq)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
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

    import numpy as np
    import torch

    from kv_cache_quantization_kqv_amd import synth
    from kv_cache_quantization_kqv_amd.kvq import KVQCache

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    w = synth.WORKLOADS[args.workload]
    scheme = args.scheme or w.scheme
    n_bits = args.bits or w.n_bits
    B, Hq, Hkv, d, N = w.B, w.Hq, w.Hkv, w.d, w.N
    print(f"[bench] workload {w.name} {scheme}{n_bits} B={B} Hq={Hq} Hkv={Hkv} d={d} N={N}",
          file=sys.stderr, flush=True)

    K, V, q = synth.make_kvq(w, device=dev)
    S = synth.bits_u16(synth.sketch_bf16(d, d, 7))
    rot_param = {"wht": None, "rht": synth.rotation_signs(d, 19),
                 "qr": synth.rotation_qr(d, 19)}[args.rotation]
    cache = KVQCache(scheme, n_bits, d, B, Hkv, N, S_bf16=S, device=dev, rotation=args.rotation,
                     rot_signs=rot_param if args.rotation == "rht" else None,
                     rot_Q=rot_param if args.rotation == "qr" else None)
    c = cache.c
    rec = record_bytes(d, c.k_bits, c.v_bits, c.k_qjl, c.v_qjl)
    in_b = 2 if w.dtype == torch.bfloat16 else 4
    q_bytes = B * Hq * d * (in_b + 4)
    dec_bytes = B * Hkv * N * rec + q_bytes
    qk_bytes = B * Hkv * N * (d * in_b + d * c.k_bits // 8 + (d // 8) * c.k_qjl + 2 * (1 + c.k_qjl))
    qv_bytes = B * Hkv * N * (d * in_b + d * c.v_bits // 8 + (d // 8) * c.v_qjl + 2 * (1 + c.v_qjl))

    from kv_cache_quantization_kqv_amd import kvq as _kvq
    splits = _kvq.kvq_decode_auto_splits(c, Hq, N)
    ws = torch.zeros(cache.workspace_bytes(Hq, N), dtype=torch.uint8, device=dev)
    out = torch.empty(B, Hq, d, dtype=torch.float32, device=dev)
    flush = torch.empty(512 * 1024 * 1024 // 4, dtype=torch.float32, device=dev)
    if args.copy_probe_mb:
        n = args.copy_probe_mb * 1024 * 1024 // 4
        a_src = torch.ones(n, dtype=torch.float32, device=dev)
        a_dst = torch.empty_like(a_src)
        a_dst.copy_(a_src)
        torch.cuda.synchronize(dev)
        del a_src, a_dst
    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        cache.quantize_k(K, 0)
        if ev is not None:
            ev[1].record(stream)
        cache.quantize_v(V, 0)
        if ev is not None:
            ev[2].record(stream)
        flush.zero_()
        if ev is not None:
            ev[3].record(stream)
        cache.decode_attention(q, N, out=out, workspace=ws)
        if ev is not None:
            ev[4].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    tk = np.array([e[0].elapsed_time(e[1]) for e in evs]) * 1e-3
    tv = np.array([e[1].elapsed_time(e[2]) for e in evs]) * 1e-3
    td = np.array([e[3].elapsed_time(e[4]) for e in evs]) * 1e-3
    print(f"[bench] timed {args.steps} steps in {wall:.3f}s", file=sys.stderr, flush=True)

    dec_t = float(td.mean())
    dec_gbps = dec_bytes / dec_t / 1e9
    quant_t = float((tk + tv).mean())
    quant_gbps = (qk_bytes + qv_bytes) / quant_t / 1e9

    # warm decode (back-to-back, LLC-resident when the cache fits) for context
    for _ in range(3):
        cache.decode_attention(q, N, out=out, workspace=ws)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(10):
        cache.decode_attention(q, N, out=out, workspace=ws)
    e1.record(stream)
    torch.cuda.synchronize(dev)
    warm_t = e0.elapsed_time(e1) * 1e-3 / 10

    prefill = None
    if args.prefill_chunk > 0:
        C = min(args.prefill_chunk, N)
        qp = synth.gaussian((B, C, Hq, d), 31, w.dtype, device=dev)
        from kv_cache_quantization_kqv_amd import kvq as _kq
        wsp = torch.empty(_kq.kvq_prefill_workspace(c, Hq, C), dtype=torch.uint8, device=dev)
        outp = torch.empty(B, C, Hq, d, dtype=torch.float32, device=dev)
        for _ in range(2):
            cache.prefill_attention(qp, N - C, N, causal=True, out=outp, workspace=wsp)
        reps = max(1, min(args.steps, 5))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize(dev)
        e0.record(stream)
        for _ in range(reps):
            cache.prefill_attention(qp, N - C, N, causal=True, out=outp, workspace=wsp)
        e1.record(stream)
        torch.cuda.synchronize(dev)
        pt = e0.elapsed_time(e1) * 1e-3 / reps
        # MFMA work per (row, visible token): q'.k (d), the K sketch (m, QKQV),
        # P V (d) and the V sketch (m)
        per = 2 * (d + d + d * c.k_qjl + d * c.v_qjl)
        vis = sum(N - C + i + 1 for i in range(C))
        flops = B * Hq * vis * per
        prefill = {"chunk": C, "q_pos0": N - C, "causal": True, "us": round(pt * 1e6, 2),
                   "TFLOPs": round(flops / pt / 1e12, 2), "peak_TFLOPs": FP32_MFMA_PEAK,
                   "pct_fp32_mfma_peak": round(100 * flops / pt / 1e12 / FP32_MFMA_PEAK, 2),
                   "kernel": "prep_kernel + prefill_kernel (fp32 MFMA 16x16x4) + finish_kernel"}
        del qp, wsp, outp

    roof = {"kernel": "kvq_decode_attention: query kernel + decode_kernel (split scan, key scores on fp16 MFMA) + merge_kernel (split merge)",
            "bound": "hbm",
            "achieved": round(dec_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(dec_gbps / HBM_PEAK_GBPS, 4), "traffic": None,
            "bytes_per_launch": dec_bytes, "per_record_bytes": rec}
    if args.traffic and os.path.exists(args.traffic) and args.rotation == "wht":
        roof["traffic"] = read_traffic(args.traffic, scheme, n_bits, w.name)

    result = {
        "metric": METRIC, "value": round(dec_gbps, 1), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "scheme": scheme, "n_bits": n_bits, "batch": B,
                   "q_heads": Hq, "kv_heads": Hkv, "head_dim": d, "context": N,
                   "input_dtype": str(w.dtype).replace("torch.", ""), "keys": w.keys,
                   "splits": splits, "rotation": args.rotation},
        "decode": {"us": round(dec_t * 1e6, 2), "GBps": round(dec_gbps, 1),
                   "pct_hbm_peak": round(100 * dec_gbps / HBM_PEAK_GBPS, 2),
                   "kv_tokens_per_s": round(B * N / dec_t, 1),
                   "records_per_s": round(B * Hkv * N / dec_t, 1),
                   "warm_us": round(warm_t * 1e6, 2),
                   "warm_GBps": round(dec_bytes / warm_t / 1e9, 1)},
        "quantize": {"us_k": round(float(tk.mean()) * 1e6, 2), "us_v": round(float(tv.mean()) * 1e6, 2),
                     "GBps": round(quant_gbps, 1),
                     "pct_hbm_peak": round(100 * quant_gbps / HBM_PEAK_GBPS, 2),
                     "GBps_k": round(qk_bytes / float(tk.mean()) / 1e9, 1),
                     "GBps_v": round(qv_bytes / float(tv.mean()) / 1e9, 1)},
        "roofline": roof,
    }
    if prefill is not None:
        result["prefill"] = prefill

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, scheme, n_bits, K, V, q, S, args.cpu_units, rec,
                                              args.rotation, rot_param)
    print(json.dumps(result), flush=True)


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
    """Measured HBM bytes per decode launch from a profile summary's json block;
    None unless it was taken on this workload and on the current sources."""
    text = open(path).read()
    if "```json" not in text:
        return None
    blk = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
    if blk.get("workload") != workload or blk.get("scheme") != f"{scheme}{n_bits}":
        return None
    if blk.get("source_sha256") != kernel_source_digest():
        return None
    return blk.get("decode_bytes_per_launch")


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
    del np
    return {"value": round(dec_bytes / ta / 1e9, 4), "unit": "GB/s", "cores": cores,
            "kind": "oracle",
            "sample": f"b < {nb}, {hk} of {w.Hkv} KV heads x {G} query heads ({units} units), "
                      f"full context {w.N}: "
                      f"oracle quantize {tq:.2f}s, fp64 decode attention {ta:.2f}s",
            "quantize_GBps": round(q_bytes / tq / 1e9, 4),
            "decode_kv_tokens_per_s": round(w.N * units / w.Hkv / ta, 1)}


def synth_bits(x):
    from kv_cache_quantization_kqv_amd import synth
    return synth.bits_u16(x)


if __name__ == "__main__":
    main()
