#!/usr/bin/env python3
"""Benchmark of certified quantized-KV decode attention on one MI355X.

A step is one certified decode-attention call for one layer (all heads of
the batch): INT8 scoring, selection and bounds, FP16 paging from pinned host
memory, tail / promoted passes, rank check and any fallback.  Steps cycle
through all layers of the workload in order, so each layer-step reads its
own 227 MB of tier 1 (the 256 MB Infinity Cache cannot serve it from a
previous step).  Inputs are synthetic (datagen) and resident before the
timed region starts.

Prints one JSON line.  `value` = KV tokens (batch x context) per second per
layer-step.  `roofline` is measured for the dominant kernel with HIP events
recorded by the library on the stream that kernel runs on.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "certified decode-attn KV tokens/s per layer-step + achieved HBM GB/s @32K/128K"
HBM_PEAK_GBS = 8000.0


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--workload", default="llama_32k",
                    choices=["llama_32k", "needle_128k", "needle_64k", "llama_8k", "stress_32k"])
    ap.add_argument("--layers", type=int, default=0, help="layers to build (0: the workload's)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 1 GiB read+write kernel (counter calibration)")
    return ap.parse_args()


def block_layout(k, v):
    """[B][T][Hkv][d] FP16 bits -> the FP16 block layout of the library."""
    import numpy as np
    B, T, Hkv, d = k.shape
    kb = k.reshape(B, T // 64, 64, Hkv, d // 8, 8).transpose(0, 3, 1, 4, 2, 5)
    vb = v.reshape(B, T // 64, 64, Hkv, d).transpose(0, 3, 1, 2, 4)
    return np.ascontiguousarray(kb), np.ascontiguousarray(vb)


def counters_for(kernel, workload):
    """HBM traffic per dispatch from a committed rocprofv3 --pmc summary, if it
    was taken on the current kernel source (else None)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_counters.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    src = open(os.path.join(ROOT, "certified_quantized_kv_amd", "csrc", "ckv_decode.hip"), "rb").read()
    if rec.get("source_sha1") != hashlib.sha1(src).hexdigest():
        return None
    return rec.get("traffic_bytes_per_dispatch")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this build has no "
              "multi-GPU path: one process per GPU, each on its own shard of (sequence, kv head).",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import certified_quantized_kv_amd as ckv
    import datagen

    cfg = datagen.CONFIGS[args.workload]
    L = args.layers or cfg["L"]
    B, T, Hq, Hkv, d = cfg["B"], cfg["T"], cfg["Hq"], cfg["Hkv"], cfg["d"]
    dev = torch.device("cuda:0")
    log(f"workload {args.workload}: {L} layers, batch {B}, context {T}, {Hq}/{Hkv} heads, d {d}")
    t0 = time.time()
    cache = ckv.Cache(L, B, Hq, Hkv, d, T, device=0)
    fp = cache.footprint()
    log(f"cache created in {time.time() - t0:.1f}s: device {fp['device'] / 2**30:.2f} GiB "
        f"(tier 1 {fp['tier1'] / 2**30:.2f} GiB), pinned host {fp['host'] / 2**30:.2f} GiB")
    qs = []
    n_dense = 0 if args.no_dense else min(L, 4)
    dense_kv = []
    sample = None
    for l in range(L):
        t1 = time.time()
        lay = datagen.make_layer(args.workload, l)
        for n in range(B):
            cache.append_kv(l, n, lay.k[n], lay.v[n])
        qs.append(torch.from_numpy(lay.q.view(np.float16)).to(dev))
        if l < n_dense:
            kb, vb = block_layout(lay.k, lay.v)
            dense_kv.append((torch.from_numpy(kb.view(np.float16)).to(dev),
                             torch.from_numpy(vb.view(np.float16)).to(dev)))
        if l == 0:
            sample = (lay.k[:1].copy(), lay.v[:1].copy(), lay.q[:1].copy(), lay.sm)
        log(f"layer {l} generated and appended in {time.time() - t1:.1f}s")
    sm = cfg["sm"]
    th = ckv.default_thresholds(sm)
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)

    for i in range(args.warmup):
        cache.certified_decode_attention(i % L, qs[i % L], th, out=out)
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done")

    # timed region: K layer-steps, library-side HIP events on the launch streams
    cache.set_profiling(True)
    rungs = np.zeros(5, np.int64)
    kstar = []
    nvp = []
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    reps = []
    for i in range(args.steps):
        l = (args.warmup + i) % L
        _, rep = cache.certified_decode_attention(l, qs[l], th, out=out)
        reps.append(rep)
    torch.cuda.synchronize()
    t_end = time.perf_counter()
    phases, paged = cache.phase_times()
    cache.set_profiling(False)
    for rep in reps:
        for r in range(5):
            rungs[r] += int((rep["rung_max"] == r).sum())
        kstar.append(float(rep["kstar"].mean()))
        nvp.append(float(rep["n_v_promoted"].mean()))
    elapsed = t_end - t_start
    ms_step = 1e3 * elapsed / args.steps
    tokens = B * T
    value = tokens * args.steps / elapsed
    log(f"timed {args.steps} steps: {ms_step:.3f} ms/step, {value:.4g} KV tokens/s")

    # algorithmic bytes (per token per kv head): INT8 K + K meta, INT4 V + V meta, eta
    kbytes = d + 4 * d / 64
    vbytes = d / 2 + 4 * (d / 32) + 4 / 64
    per_step_tier1 = B * T * Hkv * (kbytes + vbytes)
    paged_per_step = paged / args.steps
    hbm_e2e = (per_step_tier1 + paged_per_step) / (elapsed / args.steps) / 1e9

    def avg_ms(name):
        ms, cnt = phases[name]
        return ms / cnt if cnt else 0.0

    score_ms = avg_ms("score")
    tail_ms = avg_ms("tail")
    score_bytes = B * T * Hkv * kbytes
    tail_bytes = B * T * Hkv * vbytes   # upper bound: blocks outside P and VP are read
    cand = {"k_score": (score_ms, score_bytes), "k_tail": (tail_ms, tail_bytes)}
    dom = max(cand, key=lambda k: cand[k][0])
    dms, dbytes = cand[dom]
    achieved = dbytes / (dms * 1e-3) / 1e9 if dms > 0 else 0.0
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": counters_for(dom, args.workload),
                "avg_launch_ms": round(dms, 5), "algorithmic_bytes_per_launch": int(dbytes)}
    other = "k_tail" if dom == "k_score" else "k_score"
    oms, obytes = cand[other]
    roofline_other = {"kernel": other, "avg_launch_ms": round(oms, 5),
                      "achieved": round(obytes / (oms * 1e-3) / 1e9, 1) if oms > 0 else None}

    # fast dense comparator on device-resident FP16 (same shapes)
    dense = None
    if n_dense:
        for i in range(2 * n_dense):
            kb, vb = dense_kv[i % n_dense]
            cache.dense_decode_attention(kb, vb, T, qs[i % n_dense], sm, out=out)
        torch.cuda.synchronize()
        reps_d = 8 * n_dense
        t1 = time.perf_counter()
        for i in range(reps_d):
            kb, vb = dense_kv[i % n_dense]
            cache.dense_decode_attention(kb, vb, T, qs[i % n_dense], sm, out=out)
        torch.cuda.synchronize()
        dms_step = 1e3 * (time.perf_counter() - t1) / reps_d
        dense = {"ms_per_step": round(dms_step, 4),
                 "hbm_GBps": round(B * T * Hkv * 4 * d / (dms_step * 1e-3) / 1e9, 1),
                 "certified_over_dense": round(ms_step / dms_step, 3),
                 "layers_cycled": n_dense}
        log(f"dense comparator: {dms_step:.3f} ms/step")

    copy_probe = None
    if args.copy_probe:
        a = torch.empty(2 ** 28, dtype=torch.float32, device=dev).fill_(1.0)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(3):
            torch.mul(a, 1.0, out=b)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for _ in range(10):
            torch.mul(a, 1.0, out=b)
        torch.cuda.synchronize()
        cms = 1e3 * (time.perf_counter() - t1) / 10
        copy_probe = {"bytes_read": 2 ** 30, "bytes_written": 2 ** 30, "ms": round(cms, 4),
                      "GBps": round(2 * 2 ** 30 / (cms * 1e-3) / 1e9, 1)}

    cpu = None
    if not args.no_cpu_baseline and sample is not None:
        import oracle
        k1, v1, q1, sm1 = sample
        Tc = min(T, 32768)
        t1 = time.perf_counter()
        oracle.certified_decode(k1[:, :Tc], v1[:, :Tc], q1, oracle.default_thresholds(sm1),
                                trace=False)
        cs = time.perf_counter() - t1
        cpu = {"value": round(Tc / cs, 1), "unit": "KV tokens/s", "cores": 1, "kind": "oracle",
               "sample": f"layer 0, sequence 0, first {Tc} tokens, all {Hq} q heads "
                         f"(one layer-step of one sequence): {cs:.1f} s"}
        log(f"cpu baseline: {cs:.1f}s for the sample")

    rec = {
        "metric": METRIC, "value": round(value, 1), "unit": "KV tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": B, "context": T, "layers": L,
                   "q_heads": Hq, "kv_heads": Hkv, "head_dim": d, "tau_cov": th["tau_cov"],
                   "k_tol": th["k_tol"], "v_tol": th["v_tol"], "rank_tol": th["rank_tol"]},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "hbm_GBps_end_to_end": round(hbm_e2e, 1),
        "paged_MiB_per_step": round(paged_per_step / 2 ** 20, 3),
        "phases_ms_per_step": {k: round(v[0] / max(args.steps, 1), 4) for k, v in phases.items()
                               if k != "copies"},
        "h2d_copies_per_step": round(phases["copies"][1] / max(args.steps, 1), 1),
        "other_kernel": roofline_other,
        "rungs_max_hist": rungs.tolist(),
        "kstar_mean": round(float(np.mean(kstar)), 2),
        "v_promoted_mean": round(float(np.mean(nvp)), 2),
        "dense_comparator": dense,
        "copy_probe": copy_probe,
        "footprint": {"tier1_bytes_per_token_per_kv_head": round(kbytes + vbytes, 2),
                      "fraction_of_fp16": round((kbytes + vbytes) / (4 * d), 4)},
    }
    print(json.dumps(rec), flush=True)
    cache.close()


if __name__ == "__main__":
    main()
