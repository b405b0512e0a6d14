#!/usr/bin/env python3
"""Benchmark of certified quantized-KV decode attention on one MI355X.

A step is one certified decode-attention call for one layer (all heads of
the batch): INT8 scoring, selection and bounds, FP16 paging from pinned host
memory, tail / promoted passes, rank check and any fallback.  Steps cycle
through all layers of the workload in order, so each layer-step reads its
own tier 1 (227 MB at 32K x 4 and at 128K: the 256 MB Infinity Cache cannot
serve it from a previous step).  Inputs are synthetic (datagen) and resident
(tier 1 in HBM, tier 2 in pinned host memory) before the timed region.

Order: the headline layer-steps of every workload (each in a cache of its
own), then the comparison lines of the first two workloads (device paging,
run copies, threshold variants, cache configurations, decode loops, the
dense comparator; fresh caches), then the CPU oracle baseline, so that no
comparison line's allocations or the oracle's threads perturb a headline.

Prints one JSON line.  `value` = KV tokens (batch x context) per second per
layer-step of the first workload (the 32K x 4 LLaMA-3.1-8B-shaped layer by
default); the 128K workload's figures are in `other_workloads`.  `roofline`
is measured for the dominant kernel (largest time per step among the passes
whose algorithmic bytes are defined); each kernel's launch duration is its
own execution span (first wave's start to last wave's end), stamped by the
kernel on the device's constant-rate wall clock while the timed steps run.
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
    ap.add_argument("--workload", default="llama_32k,needle_128k,llama_8k,needle_64k,stress_32k",
                    help="comma-separated workloads; the first one is the reported value, the "
                         "comparison lines (--no-extras) run on the first two")
    ap.add_argument("--layers", type=int, default=0, help="layers to build (0: the workload's)")
    ap.add_argument("--decode-steps", type=int, default=4,
                    help="decode-loop steps after the timed region, first workload only: one token "
                         "appended to every sequence of every layer, then that layer's certified step")
    ap.add_argument("--no-extras", action="store_true",
                    help="only the headline layer-steps (no device-paging, variant or decode-loop lines): "
                         "for profiler runs")
    ap.add_argument("--staged-threads", type=int, default=-1,
                    help="host threads packing the paged blocks into pinned chunks "
                         "(0: one copy per run of blocks; -1: the library's default)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="accepted for older command lines: the plain 1 GiB read+write kernel "
                         "(counter calibration) always runs")
    return ap.parse_args()


def block_layout(k, v):
    """[B][T][Hkv][d] FP16 bits -> the FP16 block layout of the library."""
    import numpy as np
    B, T, Hkv, d = k.shape
    kb = k.reshape(B, T // 64, 64, Hkv, d // 8, 8).transpose(0, 3, 1, 4, 2, 5)
    vb = v.reshape(B, T // 64, 64, Hkv, d).transpose(0, 3, 1, 4, 2)
    return np.ascontiguousarray(kb), np.ascontiguousarray(vb)


def counters_for(kernel, workload):
    """HBM traffic per layer-step (the kernel's dispatches of one step summed,
    like its algorithmic bytes and kernel-clock time) from a committed
    rocprofv3 --pmc summary, if it was taken on the current kernel source
    (else None)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_counters.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    src = open(os.path.join(ROOT, "certified_quantized_kv_amd", "csrc", "ckv_decode.hip"), "rb").read()
    if rec.get("source_sha1") != hashlib.sha1(src).hexdigest():
        return None
    return rec.get("traffic_bytes_per_step", rec.get("traffic_bytes_per_dispatch"))


def cpu_info():
    """Host CPU model and the cores this process may use."""
    model = "unknown"
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return model, os.cpu_count(), usable


def run_workload(name, args, decode_steps=0, extras=False):
    import numpy as np
    import torch

    import certified_quantized_kv_amd as ckv
    import datagen

    cfg = datagen.CONFIGS[name]
    L = args.layers or cfg["L"]
    B, T, Hq, Hkv, d = cfg["B"], cfg["T"], cfg["Hq"], cfg["Hkv"], cfg["d"]
    dev = torch.device("cuda:0")
    log(f"workload {name}: {L} layers, batch {B}, context {T}, {Hq}/{Hkv} heads, d {d}")
    t0 = time.time()
    # room for the decode loop's tokens (one more block)
    cache = ckv.Cache(L, B, Hq, Hkv, d, T + (64 if decode_steps else 0), device=0)
    if args.staged_threads >= 0:
        cache.set_staged_paging(args.staged_threads)
    fp = cache.footprint()
    log(f"cache created in {time.time() - t0:.1f}s: device {fp['device'] / 2**30:.2f} GiB "
        f"(tier 1 {fp['tier1'] / 2**30:.2f} GiB), pinned host {fp['host'] / 2**30:.2f} GiB")
    qs = []
    n_dense = 0 if (args.no_dense or not extras) else min(L, 4)
    dense_kv = []
    for l in range(L):
        t1 = time.time()
        lay = datagen.make_layer(name, l)
        for n in range(B):
            cache.append_kv(l, n, lay.k[n], lay.v[n])
        qs.append(torch.from_numpy(lay.q.view(np.float16)).to(dev))
        if l < n_dense:
            kb, vb = block_layout(lay.k, lay.v)
            dense_kv.append((torch.from_numpy(kb.view(np.float16)).to(dev),
                             torch.from_numpy(vb.view(np.float16)).to(dev)))
        if l % 8 == 0 or l == L - 1:
            log(f"layer {l} generated and appended in {time.time() - t1:.1f}s")
    sm = cfg["sm"]
    th = ckv.default_thresholds(sm)
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)

    for i in range(args.warmup):
        cache.certified_decode_attention(i % L, qs[i % L], th, out=out)
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done")

    # timed region: K layer-steps; with profiling on, each timed kernel
    # stamps its execution span on the device clock; every call returns
    # after its report is on the host, so the host clock times each step
    cache.set_profiling(True)
    reps = []
    step_s = []
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        l = (args.warmup + i) % L
        t_i = time.perf_counter()
        _, rep = cache.certified_decode_attention(l, qs[l], th, out=out)
        step_s.append(time.perf_counter() - t_i)
        reps.append(rep)
    torch.cuda.synchronize()
    t_end = time.perf_counter()
    prof = cache.profile()
    cache.set_profiling(False)
    rungs = np.zeros(5, np.int64)
    for rep in reps:
        for r in range(5):
            rungs[r] += int((rep["rung_max"] == r).sum())
    kstar = float(np.mean([rep["kstar"].mean() for rep in reps]))
    nvp = float(np.mean([rep["n_v_promoted"].mean() for rep in reps]))
    K = args.steps
    elapsed = t_end - t_start
    ms_step = 1e3 * elapsed / K
    value = B * T * K / elapsed
    log(f"timed {K} steps: {ms_step:.3f} ms/step, {value:.4g} KV tokens/s")

    # algorithmic bytes: INT8 K + K metadata (scoring), INT4 V + V metadata
    # (tail, promoted INT4), FP16 blocks (promoted), per block of 64 tokens
    q8_blk = 64 * d + 4 * d
    i4_blk = 64 * (d // 2) + 64 * 4 * (d // 32)
    f16_blk = 64 * d * 2
    ph = prof["phases"]

    def per_step(phase):
        ms, cnt = ph[phase]
        return ms / K, cnt

    kern = {
        "k_score": ("score", prof["q8_blocks"] * q8_blk),
        "k_values_tail": ("tail", prof["tail_blocks"] * i4_blk),
        "k_keys16": ("keys16", prof["k16_blocks"] * f16_blk),
        "k_promoted4": ("promoted4", prof["int4p_blocks"] * i4_blk),
        "k_promoted16": ("promoted16", prof["v16_blocks"] * f16_blk),
    }
    table = {}
    for kname, (phase, total_bytes) in kern.items():
        ms_tot, cnt = ph[phase]
        if not cnt:
            continue
        avg = ms_tot / cnt
        per_launch = total_bytes / cnt
        table[kname] = dict(avg_launch_ms=round(avg, 5), algorithmic_bytes_per_launch=int(per_launch),
                            achieved_GBps=round(per_launch / (avg * 1e-3) / 1e9, 1))
    dom = max(table, key=lambda k: table[k]["avg_launch_ms"])
    ach = table[dom]["achieved_GBps"]
    roofline = {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": counters_for(dom, name),
                "kernel": dom, "avg_launch_ms": table[dom]["avg_launch_ms"],
                "algorithmic_bytes_per_launch": table[dom]["algorithmic_bytes_per_launch"]}
    # the scoring and tail passes together (the INT8/INT4 tier-1 stream)
    k13 = [k for k in ("k_score", "k_values_tail") if k in table]
    if len(k13) == 2:
        b13 = sum(table[k]["algorithmic_bytes_per_launch"] for k in k13)
        t13 = sum(table[k]["avg_launch_ms"] for k in k13)
        k13_rec = {"achieved": round(b13 / (t13 * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                   "frac": round(b13 / (t13 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    else:
        k13_rec = None
    tier1_step = prof["q8_blocks"] * q8_blk / K + B * T * Hkv * (d / 2 + 4 * d / 32 + 4 / 64)
    paged_step = prof["bytes_paged"] / K
    st_ms = np.sort(np.array(step_s)) * 1e3
    rec = {
        "ms_per_step": round(ms_step, 4), "value": round(value, 1),
        "ms_per_step_p10_p50_p90": [round(float(np.percentile(st_ms, q)), 4) for q in (10, 50, 90)],
        "roofline": roofline, "kernels": table, "score_and_tail_hbm": k13_rec,
        "hbm_algorithmic_GBps_end_to_end": round((tier1_step + paged_step) / (elapsed / K) / 1e9, 1),
        "paged_MiB_per_step": round(paged_step / 2 ** 20, 2),
        "blocks_per_step": {k: round(prof[k] / K, 1) for k in
                            ("q8_blocks", "tail_blocks", "k16_blocks", "v16_blocks", "int4p_blocks",
                             "dense_blocks")},
        "h2d_copies_per_step": round(prof["copies"] / K, 1),
        "phases_ms_per_step": {k: round(v[0] / K, 4) for k, v in ph.items()},
        "rungs_max_hist": rungs.tolist(), "kstar_mean": round(kstar, 2),
        "v_promoted_mean": round(nvp, 2),
        "config": {"workload": name, "batch": B, "context": T, "layers": L, "q_heads": Hq,
                   "kv_heads": Hkv, "head_dim": d, "tau_cov": th["tau_cov"], "k_tol": th["k_tol"],
                   "v_tol": th["v_tol"], "rank_tol": th["rank_tol"],
                   "paging": "staged, %d host threads" % prof["staged_threads"]
                   if prof["staged_threads"] > 0 else "runs"},
    }

    if extras:
        extra_lines(rec, args, name, cache, dense_kv, n_dense, qs, th, out, T, sm, B, Hq, Hkv, d, L, cfg,
                    ms_step, decode_steps)
    cache.close()
    del dense_kv

    return rec


def cpu_baseline(name):
    """The CPU oracle on one sequence of layer 0 of workload `name` (a full
    layer-step of that sequence: every head, scoring through outputs), on one
    thread and on every core this process may use (its heads run on OpenMP
    threads).  Run after every GPU measurement: the oracle's threads must not
    compete with the paging threads."""
    import datagen
    import oracle
    cfg = datagen.CONFIGS[name]
    B, T, Hq = cfg["B"], cfg["T"], cfg["Hq"]
    lay = datagen.make_layer(name, 0)
    k1, v1, q1, sm1 = lay.k[:1].copy(), lay.v[:1].copy(), lay.q[:1].copy(), lay.sm
    del lay
    model, ncpu, usable = cpu_info()
    runs = {}
    for thr in (1, usable):
        oracle.set_threads(thr)
        t1 = time.perf_counter()
        oracle.certified_decode(k1, v1, q1, oracle.default_thresholds(sm1), trace=False)
        runs[thr] = time.perf_counter() - t1
        log(f"cpu baseline: {runs[thr]:.2f}s for the sample on {thr} thread(s)")
    oracle.set_threads(usable)
    return {
        "value": round(T / runs[1], 1), "unit": "KV tokens/s", "cores": 1, "kind": "oracle",
        "sample": f"{name} layer 0, sequence 0 of {B}: one full layer-step of one sequence "
                  f"({T} tokens, {Hq} q heads), {runs[1]:.1f} s on one thread",
        "all_cores": {"value": round(T / runs[usable], 1), "cores": usable,
                      "seconds": round(runs[usable], 2)},
        "cpu_model": model, "nproc": ncpu, "usable_cores": usable}


def extra_lines(rec, args, name, cache, dense_kv, n_dense, qs, th, out, T, sm, B, Hq, Hkv, d, L, cfg,
                ms_step, decode_steps):
    """Comparison lines after the headline layer-steps: device-initiated
    paging, the threshold variants against dense attention, the decode loop
    (with and without the FP16 cache) and the dense comparator."""
    import torch
    # the same layer-steps with device-initiated paging (a kernel reading
    # pinned host memory instead of host-issued copies): a comparison line
    cache.set_device_paging(True)
    Kd = min(args.steps, L)
    for i in range(min(args.warmup, 4)):
        cache.certified_decode_attention(i % L, qs[i % L], th, out=out)
    torch.cuda.synchronize()
    cache.set_profiling(True)
    t1 = time.perf_counter()
    for i in range(Kd):
        l = (args.warmup + i) % L
        cache.certified_decode_attention(l, qs[l], th, out=out)
    torch.cuda.synchronize()
    eld = time.perf_counter() - t1
    profd = cache.profile()
    cache.set_profiling(False)
    cache.set_device_paging(False)
    rec["device_paging"] = {"steps": Kd, "ms_per_step": round(1e3 * eld / Kd, 4),
                            "value": round(B * T * Kd / eld, 1),
                            "paged_MiB_per_step": round(profd["bytes_paged"] / Kd / 2 ** 20, 2),
                            "page_ms_per_step": round(profd["phases"]["page"][0] / Kd, 4),
                            # the K gather's first wave after the selection
                            # kernel's last wave, on the device clock: the
                            # paging starts without the host's round trip
                            "gather_start_after_select_us": round(
                                1e3 * profd["gather_lead_ms"] / max(profd["gather_steps"], 1), 2)}
    log(f"device paging: {1e3 * eld / Kd:.3f} ms/step")

    # the same layer-steps with the listed blocks copied as runs (one copy
    # per run of blocks, small gaps filled) instead of host-packed chunks
    staged = rec["config"]["paging"]
    staged = int(staged.split()[1]) if staged.startswith("staged") else 0
    cache.set_staged_paging(0)
    for i in range(min(args.warmup, 4)):
        cache.certified_decode_attention(i % L, qs[i % L], th, out=out)
    torch.cuda.synchronize()
    cache.set_profiling(True)
    t1 = time.perf_counter()
    for i in range(Kd):
        l = (args.warmup + i) % L
        cache.certified_decode_attention(l, qs[l], th, out=out)
    torch.cuda.synchronize()
    elr = time.perf_counter() - t1
    profr = cache.profile()
    cache.set_profiling(False)
    cache.set_staged_paging(staged)
    rec["run_copies"] = {"steps": Kd, "ms_per_step": round(1e3 * elr / Kd, 4),
                         "value": round(B * T * Kd / elr, 1),
                         "paged_MiB_per_step": round(profr["bytes_paged"] / Kd / 2 ** 20, 2),
                         "h2d_copies_per_step": round(profr["copies"] / Kd, 1),
                         "page_ms_per_step": round(profr["phases"]["page"][0] / Kd, 4)}
    log(f"run copies: {1e3 * elr / Kd:.3f} ms/step")

    if n_dense:
        rec["variants"] = variants(cache, dense_kv, qs, th, T, sm, n_dense)
        rec["cache_configs"] = cache_configs(name, cfg, cache, dense_kv, qs, th, T, sm, n_dense)

    if decode_steps:
        rec["decode_loop"] = decode_loop(cache, L, B, Hq, Hkv, d, T, cfg, th, out, decode_steps)
        # the same loop with paged FP16 blocks kept in device memory across
        # steps (the first step of each layer pages, later ones only new blocks)
        free, _ = torch.cuda.mem_get_info()
        nl = cache.enable_fp16_cache(int(free * 0.8))
        rec["decode_loop_fp16_cache"] = dict(decode_loop(cache, L, B, Hq, Hkv, d, T, cfg, th, out, decode_steps),
                                             layers_cached=nl)

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
        dms = 1e3 * (time.perf_counter() - t1) / reps_d
        rec["dense_comparator"] = {"ms_per_step": round(dms, 4),
                                   "hbm_GBps": round(B * T * Hkv * 4 * d / (dms * 1e-3) / 1e9, 1),
                                   "certified_over_dense": round(ms_step / dms, 2),
                                   "layers_cycled": n_dense}
        log(f"dense comparator: {dms:.3f} ms/step")


def variants(cache, dense_kv, qs, th, T, sm, n):
    """The documented variants on the first n layers, each against exact dense
    attention on the FP16 originals: the certified step; plain quantized
    attention (tau_cov = 0, infinite tolerances: no FP16 blocks, its bounds
    still reported); FP16 values for every promoted head (v_tol = 0); and a
    v_tol sweep."""
    import numpy as np
    import torch
    inf = float("inf")
    cases = [("certified", dict(th)),
             ("naive_int8_int4", dict(th, tau_cov=0.0, k_tol=inf, v_tol=inf)),
             ("fp16_values", dict(th, v_tol=0.0)),
             ("v_tol_0.1", dict(th, v_tol=0.1)),
             ("v_tol_0.001", dict(th, v_tol=1e-3))]
    dense = []
    for l in range(n):
        kb, vb = dense_kv[l]
        dense.append(cache.dense_decode_attention(kb, vb, T, qs[l], sm).clone())
    res = {}
    for tag, thv in cases:
        cache.set_profiling(True)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        outs = [cache.certified_decode_attention(l, qs[l], thv) for l in range(n)]
        torch.cuda.synchronize()
        el = time.perf_counter() - t1
        pr = cache.profile()
        cache.set_profiling(False)
        err = max(float((o - dense[l]).abs().max()) for l, (o, _) in enumerate(outs))
        reps = [r for _, r in outs]
        res[tag] = {"ms_per_step": round(1e3 * el / n, 4),
                    "paged_MiB_per_step": round(pr["bytes_paged"] / n / 2 ** 20, 2),
                    "max_abs_err_vs_dense": float(f"{err:.3g}"),
                    "e_key_max": float(f"{max(float(r['e_key'].max()) for r in reps):.3g}"),
                    "e_val_max": float(f"{max(float(r['e_val'].max()) for r in reps):.3g}"),
                    "kstar_mean": round(float(np.mean([r["kstar"].mean() for r in reps])), 2),
                    "v_promoted_mean": round(float(np.mean([r["n_v_promoted"].mean() for r in reps])), 2),
                    "rungs_max_hist": np.bincount(np.concatenate([r["rung_max"].ravel() for r in reps]),
                                                  minlength=5).tolist()}
        log(f"variant {tag}: {res[tag]}")
    return res


def cache_configs(name, cfg, cache, dense_kv, qs, th, T, sm, n):
    """The design's asymmetric cache (INT8 keys, INT4 values) against the
    symmetric one (values at the keys' 8 bits) on the first n layers, each in
    a cache of its own: tier-1 bytes per token and kv head (and against the
    2 d bytes of FP16 K + V), certified and plain quantized latency, and the
    error against dense attention on the FP16 originals."""
    import numpy as np
    import torch

    import certified_quantized_kv_amd as ckv
    import datagen
    B, Hq, Hkv, d = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["d"]
    inf = float("inf")
    dense = [cache.dense_decode_attention(kb, vb, T, qs[l], sm).clone() for l, (kb, vb) in enumerate(dense_kv[:n])]
    res = {}
    for vbits in (4, 8):
        c = ckv.Cache(n, B, Hq, Hkv, d, T, device=0, v_bits=vbits)
        for l in range(n):
            lay = datagen.make_layer(name, l)
            for s_ in range(B):
                c.append_kv(l, s_, lay.k[s_], lay.v[s_])
        per_tok = c.footprint()["tier1"] / (n * B * Hkv * T)
        r = {"tier1_bytes_per_token_per_kv_head": round(per_tok, 2),
             "tier1_vs_fp16_kv": round(per_tok / (4 * d), 4)}
        for tag, thv in (("certified", dict(th)), ("plain_quantized", dict(th, tau_cov=0.0, k_tol=inf, v_tol=inf))):
            for l in range(n):
                c.certified_decode_attention(l, qs[l], thv)
            torch.cuda.synchronize()
            t1 = time.perf_counter()
            outs = [c.certified_decode_attention(l, qs[l], thv) for _ in range(2) for l in range(n)]
            torch.cuda.synchronize()
            el = time.perf_counter() - t1
            err = max(float((o - dense[i % n]).abs().max()) for i, (o, _) in enumerate(outs))
            r[tag] = {"ms_per_step": round(1e3 * el / (2 * n), 4), "max_abs_err_vs_dense": float(f"{err:.3g}"),
                      "e_val_max": float(f"{max(float(rp['e_val'].max()) for _, rp in outs):.3g}"),
                      "v_promoted_mean": round(float(np.mean([rp["n_v_promoted"].mean() for _, rp in outs])), 2)}
        c.close()
        res["asymmetric_int8_int4" if vbits == 4 else "symmetric_int8_int8"] = r
        log(f"cache config v_bits={vbits}: {r}")
    return res


def decode_loop(cache, L, B, Hq, Hkv, d, T, cfg, th, out, steps):
    """Steady-state decode: per step, one new token (synthetic K, V of the
    workload's distributions, from device memory) appended to every sequence
    of every layer (one batched append per layer), each layer's certified
    step right after its appends, a fresh q per layer-step.  Timed from the
    first append to the last step."""
    import torch
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev).manual_seed(4321)
    toks = (torch.randn((steps * L, B, Hkv, d), generator=gen, device=dev).half(),
            torch.randn((steps * L, B, Hkv, d), generator=gen, device=dev).half())
    qs = (torch.randn((steps * L, B, Hq, d), generator=gen, device=dev) * cfg["q_std"]).half()
    T0 = cache.seq_length(0, 0)
    torch.cuda.synchronize()
    t_app = 0.0
    cache.set_profiling(True)
    per_step = []
    for s in range(steps):
        t0 = time.perf_counter()
        for l in range(L):
            i = s * L + l
            ta = time.perf_counter()
            cache.append_token(l, toks[0][i], toks[1][i])   # the batch's tokens in one call
            t_app += time.perf_counter() - ta
            cache.certified_decode_attention(l, qs[i], th, out=out)
        torch.cuda.synchronize()
        per_step.append(time.perf_counter() - t0)
    prof = cache.profile()
    cache.set_profiling(False)
    el = sum(per_step)
    ls = steps * L
    log(f"decode loop: {steps} steps x {L} layers: {1e3 * el / ls:.3f} ms per layer-step "
        f"({1e3 * t_app / ls:.3f} ms of appends), {B * steps / el:.2f} tokens/s; "
        f"per step {[round(1e3 * x / L, 3) for x in per_step]} ms per layer-step")
    return {"steps": steps, "layer_steps": ls, "context_start": T0, "context_end": T0 + steps,
            "ms_per_layer_step": round(1e3 * el / ls, 4),
            "ms_per_layer_step_by_step": [round(1e3 * x / L, 4) for x in per_step],
            "append_ms_per_layer_step": round(1e3 * t_app / ls, 4),
            "paged_MiB_per_layer_step": round(prof["bytes_paged"] / ls / 2 ** 20, 2),
            "generated_tokens_per_s": round(B * steps / el, 3),
            "kv_tokens_per_s": round(B * (T0 + steps / 2) * ls / el, 1)}


def h2d_probe():
    """Pinned host -> device copies: bandwidth of 256 MiB copies (the figure
    the paging time is compared with), and the time per copy of the paging's
    smallest (16 KiB, one block) and of 16 MiB copies, issued back to back on
    one stream."""
    import torch
    x = torch.empty(256 * 2 ** 20, dtype=torch.uint8).pin_memory()
    y = torch.empty_like(x, device="cuda:0")
    y.copy_(x, non_blocking=True)
    torch.cuda.synchronize()
    t = time.perf_counter()
    for _ in range(4):
        y.copy_(x, non_blocking=True)
    torch.cuda.synchronize()
    big = 4 * x.numel() / (time.perf_counter() - t) / 1e9
    res = {"GBps_256MiB": round(big, 1)}
    for size, reps in ((16 * 2 ** 10, 512), (16 * 2 ** 20, 16)):
        xs, ys = x[:size * 2], y[:size * 2]
        for i in range(4):
            ys[(i % 2) * size:(i % 2 + 1) * size].copy_(xs[(i % 2) * size:(i % 2 + 1) * size], non_blocking=True)
        torch.cuda.synchronize()
        t = time.perf_counter()
        for i in range(reps):
            o = (i % 2) * size
            ys[o:o + size].copy_(xs[o:o + size], non_blocking=True)
        torch.cuda.synchronize()
        el = time.perf_counter() - t
        tag = "16KiB" if size < 2 ** 20 else "16MiB"
        res[f"us_per_{tag}_copy"] = round(1e6 * el / reps, 2)
        res[f"GBps_{tag}"] = round(size * reps / el / 1e9, 2)
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the path has no "
              "multi-GPU mode: one process per GPU, each on its own shard of (sequence, kv head).",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import certified_quantized_kv_amd as ckv

    names = [w for w in args.workload.split(",") if w]
    # the headline layer-steps of every workload first, each in a cache of
    # its own, then the comparison lines of the first two (another cache
    # each: they leave large allocations behind), then the CPU oracle
    recs = [run_workload(w, args) for w in names]
    if not args.no_extras:
        for i, w in enumerate(names[:2]):
            ex = run_workload(w, args, decode_steps=(args.decode_steps if i == 0 else 0), extras=True)
            for k, v in ex.items():
                if k not in recs[i]:
                    recs[i][k] = v
    if not args.no_cpu_baseline:
        recs[0]["cpu_baseline"] = cpu_baseline(names[0])
    first = recs[0]
    # achievable HBM rate of a plain streaming kernel (torch's elementwise
    # multiply over 1 GiB: one read and one write of every byte); also the
    # calibration kernel of the traffic counters
    dev = torch.device("cuda:0")
    a = torch.empty(2 ** 28, dtype=torch.float32, device=dev).fill_(1.0)
    b = torch.empty_like(a)
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
    # a read-only pass over the same 1 GiB (torch's sum: every byte read once,
    # one value written): the calibration kernel of the FETCH_SIZE counter
    # (its rate is that of torch's reduction, not a ceiling for reads)
    for _ in range(3):
        a.sum()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(10):
        a.sum()
    torch.cuda.synchronize()
    rms = 1e3 * (time.perf_counter() - t1) / 10
    read_probe = {"bytes_read": 2 ** 30, "ms": round(rms, 4), "GBps": round(2 ** 30 / (rms * 1e-3) / 1e9, 1)}
    # the library's streaming read (ckv_read_probe) with the passes' load
    # shape: 8 KiB (scoring pass) or 16 KiB (FP16-key pass) per wave, every
    # load requested first.  hbm_*: 1 GiB (4x the last-level cache) read back
    # to back; cold_*: 32 distinct buffers of one 32K x 4 layer's scoring
    # bytes (142.6 MB each, 4.6 GB in all) read in turn, back to back, as the
    # scoring pass meets its layers (average per launch, the better of two
    # timed rounds after one untimed); cached_*: the first 128 MiB of the
    # 1 GiB re-read (held by the last-level cache)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    stream_read = {}

    def read_rate(nm, buf, kib, reps=20):
        for _ in range(3):
            ckv.binding.read_probe(buf, kib, sink)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            ckv.binding.read_probe(buf, kib, sink)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        nb = buf.numel() * buf.element_size()
        stream_read[nm] = {"bytes_read": nb, "wave_kib": kib, "ms": round(ms, 4),
                           "GBps": round(nb / (ms * 1e-3) / 1e9, 1)}

    for kib in (4, 8, 16):
        read_rate(f"hbm_1g_{kib}k", a, kib)
    read_rate("cached_128m_8k", a[: 2 ** 25], 8)
    layer_words = 142606336 // 4
    cold = [torch.empty(layer_words, dtype=torch.int32, device=dev).fill_(i) for i in range(32)]
    for kib in (8, 16):
        per_round = []
        for r in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for buf in cold:
                ckv.binding.read_probe(buf, kib, sink)
            e1.record()
            torch.cuda.synchronize()
            per_round.append(e0.elapsed_time(e1) / len(cold))
        ms = min(per_round[1:])
        stream_read[f"cold_143m_{kib}k"] = {"bytes_read": layer_words * 4, "wave_kib": kib,
                                            "ms": round(ms, 4), "GBps": round(layer_words * 4 / (ms * 1e-3) / 1e9, 1)}
    del cold
    del a, b
    line = {
        "metric": METRIC, "value": first["value"], "unit": "KV tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": first["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        # the path's arithmetic: INT8 scores on the int8 matrix cores, FP16-key
        # scores as FP64 chains, values on the f16 matrix cores, softmax and
        # outputs in FP32, bounds in FP64
        "dtype": "i8/f16/f32/f64",
        "data": "synthetic",
        "config": first["config"],
        "roofline": first["roofline"],
        "cpu_baseline": first.get("cpu_baseline"),
    }
    for k, v in first.items():
        if k not in line and k not in ("value",):
            line[k] = v
    line["other_workloads"] = {r["config"]["workload"]: {k: v for k, v in r.items() if k != "config"}
                               for r in recs[1:]}
    h2d = h2d_probe()
    line["pcie_h2d_GBps"] = h2d["GBps_256MiB"]
    line["pcie_h2d"] = h2d
    line["copy_probe"] = copy_probe
    line["read_probe"] = read_probe
    line["stream_read_probe"] = stream_read
    # the dominant kernel and the scoring + tail stream against the plain
    # read of the same load shape on cold data (what these loads can reach
    # here), beside their fractions of the 8 TB/s peak
    cold16, cold8 = stream_read["cold_143m_16k"]["GBps"], stream_read["cold_143m_8k"]["GBps"]
    line["vs_stream_read"] = {
        "dominant_kernel": {"kernel": first["roofline"].get("kernel"), "achieved": first["roofline"]["achieved"],
                            "probe": "cold_143m_16k", "probe_GBps": cold16,
                            "frac": round(first["roofline"]["achieved"] / cold16, 4)},
        "score_and_tail": ({"achieved": first["score_and_tail_hbm"]["achieved"], "probe": "cold_143m_8k",
                            "probe_GBps": cold8,
                            "frac": round(first["score_and_tail_hbm"]["achieved"] / cold8, 4)}
                           if first.get("score_and_tail_hbm") else None),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
