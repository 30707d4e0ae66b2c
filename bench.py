#!/usr/bin/env python3
"""Benchmark of one decoupled-sparse-attention layer step on one MI355X.

A step is the whole per-layer hot path on one synthetic video-DiT layer:
  da_reassign  (assign keys to the cached centroids, refresh centroids / mean values /
                sizes / per-query-block counts)
  da_forward   (exact attention on the plan's fixed blocks + cluster compensation)
Inputs are generated on the host from the seeded generator, copied to HBM once, and are
resident before timing starts. The cluster cache is warmed by 10 untimed reassign steps.

Prints ONE JSON line. `value` is milliseconds per attention layer (lower is better);
`roofline` describes the dominant kernel (the fused forward) against the bf16 MFMA peak
on its exact-block FLOPs; `cpu_baseline` is the fp64 oracle timed on a bounded sample on
this host and extrapolated to the same unit.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--config hunyuan13b_bf16]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 (published)
MFMA_F32_PEAK_TFLOPS = 157.3
HBM_PEAK_GBS = 8000.0
DEFAULT_CONFIG = "hunyuan13b_bf16"   # 13B-class layer at 5% density (the headline workload)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "forward_hunyuan13b_bf16_traffic.json")
FORWARD_SRC = os.path.join(ROOT, "sparse_attention_video_da_amd", "csrc", "forward.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default=DEFAULT_CONFIG)
    ap.add_argument("--heads", type=int, default=0, help="override head count (0 = config)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="approximate CPU time budget of the oracle sample")
    ap.add_argument("--no-flush", action="store_true",
                    help="skip the reassign timing with the MALL flushed between reps")
    ap.add_argument("--no-drift-chain", action="store_true",
                    help="skip the per-step chain of a workload with denoising steps")
    ap.add_argument("--variance", action="store_true",
                    help="time the variance-corrected step (da_reassign_var + da_forward_var)")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the measured bf16 MFMA and HBM copy peaks")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after timing, run one plain device copy of this many MiB (a "
                         "known-size kernel that calibrates HBM byte counters)")
    return ap.parse_args()


def forward_source_sha() -> str:
    return hashlib.sha256(open(FORWARD_SRC, "rb").read()).hexdigest()[:16]


def load_traffic(workload: str):
    """HBM bytes per forward launch from the committed rocprofv3 counter summary, or None
    when it is missing, covers another workload or was taken on a different forward kernel
    source."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if t.get("forward_source_sha") != forward_source_sha() or t.get("workload") != workload:
        return None
    return t.get("hbm_bytes_per_launch")


REASSIGN_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "reassign_hunyuan13b_bf16_traffic.json")
REASSIGN_SRC = os.path.join(ROOT, "sparse_attention_video_da_amd", "csrc", "reassign.hip")
PEAK_LIB = os.path.join(ROOT, "sparse_attention_video_da_amd", "lib", "libdapeak.so")


def source_sha(path: str) -> str:
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def load_reassign_traffic(workload: str):
    """HBM bytes per reassign step (all its kernels) from the committed counter summary, or
    None when missing, for another workload, or taken on a different reassign source."""
    try:
        t = json.load(open(REASSIGN_TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if t.get("reassign_source_sha") != source_sha(REASSIGN_SRC) or t.get("workload") != workload:
        return None
    return t.get("hbm_bytes_per_step")


def measured_peaks(torch):
    """bf16 MFMA peak (independent 32x32x16 chains, 4 waves per SIMD) and HBM copy rate (2 GiB
    read + 2 GiB written per rep), timed with HIP events on the device."""
    import ctypes
    lib = ctypes.CDLL(PEAK_LIB)
    lib.dapeak_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                     ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_double)]
    lib.dapeak_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                ctypes.c_int, ctypes.POINTER(ctypes.c_float)]
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    wgs = 4 * ncu
    out = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    ms, flop = ctypes.c_float(), ctypes.c_double()
    if lib.dapeak_mfma_bf16(wgs, 100000, ctypes.c_void_p(out.data_ptr()), ctypes.byref(ms),
                            ctypes.byref(flop)) != 0:
        return None
    mfma_tflops = flop.value / (ms.value * 1e-3) / 1e12
    nbytes = 2 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    cms = ctypes.c_float()
    if lib.dapeak_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
                       nbytes, 8 * ncu, 5, ctypes.byref(cms)) != 0:
        return None
    copy_gbs = 2.0 * nbytes / (cms.value * 1e-3) / 1e9
    lib.dapeak_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int,
                                ctypes.c_void_p, ctypes.POINTER(ctypes.c_float)]
    rout = torch.empty(8 * ncu * 256, dtype=torch.int32, device="cuda")
    rms = ctypes.c_float()
    if lib.dapeak_read(ctypes.c_void_p(src.data_ptr()), nbytes, 8 * ncu, 5,
                       ctypes.c_void_p(rout.data_ptr()), ctypes.byref(rms)) != 0:
        return None
    read_gbs = nbytes / (rms.value * 1e-3) / 1e9
    del src, dst, rout
    torch.cuda.empty_cache()
    return {"mfma_bf16_tflops": round(mfma_tflops, 1), "hbm_copy_gbs": round(copy_gbs, 1),
            "hbm_read_gbs": round(read_gbs, 1),
            "mfma_note": "v_mfma_f32_32x32x16_bf16, 8 independent accumulators per wave, "
                         "4 waves per SIMD",
            "hbm_note": "2 GiB device-to-device copy (read + write bytes counted) and 2 GiB "
                        "streaming read, 16-byte nontemporal accesses, 4 in flight a thread"}


def cpu_model() -> str:
    """The host CPU's model name (lscpu, else /proc/cpuinfo)."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, L, mask, budget_s: float):
    """The fp64 oracle on a bounded sample of the same workload, extrapolated to ms/layer."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count() or 1
    h = 0
    K = O.to_f64(L["K"][h], cfg.dtype)
    V = O.to_f64(L["V"][h], cfg.dtype)
    Q = O.to_f64(L["Q"][h], cfg.dtype)
    mu0 = O.to_f64(L["cache_init"][h], cfg.dtype)
    nb = cfg.num_blocks
    # reassign over a key sample (assignment cost is linear in keys), then the refresh and
    # counts over the whole head
    nk = min(cfg.seq_len, 16384)
    t0 = time.perf_counter()
    O.assign(K[:nk], mu0)
    t_assign = (time.perf_counter() - t0) * cfg.seq_len / nk
    a = O.assign(K[:nk], mu0)[0]
    a_full = np.concatenate([a, np.resize(a, cfg.seq_len - nk)]) if nk < cfg.seq_len else a
    t0 = time.perf_counter()
    st = O.refresh(K, V, a_full, mu0, mask[0], cfg.block, cfg.dtype, kblock=cfg.kblock)
    t_refresh = time.perf_counter() - t0
    # forward over a sample of query blocks, as many as fit the budget
    qb = list(np.random.default_rng(0).choice(nb, size=nb, replace=False))
    done, t_fwd = 0, 0.0
    t_start = time.perf_counter()
    while done < nb and (time.perf_counter() - t_start) < budget_s:
        b = qb[done]
        t0 = time.perf_counter()
        O.forward(Q, K, V, st["mu1"], st["vbar"], st["counts"], mask[0], cfg.block,
                  qblocks=[b], kblock=cfg.kblock)
        t_fwd += time.perf_counter() - t0
        done += 1
    per_head_s = t_assign + t_refresh + t_fwd * nb / max(done, 1)
    ms_layer = per_head_s * cfg.heads * 1e3
    out = {"value": round(ms_layer, 1), "unit": "ms/layer", "cores": int(cores),
           "kind": "oracle", "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
           "sample": (f"head 0 of {cfg.heads}: assignment of {nk} of {cfg.seq_len} keys, "
                      f"refresh+counts over all keys, forward of {done} of {nb} query blocks "
                      f"(fp64 numpy); extrapolated linearly to all blocks and heads")}
    # the same with one BLAS thread, on a smaller sample (the refresh and counts are not
    # threaded, so their time is reused)
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(1):
            nk1 = min(cfg.seq_len, 4096)
            t0 = time.perf_counter()
            O.assign(K[:nk1], mu0)
            t_assign1 = (time.perf_counter() - t0) * cfg.seq_len / nk1
            done1, t_fwd1 = 0, 0.0
            t_start = time.perf_counter()
            while done1 < nb and (time.perf_counter() - t_start) < budget_s / 3:
                t0 = time.perf_counter()
                O.forward(Q, K, V, st["mu1"], st["vbar"], st["counts"], mask[0], cfg.block,
                          qblocks=[qb[done1]], kblock=cfg.kblock)
                t_fwd1 += time.perf_counter() - t0
                done1 += 1
        per_head1 = t_assign1 + t_refresh + t_fwd1 * nb / max(done1, 1)
        out["value_1_thread"] = round(per_head1 * cfg.heads * 1e3, 1)
        out["sample_1_thread"] = (f"one BLAS thread: assignment of {nk1} keys, forward of "
                                  f"{done1} query blocks, refresh time reused")
    except Exception as e:  # reported, never fatal
        out["value_1_thread"] = None
        out["sample_1_thread"] = repr(e)
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the per-head "
              "decomposition shards across GPUs without communication, but no multi-GPU "
              "figure is measured here.", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    from datagen import get_config, make_layer
    import sparse_attention_video_da_amd as S

    cfg = get_config(args.config)
    if args.heads:
        cfg = cfg.with_heads(args.heads)
    H, N, d, B, C = cfg.heads, cfg.seq_len, cfg.head_dim, cfg.block, cfg.clusters
    Skb = cfg.kblock
    nb = cfg.num_blocks
    log(f"[bench] generating {cfg.name}: H={H} N={N} d={d} B={B} C={C} nb={nb}")
    t0 = time.time()
    L = make_layer(cfg, threads=16)
    mask = L["mask"]
    log(f"[bench] inputs ready in {time.time() - t0:.1f}s; exact pairs/head={int(mask.sum())}")

    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32

    def dev(x):
        a = np.ascontiguousarray(x)
        if cfg.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(a).cuda()

    Q, K, V = dev(L["Q"]), dev(L["K"]), dev(L["V"])
    cache = dev(L["cache_init"])
    del L["Q"]
    plan = S.Plan(H, N, d, B, C, mask, dtype=cfg.dtype, key_block=Skb)
    var = bool(args.variance)
    outs = [plan.reassign(K, V, cache, variance=var), None]
    outs[1] = {k: torch.empty_like(v) for k, v in outs[0].items()}
    # warm the cache: 10 Lloyd steps on the device (untimed)
    cur = cache
    for i in range(10):
        o = outs[i % 2]
        plan.reassign(K, V, cur, out=o, variance=var)
        cur = o["centroids"]
    mu0 = cur.clone()
    work = {k: torch.empty_like(v) for k, v in outs[0].items()}
    O_out = torch.empty_like(Q)
    torch.cuda.synchronize()
    log("[bench] cache warmed (10 untimed reassign steps)")

    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        plan.reassign(K, V, mu0, out=work, variance=var)
        if ev is not None:
            ev[1].record(stream)
        plan.forward(Q, K, V, work["centroids"], work["mean_values"], work["counts"], out=O_out,
                     variance=work["variance"] if var else None)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    re_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    fw_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    fw_all = [e[1].elapsed_time(e[2]) for e in evs]
    re_all = [e[0].elapsed_time(e[1]) for e in evs]
    fw_med = float(np.median(fw_all))
    log(f"[bench] {args.steps} steps: wall {wall_ms:.3f} ms/step, reassign {re_ms:.3f} ms, "
        f"forward {fw_ms:.3f} ms (median {fw_med:.3f})")

    # reassign with the 256 MB MALL flushed before each rep (a 1 GiB device write between
    # reps), for the HBM-bound reassign's cold-cache figure
    flushed = []
    if not args.no_flush:
        scratch = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        for i in range(5):
            scratch.fill_(float(i))
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ev[0].record(stream)
            plan.reassign(K, V, mu0, out=work, variance=var)
            ev[1].record(stream)
            torch.cuda.synchronize()
            flushed.append(ev[0].elapsed_time(ev[1]))
        del scratch
        torch.cuda.empty_cache()

    # denoising-step chain of a workload with drift: each step drifts K (and V) on the host,
    # uploads them (untimed), runs the step 5 times untimed (the GPU idled during the host
    # work and its clocks ramp up again), then times 5 more back-to-back reps of reassign
    # from the carried cache and the forward (medians; the cache carried on is the step's
    # refresh)
    chain = []
    if cfg.steps > 0 and not args.no_drift_chain:
        from datagen import drift_layer
        log(f"[bench] drift chain: {cfg.steps} steps")
        cur_mu = mu0.clone()
        Lh = L
        for s_ in range(cfg.steps):
            Lh = drift_layer(cfg, Lh, s_, threads=16)
            Kd, Vd = dev(Lh["K"]), dev(Lh["V"])
            torch.cuda.synchronize()
            evs_c = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(10)]
            for r in range(10):
                evs_c[r][0].record(stream)
                plan.reassign(Kd, Vd, cur_mu, out=work, variance=var)
                evs_c[r][1].record(stream)
                plan.forward(Q, Kd, Vd, work["centroids"], work["mean_values"], work["counts"],
                             out=O_out, variance=work["variance"] if var else None)
                evs_c[r][2].record(stream)
            torch.cuda.synchronize()
            rs = [e[0].elapsed_time(e[1]) for e in evs_c[5:]]
            fs = [e[1].elapsed_time(e[2]) for e in evs_c[5:]]
            r_ms, f_ms = float(np.median(rs)), float(np.median(fs))
            chain.append({"step": s_ + 1, "reassign_ms": round(r_ms, 4),
                          "forward_ms": round(f_ms, 4), "layer_ms": round(r_ms + f_ms, 4)})
            cur_mu = work["centroids"].clone()
            del Kd, Vd
        log(f"[bench] drift chain: " + ", ".join(f"{c['layer_ms']:.3f}" for c in chain) + " ms")

    # exact (query block, key block) pairs over all heads: one shared mask or one per head;
    # a pair is B queries against S keys: 2*B*S*d for the scores and as many for P V
    pairs_all = int(mask.sum()) * (H if mask.shape[0] == 1 else 1)
    pairs = pairs_all / H
    exact_flop = 4.0 * B * Skb * d * pairs_all
    comp_flop = 4.0 * N * C * d * H
    dense_flop = 4.0 * N * N * d * H
    peak = MFMA_BF16_PEAK_TFLOPS if cfg.dtype == "bf16" else MFMA_F32_PEAK_TFLOPS
    achieved = exact_flop / (fw_ms * 1e-3) / 1e12
    es = 2 if cfg.dtype == "bf16" else 4
    re_bytes = (2.0 * H * N * d * es          # K, V once
                + H * N * 4                   # assignments
                + 2.0 * H * C * d * es        # refreshed centroids + means
                + H * nb * C * 4.0)           # counts
    traffic = load_traffic(cfg.name)
    peaks = None
    if not args.no_peaks:
        log("[bench] measuring the bf16 MFMA and HBM copy peaks ...")
        try:
            peaks = measured_peaks(torch)
        except Exception as e:  # reported, never fatal
            peaks = {"error": repr(e)}
    result = {
        "metric": "ms per attention layer + achieved MFMA bf16 TFLOPS fraction at 5% density",
        "value": round(wall_ms, 4),
        "unit": "ms/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded Gaussian-mixture Q/K, N(0,1) V, 3D-local position mask)",
        "config": {"workload": cfg.name, "heads": H, "seq_len": N, "latent": [cfg.frames,
                   cfg.height, cfg.width], "head_dim": d, "block": B, "clusters": C,
                   "key_block": Skb, "exact_blocks_per_row": cfg.blocks_per_row,
                   "density": round(pairs / (nb * cfg.num_key_blocks), 4),
                   "mask_heads": int(mask.shape[0]), "variance_corrected": var,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": traffic, "kernel": f"fwd_bf16_kernel<{d},{B},{Skb},{str(var).lower()}>" if
                     cfg.dtype == "bf16" else f"fwd_f32_kernel<{d},{B}>",
                     "flops_per_launch": exact_flop,
                     "flops_basis": "exact-block MFMA work, 4*B*S*d per (query block, exact "
                                    "key block of S keys) pair",
                     "forward_source_sha": source_sha(FORWARD_SRC),
                     "frac_of_measured_peak": (round(achieved / peaks["mfma_bf16_tflops"], 4)
                                               if peaks and "mfma_bf16_tflops" in peaks
                                               else None)},
        "reassign_roofline": {
            "bound": "hbm", "achieved": round(re_bytes / (re_ms * 1e-3) / 1e9, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(re_bytes / (re_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "traffic": load_reassign_traffic(cfg.name),
            "bytes_per_step": re_bytes,
            "bytes_basis": "K and V read once, assignments, refreshed centroids and mean values, "
                           "counts written once",
            "reassign_source_sha": source_sha(REASSIGN_SRC),
            # the step's bytes are nearly all reads: against the measured streaming-read rate
            "frac_of_measured_peak": (round(re_bytes / (re_ms * 1e-3) / 1e9
                                            / peaks["hbm_read_gbs"], 4)
                                      if peaks and "hbm_read_gbs" in peaks else None),
            "assign_mfma_flop": 2.0 * C * d * N * H},
        "peaks_measured": peaks,
        "breakdown": {
            "forward_ms": round(fw_ms, 4), "forward_ms_median": round(fw_med, 4),
            "forward_ms_p10_p90": [round(float(np.percentile(fw_all, 10)), 4),
                                   round(float(np.percentile(fw_all, 90)), 4)],
            "reassign_ms": round(re_ms, 4),
            "reassign_ms_median": round(float(np.median(re_all)), 4),
            "reassign_ms_p10_p90": [round(float(np.percentile(re_all, 10)), 4),
                                    round(float(np.percentile(re_all, 90)), 4)],
            "forward_tflops_exact": round(achieved, 1),
            "forward_tflops_exact_plus_compensation": round(
                (exact_flop + comp_flop) / (fw_ms * 1e-3) / 1e12, 1),
            "dense_equivalent_tflops": round(dense_flop / (fw_ms * 1e-3) / 1e12, 1),
            "reassign_algorithmic_gbs": round(re_bytes / (re_ms * 1e-3) / 1e9, 1),
            "reassign_hbm_frac": round(re_bytes / (re_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "reassign_ms_mall_flushed": round(float(np.median(flushed)), 4) if flushed else None,
            "reassign_hbm_frac_mall_flushed": (round(re_bytes / (float(np.median(flushed)) * 1e-3)
                                                     / 1e9 / HBM_PEAK_GBS, 4) if flushed else None),
        },
        "cpu_baseline": None,
    }
    if chain:
        result["drift_chain"] = {"steps": chain, "mean_layer_ms": round(
            float(np.mean([c["layer_ms"] for c in chain])), 4)}
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle sample on the host ...")
        try:
            L2 = make_layer(cfg, heads=[0], threads=4)
            result["cpu_baseline"] = cpu_baseline(cfg, L2, mask, args.cpu_seconds)
        except Exception as e:  # reported, never fatal to the GPU figure
            result["cpu_baseline"] = {"error": repr(e)}
    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_probe_bytes"] = {"read": n * 4, "write": n * 4}
        del src, dst
    plan.close()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
