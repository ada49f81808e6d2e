"""Throughput of cached block-wise masked-diffusion decoding on one MI355X.

A step is one dllm_generate over one batch: prefill (refresh of block 0), then every block
(refresh at its start, cached denoising steps until it is committed).  The default workload is
the LLaDA-8B shape (32 layers, d_model 4096, 32 heads x 128, SwiGLU 12288, vocab 126464) with
seeded random-init bf16 weights, batch 1, a 512-token uniform random prompt, gen_length 256,
block_size 32, threshold 0.9, dual prefix+suffix KV cache.

Prints one JSON line with:
  value        committed tokens/s over the timed generates (inputs resident in HBM)
  roofline     the kernel class with the most time: algorithmic bytes (HBM-bound class) or
               flops (MFMA-bound class) per launch over its average duration, measured with HIP
               events around each launch in one more generate of the same workload after the
               timed ones (events add a gap per launch, so the timed generates run without them),
               against MI355X's published peak
  cpu_baseline the fp64 oracle timed on the host cores on a bounded sample of the same
               workload, projected to tokens/s with this run's refresh/step counts
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
F32_PEAK_TFLOPS = 157.3     # MI355X fp32 vector, published


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def phase_latency(h, prompt, cfg, nb):
    """Median block-refresh and cached-step latency (ms) over the first nb blocks, timed with
    events on the stream."""
    import torch
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    h.prefill(prompt)
    refresh, step = [], []
    for b in range(nb):
        if b:
            e0, e1 = ev(), ev()
            e0.record()
            h.block_begin(b)
            e1.record()
            torch.cuda.synchronize()
            refresh.append(e0.elapsed_time(e1))
        first = True
        done = False
        while not done:
            e0, e1 = ev(), ev()
            e0.record()
            _, done = h.denoise_step()
            e1.record()
            torch.cuda.synchronize()
            if not first:
                step.append(e0.elapsed_time(e1))
            first = False
    med = lambda v: sorted(v)[len(v) // 2] if v else None  # noqa: E731
    return med(refresh), med(step)


def counter_traffic(kernel_class, workload):
    """HBM bytes per launch of a kernel class from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary of the same workload, or None when there is none or the kernel's source
    has changed since the counters were taken (its sha256 no longer matches)."""
    import glob
    import hashlib
    import re
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*_traffic.md"))):
        m = re.search(r"```json\n(.*?)\n```", open(path).read(), re.S)
        if not m:
            continue
        d = json.loads(m.group(1))
        if d.get("kernel_class") != kernel_class or d.get("workload") != workload:
            continue
        src = os.path.join(ROOT, d["source"])
        if not os.path.exists(src):
            return None
        if hashlib.sha256(open(src, "rb").read()).hexdigest() != d["source_sha256"]:
            return None
        return d["traffic_bytes_per_dispatch"]
    return None


def roofline(prof, dtype, workload):
    """Roofline entry for the kernel class with the largest timed share; `workload` names the
    run's configuration for the counter-based traffic (None: a configuration without counters)."""
    name, k = max(prof.items(), key=lambda kv: kv[1]["ms"])
    if k["launches"] == 0 or k["ms"] <= 0:
        return None, name
    t = k["ms"] / 1e3
    if name == "gemm_tiled":
        peak = BF16_PEAK_TFLOPS if dtype == "bf16" else F32_PEAK_TFLOPS
        ach = k["flops"] / t / 1e12
        return {"bound": "mfma", "achieved": ach, "peak": peak, "unit": "TFLOP/s",
                "frac": ach / peak, "traffic": counter_traffic(name, workload), "kernel": name,
                "launches": k["launches"], "avg_us": k["ms"] / k["launches"] * 1e3}, name
    ach = k["bytes"] / t / 1e9
    return {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": ach / HBM_PEAK_GBS, "traffic": counter_traffic(name, workload), "kernel": name,
            "launches": k["launches"], "avg_us": k["ms"] / k["launches"] * 1e3}, name


def phase_roofline(cfg, refresh_ms, step_ms):
    """Roofline time of a refresh and of a cached step from their algorithmic work, against the
    measured medians, for the dual-cache full-context decode (the rows and context of the other
    modes vary by block; null there).  Work counted once: every weight (bf16) per forward, every
    cached K/V element (a 4-byte hi/lo pair) read once per (batch row, K/V head, layer), 2 flops
    per multiply-add of the projections, the lm_head over the block rows and the attention."""
    if cfg["use_cache"] != 2 or cfg["suffix_window"] >= 0 or cfg["attention"] != "full":
        return None
    B, L, Bs = cfg["batch"], cfg["prompt_len"] + cfg["gen_length"], cfg["block_size"]
    d, H, Hkv, hd, F, V, nl = (cfg["d_model"], cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"],
                               cfg["ffn_dim"], cfg["vocab"], cfg["n_layers"])
    wsz = 2 if cfg["dtype"] == "bf16" else 4
    layer_params = d * (H + 2 * Hkv) * hd + H * hd * d + 3 * d * F
    wbytes = (nl * layer_params + V * d) * wsz
    kv = 2.0 * B * Hkv * L * hd * 4 * nl
    peak_f = (BF16_PEAK_TFLOPS if cfg["dtype"] == "bf16" else F32_PEAK_TFLOPS) * 1e12
    out = {}
    for name, M, keys_read, ms in (("refresh", B * L, 0.0, refresh_ms),
                                   ("cached_step", B * Bs, kv, step_ms)):
        flops = 2.0 * M * nl * layer_params + 2.0 * B * Bs * V * d + 4.0 * M * L * H * hd * nl
        kv_written = 2.0 * M * Hkv * hd * 4 * nl
        byts = wbytes + keys_read + kv_written
        t_hbm, t_mfma = byts / (HBM_PEAK_GBS * 1e9), flops / peak_f
        roof = max(t_hbm, t_mfma) * 1e3
        out[name] = {"bound": "hbm" if t_hbm >= t_mfma else "mfma", "roofline_ms": roof,
                     "measured_ms": ms, "frac": roof / ms if ms else None,
                     "bytes": byts, "flops": flops}
    return out


def cpu_baseline(cfg, W, n_full, n_cached, tokens, sample_layers=2):
    """The oracle on a bounded sample: `sample_layers` of the model's layers, one refresh forward
    over block 1's context and one dual-cache step over its block rows in batch row 0, plus the
    lm_head statistics; scaled by n_layers / sample_layers and projected with the GPU run's
    refresh and cached-step counts."""
    import numpy as np
    import synth
    from oracle import decode as od
    from oracle import model as om
    nl = cfg["n_layers"]
    sc = dict(cfg, n_layers=sample_layers)
    names = synth.configs.weight_names(sample_layers)
    w_host = {n: W[n].float().cpu().numpy() for n in names}
    m = om.Model(sc, w_host)
    x = synth.block_state_np(cfg, 1)[0].astype(np.int64)
    act = od.Decoder(m).active(1)  # block 1's context (all positions unless pruned)
    L = len(act)
    s = cfg["prompt_len"] + cfg["block_size"]
    e = s + cfg["block_size"]
    cache = m.new_cache()
    t0 = time.perf_counter()
    hid = m.forward_rows(x, act, act, cache)
    t_full = time.perf_counter() - t0
    t0 = time.perf_counter()
    m.stats(hid[s:e])
    t_stats = time.perf_counter() - t0
    t0 = time.perf_counter()
    hid = m.forward_rows(x, np.arange(s, e), act, cache)
    t_step = time.perf_counter() - t0
    scale = nl / sample_layers
    T_refresh = t_full * scale + t_stats
    T_step = t_step * scale + t_stats
    total = cfg["batch"] * (n_full * T_refresh + n_cached * T_step)
    cores = len(os.sched_getaffinity(0))
    threads = int(os.environ.get("OMP_NUM_THREADS", cores))
    return {"value": tokens / total, "unit": "tokens/s (projected)", "cores": min(cores, threads),
            "kind": "oracle",
            "sample": (f"{sample_layers} of {nl} layers, batch row 0: one refresh forward over "
                       f"{L} positions ({t_full:.2f}s), one dual-cache step over "
                       f"{cfg['block_size']} block rows ({t_step:.2f}s), lm_head statistics "
                       f"({t_stats:.2f}s); per-layer times x{scale:g}, projected with "
                       f"{n_full} refreshes + {n_cached} cached steps per batch row"),
            "refresh_s": T_refresh, "step_s": T_step}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="llada8b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-profile", action="store_true",
                    help="skip the event-instrumented pass (roofline and kernel classes)")
    ap.add_argument("--suffix-window", type=int, default=None,
                    help="approximate suffix pruning window (default: the workload's, -1 = off)")
    ap.add_argument("--attention", choices=["full", "block_causal"], default=None,
                    help="attention pattern (default: the workload's, full)")
    ap.add_argument("--exit-steps", type=int, default=None,
                    help="early exit for converged tokens: run length (default: the workload's, 0 = off)")
    ap.add_argument("--exit-floor", type=float, default=None,
                    help="early exit: confidence a converged token stays above")
    ap.add_argument("--first-threshold", type=float, default=None,
                    help="first-step confidence scheduling: first-step threshold (< 0 = off)")
    ap.add_argument("--blocks", type=int, default=0,
                    help="time prefill plus only the first N blocks (default: the whole generate)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy three times (the reference kernel that "
                         "scales the FETCH_SIZE / WRITE_SIZE counters to bytes)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: this build runs on one GPU only; --gpus must be 1 "
              "(the multi-GPU sharding is a design note, not built)", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        n = 256 << 20  # fp32 elements: 1 GiB
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "copies": 3}))
        return

    import synth
    from diffusion_block_denoise_amd import dllm

    cfg = synth.configs.get(args.workload)
    if args.suffix_window is not None:
        cfg["suffix_window"] = args.suffix_window
    if args.attention is not None:
        cfg["attention"] = args.attention
    for key, val in (("exit_steps", args.exit_steps), ("exit_floor", args.exit_floor),
                     ("first_threshold", args.first_threshold)):
        if val is not None:
            cfg[key] = val
    nb_all = cfg["gen_length"] // cfg["block_size"]
    nblocks = args.blocks if 0 < args.blocks < nb_all else nb_all
    torch.cuda.set_device(0)
    t0 = time.time()
    W = synth.weights_torch(cfg, device="cuda")
    torch.cuda.synchronize()
    log(f"weights generated in {time.time() - t0:.1f}s")
    h = dllm.Handle(cfg, W)
    prompt = synth.prompt_np(cfg)

    def run():
        """One step: the whole generate, or prefill plus the first `nblocks` blocks."""
        if nblocks == nb_all:
            return h.generate(prompt)[1]
        h.prefill(prompt)
        for b in range(nblocks):
            if b:
                h.block_begin(b)
            done = False
            while not done:
                _, done = h.denoise_step()
        return h.get_stats()

    for i in range(args.warmup):
        st = run()
        log(f"warmup {i}: {st['steps']} denoise steps")
    # Timed region: plain decode calls, no instrumentation.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    stats = []
    for i in range(args.steps):
        st = run()
        stats.append(st)
        log(f"step {i}: {st['steps']} denoise steps")
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    B, G = cfg["batch"], cfg["gen_length"]
    tokens = B * cfg["block_size"] * nblocks
    value = tokens * args.steps / el
    # Kernel-class durations: the same generate again with HIP events around every launch of the
    # three classes, on the handle's stream (events add a gap per launch, so this pass is not the
    # timed one).
    prof, roof = {}, None
    if not args.no_profile:
        mask = (1 << dllm.DLLM_KC_GEMM_SKINNY) | (1 << dllm.DLLM_KC_GEMM_TILED) | \
            (1 << dllm.DLLM_KC_ATTENTION)
        h.set_profiling(mask)
        run()
        prof = h.get_profile()
        h.set_profiling(0)
    headline = (cfg["name"] == "llada8b" and cfg["suffix_window"] < 0 and nblocks == nb_all
                and cfg["attention"] == "full" and cfg["exit_steps"] == 0
                and cfg["first_threshold"] < 0)
    if not args.no_profile:
        roof, _ = roofline(prof, cfg["dtype"], "llada8b" if headline else None)
    refresh_ms, step_ms = phase_latency(h, prompt, cfg, nblocks)
    st = stats[-1]
    out = {
        "metric": ("committed tokens/s (LLaDA-8B shape, block 32, threshold 0.9)" if headline
                   else f"committed tokens/s ({cfg['name']})"),
        "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": el / args.steps * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": cfg["dtype"],
        "data": "synthetic (seeded random-init weights, uniform random prompt)",
        "config": {"workload": cfg["name"], "layers": cfg["n_layers"], "d_model": cfg["d_model"],
                   "batch": B, "prompt_len": cfg["prompt_len"], "gen_length": G,
                   "block_size": cfg["block_size"], "threshold": cfg["threshold"],
                   "use_cache": ["none", "prefix", "dual"][cfg["use_cache"]],
                   "suffix_window": cfg["suffix_window"], "attention": cfg["attention"],
                   "exit_steps": cfg["exit_steps"], "exit_floor": cfg["exit_floor"],
                   "first_threshold": cfg["first_threshold"], "blocks_timed": nblocks},
        "roofline": roof,
        "denoise_steps_per_generate": st["steps"],
        "refreshes_per_generate": st["full_forwards"],
        "cached_steps_per_generate": st["cached_forwards"],
        "early_exits_per_generate": st["early_exits"],
        "refresh_latency_ms": refresh_ms, "cached_step_latency_ms": step_ms,
        "phase_roofline": phase_roofline(cfg, refresh_ms, step_ms),
        "kernel_classes": {k: {"launches": v["launches"], "ms": v["ms"],
                               "GB_per_s": v["bytes"] / (v["ms"] / 1e3) / 1e9 if v["ms"] else None,
                               "TFLOP_per_s": v["flops"] / (v["ms"] / 1e3) / 1e12 if v["ms"] else None,
                               "hbm_frac": v["bytes"] / (v["ms"] / 1e3) / 1e9 / HBM_PEAK_GBS
                               if v["ms"] else None,
                               "mfma_frac": v["flops"] / (v["ms"] / 1e3) / 1e12 / (
                                   BF16_PEAK_TFLOPS if cfg["dtype"] == "bf16" else F32_PEAK_TFLOPS)
                               if v["ms"] else None}
                           for k, v in prof.items()},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline and cfg["attention"] == "full":  # the sample is a full-context one
        t0 = time.time()
        out["cpu_baseline"] = cpu_baseline(cfg, W, st["full_forwards"], st["cached_forwards"],
                                           tokens)
        log(f"cpu baseline sample took {time.time() - t0:.1f}s")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
