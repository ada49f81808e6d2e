"""Throughput of cached block-wise masked-diffusion decoding on one MI355X.

A step is one dllm_generate over one batch: prefill (refresh of block 0), then every block
(refresh at its start, cached denoising steps until it is committed).  The default workload is
the LLaDA-8B shape (32 layers, d_model 4096, 32 heads x 128, SwiGLU 12288, vocab 126464) with
seeded random-init bf16 weights, batch 1, a 512-token uniform random prompt, gen_length 256,
block_size 32, threshold 0.9, dual prefix+suffix KV cache.

Prints one JSON line.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="llada8b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: this build runs on one GPU only; --gpus must be 1 "
              "(multi-GPU sharding is described, not built)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    from diffusion_block_denoise_amd import dllm

    cfg = synth.configs.get(args.workload)
    torch.cuda.set_device(0)
    t0 = time.time()
    W = synth.weights_torch(cfg, device="cuda")
    torch.cuda.synchronize()
    log(f"weights generated in {time.time() - t0:.1f}s")
    h = dllm.Handle(cfg, W)
    prompt = synth.prompt_np(cfg)
    for i in range(args.warmup):
        _, st = h.generate(prompt)
        log(f"warmup {i}: {st['steps']} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    steps = []
    for i in range(args.steps):
        _, st = h.generate(prompt)
        steps.append(st)
        log(f"step {i}: {st['steps']} denoise steps")
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    B, G = cfg["batch"], cfg["gen_length"]
    value = B * G * args.steps / el
    out = {
        "metric": "committed tokens/s (LLaDA-8B shape, block 32, threshold 0.9)",
        "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": el / args.steps * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded random-init weights, uniform random prompt)",
        "config": {"workload": cfg["name"], "batch": B, "prompt_len": cfg["prompt_len"],
                   "gen_length": G, "block_size": cfg["block_size"],
                   "threshold": cfg["threshold"], "use_cache": "dual"},
        "denoise_steps_per_generate": steps[-1]["steps"],
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
