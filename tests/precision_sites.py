"""Diagnostic: how much each bf16 storage site of the GPU path moves the step statistics.

The GPU path stores the operands of its matrix products in bf16.  This diagnostic replays the
oracle's refresh forward (fp64, the same weights) with one bf16 rounding applied at chosen
sites and reports how far the block rows' confidences and logits move from the exact fp64
values.  It decides which sites may hold a single bf16 value and which need the hi/lo pair
(two bf16 values whose sum carries about 16 mantissa bits).

Sites (each a value the GPU writes to memory and then feeds to an MFMA):
  a_qkv   RMSNorm output entering the Q/K/V projection
  q       rotated queries
  k       rotated keys (the K cache)
  v       values (the V cache)
  p       attention probabilities exp(s - max) entering the P.V product (the normaliser is
          summed from the unrounded values, as the kernels do)
  a_o     attention output entering the output projection
  a_gu    RMSNorm output entering the gate/up projection
  a_down  SwiGLU output entering the down projection
  a_lm    final RMSNorm output entering the lm_head
Each site is either exact (fp64), "bf16" (one round-to-nearest-even bf16 value of the fp32
number) or "pair" (hi = bf16(x), lo = bf16(x - hi); the value used is hi + lo).

This is test infrastructure: it is never used to pass a parity test (the oracle stays exact
fp64); it only explains the precision that the GPU path keeps.

Usage (full LLaDA-8B shape, about 1 minute of fp64 work per experiment on 8 cores):
    python tests/precision_sites.py --workload llada8b --block 0
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
for p in (ROOT, HERE):
    if p not in sys.path:
        sys.path.insert(0, p)

import synth  # noqa: E402
from oracle import model as om  # noqa: E402

SITES = ["a_qkv", "q", "k", "v", "p", "a_o", "a_gu", "a_down", "a_lm"]


def bf16_round(x: np.ndarray) -> np.ndarray:
    """fp64 -> fp32 -> bf16 (round to nearest even), returned as fp64."""
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    b = x32.view(np.uint32).astype(np.uint64)
    r = ((b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000).astype(np.uint32)
    return r.view(np.float32).astype(np.float64)


def pair_round(x: np.ndarray) -> np.ndarray:
    """hi + lo with hi = bf16(x), lo = bf16(x - hi) (x taken as fp32)."""
    x32 = np.asarray(x, dtype=np.float32).astype(np.float64)
    hi = bf16_round(x32)
    lo = bf16_round(x32 - hi)
    return hi + lo


class Experiment:
    """One forward with a site -> rounding mode map ('bf16' | 'pair'; absent = exact)."""

    def __init__(self, name: str, modes: dict):
        self.name = name
        self.modes = modes
        self.h = None

    def site(self, name: str, x: np.ndarray) -> np.ndarray:
        m = self.modes.get(name)
        if m == "bf16":
            return bf16_round(x)
        if m == "pair":
            return pair_round(x)
        return x


def attention_sites(ex: Experiment, q, k, v):
    """oracle attention with the probability site; q [n, H, hd], k/v [L, Hkv, hd]."""
    n, H, hd = q.shape
    group = H // k.shape[1]
    out = np.empty_like(q)
    for j in range(H):
        g = j // group
        s = q[:, j, :] @ k[:, g, :].T / np.sqrt(hd)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        out[:, j, :] = (ex.site("p", p) @ v[:, g, :]) / p.sum(axis=1, keepdims=True)
    return out


def default_experiments():
    """Exact, every site as a pair, every site single bf16, then each site alone."""
    exps = [Experiment("exact", {}),
            Experiment("all pairs", {s: "pair" for s in SITES}),
            Experiment("all bf16", {s: "bf16" for s in SITES})]
    for s in SITES:
        exps.append(Experiment(f"{s} bf16", {s: "bf16"}))
    exps.append(Experiment("k+v bf16", {"k": "bf16", "v": "bf16"}))
    exps.append(Experiment("q+k+v+p bf16", {"q": "bf16", "k": "bf16", "v": "bf16", "p": "bf16"}))
    exps.append(Experiment("GEMM inputs bf16",
                           {"a_qkv": "bf16", "a_o": "bf16", "a_gu": "bf16", "a_down": "bf16"}))
    return exps


def run(cfg: dict, block: int, exps, log=print):
    """Refresh forward of block `block` for batch row 0 under every experiment, in lockstep
    (the weights of a layer are generated once and shared).  Returns the block rows' head
    statistics per experiment."""
    x = synth.block_state_np(cfg, block)[0].astype(np.int64)
    L = len(x)
    d, H, Hkv, hd = cfg["d_model"], cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    eps = cfg["rms_eps"]
    names = synth.configs.weight_names(cfg["n_layers"])

    def W(name):
        return synth.tensor_np(cfg, name).astype(np.float64)

    emb = W("embed")
    for ex in exps:
        ex.h = emb[x].copy()
    del emb
    cos, sin = om.rope_tables(np.arange(L), hd, cfg["rope_base"])
    for l in range(cfg["n_layers"]):
        t0 = time.time()
        p = f"layers.{l}."
        g1, wq, wk, wv, wo = W(p + "attn_norm"), W(p + "wq"), W(p + "wk"), W(p + "wv"), W(p + "wo")
        g2, wg, wu, wd = W(p + "ffn_norm"), W(p + "w_gate"), W(p + "w_up"), W(p + "w_down")
        for ex in exps:
            a = ex.site("a_qkv", om.rms_norm(ex.h, g1, eps))
            q = om.apply_rope((a @ wq.T).reshape(L, H, hd), cos, sin)
            k = om.apply_rope((a @ wk.T).reshape(L, Hkv, hd), cos, sin)
            v = (a @ wv.T).reshape(L, Hkv, hd)
            o = attention_sites(ex, ex.site("q", q), ex.site("k", k), ex.site("v", v))
            ex.h = ex.h + ex.site("a_o", o.reshape(L, H * hd)) @ wo.T
            f = ex.site("a_gu", om.rms_norm(ex.h, g2, eps))
            act = om.silu(f @ wg.T) * (f @ wu.T)
            ex.h = ex.h + ex.site("a_down", act) @ wd.T
        log(f"layer {l} done in {time.time() - t0:.1f}s")
    s = cfg["prompt_len"] + block * cfg["block_size"]
    e = s + cfg["block_size"]
    gf, wlm = W("final_norm"), W("lm_head")
    out = {}
    for ex in exps:
        z = ex.site("a_lm", om.rms_norm(ex.h[s:e], gf, eps))
        out[ex.name] = om.head_stats(z, wlm, cfg["logit_scale"], cfg["mask_id"])
    return out


def summarize(stats: dict) -> list:
    """Per experiment: max and median relative confidence error, max per-row logit error
    (max|dl| / max|l|), and argmax disagreements, against the exact run."""
    ref = stats["exact"]
    fin = np.isfinite(ref["logits"])
    lmax = np.abs(np.where(fin, ref["logits"], 0)).max(axis=1)
    rows = []
    for name, st in stats.items():
        crel = np.abs(st["conf"] - ref["conf"]) / ref["conf"]
        dl = np.where(fin, np.abs(st["logits"] - np.where(fin, ref["logits"], 0)), 0).max(axis=1)
        rows.append(dict(name=name, conf_rel_max=float(crel.max()),
                         conf_rel_median=float(np.median(crel)),
                         logit_rel_max=float((dl / lmax).max()),
                         argmax_diff=int((st["tok"] != ref["tok"]).sum())))
    return rows


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="llada8b")
    ap.add_argument("--block", type=int, default=0)
    ap.add_argument("--layers", type=int, default=0, help="override n_layers (0: the workload's)")
    ap.add_argument("--out", default=None, help="write the table as JSON")
    args = ap.parse_args()
    over = {"n_layers": args.layers} if args.layers else {}
    cfg = synth.configs.get(args.workload, **over)
    t0 = time.time()
    stats = run(cfg, args.block, default_experiments(),
                log=lambda *a: print(*a, file=sys.stderr, flush=True))
    rows = summarize(stats)
    print(f"{cfg['name']} ({cfg['n_layers']} layers, d {cfg['d_model']}), block {args.block}, "
          f"batch row 0, {time.time() - t0:.0f}s")
    print(f"{'sites':24s} {'conf rel max':>13s} {'median':>10s} {'logit rel':>10s} {'argmax':>7s}")
    for r in rows:
        print(f"{r['name']:24s} {r['conf_rel_max']:13.2e} {r['conf_rel_median']:10.2e} "
              f"{r['logit_rel_max']:10.2e} {r['argmax_diff']:7d}")
    if args.out:
        with open(args.out, "w") as f:
            json.dump(dict(workload=cfg["name"], n_layers=cfg["n_layers"], block=args.block,
                           rows=rows), f, indent=1)


if __name__ == "__main__":
    main()
