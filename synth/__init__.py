"""Seeded synthetic inputs shared by the oracle and the GPU path (data only).

``synth.configs`` names the workloads; ``synth.gen`` is the counter-based
generator; this module assembles whole weight sets, prompts and block-start
token states from them.  Nothing here computes any step of the decoding method.
"""

from __future__ import annotations

import numpy as np

from . import configs, gen

__all__ = ["configs", "gen", "weights_np", "weights_torch", "prompt_np", "prompt_torch",
           "block_state_np", "tensor_np", "GAIN_STD"]

GAIN_STD = 0.1  # spread of norm gains when a workload asks for random gains


def _kind(name: str) -> str:
    return "gain" if name.endswith("norm") else "matrix"


def tensor_np(cfg: dict, name: str) -> np.ndarray:
    """One weight tensor as fp32 values (bf16-representable for bf16 workloads)."""
    names = configs.weight_names(cfg["n_layers"])
    tid = names.index(name)
    shape = configs.weight_shapes(cfg)[name]
    if _kind(name) == "gain":
        if not cfg.get("random_gains"):
            return np.ones(shape, dtype=np.float32)
        g = np.float32(1.0) + gen.normal_np(shape, cfg["weight_seed"], tid, GAIN_STD, "f32")
        if cfg["dtype"] == "bf16":
            g = gen.bf16_bits_to_f32(gen.f32_to_bf16_bits(g))
        return g.astype(np.float32)
    return gen.normal_np(shape, cfg["weight_seed"], tid, cfg["weight_std"], cfg["dtype"])


def weights_np(cfg: dict) -> dict[str, np.ndarray]:
    return {n: tensor_np(cfg, n) for n in configs.weight_names(cfg["n_layers"])}


def weights_torch(cfg: dict, device="cuda", progress=None) -> dict:
    """The same tensors as :func:`weights_np`, in the storage dtype, on ``device``."""
    import torch
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32}[cfg["dtype"]]
    names = configs.weight_names(cfg["n_layers"])
    shapes = configs.weight_shapes(cfg)
    out = {}
    for tid, name in enumerate(names):
        shape = shapes[name]
        if _kind(name) == "gain":
            if cfg.get("random_gains"):
                g = 1.0 + gen.normal_torch(shape, cfg["weight_seed"], tid, GAIN_STD, "f32", device)
                out[name] = g.to(tdt)
            else:
                out[name] = torch.ones(shape, dtype=tdt, device=device)
        else:
            out[name] = gen.normal_torch(shape, cfg["weight_seed"], tid, cfg["weight_std"],
                                         cfg["dtype"], device)
        if progress is not None:
            progress(tid, len(names), name)
    return out


def prompt_np(cfg: dict) -> np.ndarray:
    """Prompt ids uniform in [0, mask_id), shape [batch, prompt_len]."""
    return gen.tokens_np((cfg["batch"], cfg["prompt_len"]), cfg["prompt_seed"], 0, cfg["mask_id"])


def prompt_torch(cfg: dict, device="cpu"):
    return gen.tokens_torch((cfg["batch"], cfg["prompt_len"]), cfg["prompt_seed"], 0,
                            cfg["mask_id"], device)


def block_state_np(cfg: dict, block: int) -> np.ndarray:
    """Token state at the start of ``block``: prompt, uniform ids for earlier blocks, masks after.

    Used to start a teacher-forced comparison at a later block without decoding
    the earlier ones.
    """
    B, P, G, Bs = cfg["batch"], cfg["prompt_len"], cfg["gen_length"], cfg["block_size"]
    x = np.full((B, P + G), cfg["mask_id"], dtype=np.int32)
    x[:, :P] = prompt_np(cfg)
    filled = gen.tokens_np((B, G), cfg["prompt_seed"], 1, cfg["mask_id"])
    x[:, P:P + block * Bs] = filled[:, :block * Bs]
    return x
