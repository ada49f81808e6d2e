"""Seeded synthetic workloads: model shapes and decode knobs (data only, no arithmetic).

The five workloads stand in for the backbones and generation settings that the
pages measure (Dream-7B and LLaDA-1.5 at generation lengths 256 and 512, in the
Streaming-dLLM README's throughput tables), with seeded random-init weights and
uniform random prompts, because trained checkpoints and benchmark datasets are
not available.  The decode knobs follow the Fast-dLLM README Quick Start
(``gen_length``, ``steps``, ``block_size``) and its Dream evaluation command
(``threshold=0.9``, ``use_cache``).

Fields
------
n_layers, d_model, n_heads, n_kv_heads, head_dim, ffn_dim, vocab, mask_id
    Transformer shape.  ``n_heads % n_kv_heads == 0`` (grouped-query attention).
rms_eps, rope_base, logit_scale
    RMSNorm epsilon, rotary base, and the factor applied to the lm_head output.
dtype
    ``"f32"`` or ``"bf16"``: storage type of weights and of the KV cache.
batch, prompt_len, gen_length, block_size
    Decode geometry; the sequence is ``prompt_len + gen_length`` tokens.
steps
    Diffusion step budget (0 means ``gen_length``).
threshold
    Confidence threshold; a masked position commits when its confidence is
    strictly greater.
use_cache
    0 = no cache (full forward every step), 1 = prefix cache, 2 = dual
    (prefix + suffix) cache.
weight_seed, prompt_seed, weight_std
    Generator seeds and the weight standard deviation.
suffix_window, attention
    Approximate suffix pruning window (< 0: whole context); "full" or "block_causal".
exit_steps, exit_floor
    Early exit for converged tokens: a row's block ends once every masked position kept its
    argmax above exit_floor for exit_steps consecutive steps (0: off).
first_threshold
    First-step confidence scheduling: the threshold of a block's first step (< 0: off).
"""

from __future__ import annotations

import copy

NO_CACHE, PREFIX_CACHE, DUAL_CACHE = 0, 1, 2

_COMMON = dict(rms_eps=1e-5, rope_base=10000.0, logit_scale=20.0, steps=0, threshold=0.9,
               weight_seed=1234, prompt_seed=5678, weight_std=0.02, random_gains=False,
               suffix_window=-1, attention="full", exit_steps=0, exit_floor=0.9,
               first_threshold=-1.0)

CONFIGS = {
    # Tiny LLaDA-style model in fp32.
    "tiny_f32": dict(_COMMON, n_layers=2, d_model=128, n_heads=4, n_kv_heads=4, head_dim=32,
                     ffn_dim=344, vocab=512, mask_id=511, dtype="f32", batch=1, prompt_len=32,
                     gen_length=64, block_size=16, use_cache=DUAL_CACHE),
    # Small bf16 model, prefix-only cache.
    "small_bf16": dict(_COMMON, n_layers=8, d_model=1024, n_heads=16, n_kv_heads=16, head_dim=64,
                       ffn_dim=2816, vocab=32000, mask_id=31999, dtype="bf16", batch=1,
                       prompt_len=256, gen_length=256, block_size=32, use_cache=PREFIX_CACHE),
    # LLaDA-8B shape, batch 1, dual cache.
    "llada8b": dict(_COMMON, n_layers=32, d_model=4096, n_heads=32, n_kv_heads=32, head_dim=128,
                    ffn_dim=12288, vocab=126464, mask_id=126336, dtype="bf16", batch=1,
                    prompt_len=512, gen_length=256, block_size=32, use_cache=DUAL_CACHE),
    # Dream-7B (Qwen2.5-7B) shape with grouped-query attention, batch 8.
    "dream7b": dict(_COMMON, n_layers=28, d_model=3584, n_heads=28, n_kv_heads=4, head_dim=128,
                    ffn_dim=18944, vocab=152064, mask_id=151666, dtype="bf16", batch=8,
                    prompt_len=1024, gen_length=512, block_size=32, use_cache=DUAL_CACHE),
    # LLaDA-8B shape at long context and batch 16.
    "llada8b_long": dict(_COMMON, n_layers=32, d_model=4096, n_heads=32, n_kv_heads=32,
                         head_dim=128, ffn_dim=12288, vocab=126464, mask_id=126336, dtype="bf16",
                         batch=16, prompt_len=4096, gen_length=1024, block_size=64,
                         use_cache=DUAL_CACHE),
}

ORDER = ["tiny_f32", "small_bf16", "llada8b", "dream7b", "llada8b_long"]


def get(name: str, **overrides) -> dict:
    """Return a copy of a named workload with ``overrides`` applied."""
    if name not in CONFIGS:
        raise KeyError(f"unknown workload {name!r}; known: {ORDER}")
    cfg = copy.deepcopy(CONFIGS[name])
    cfg["name"] = name
    for k, v in overrides.items():
        if k not in cfg:
            raise KeyError(f"unknown field {k!r}")
        cfg[k] = v
    return cfg


def derived(cfg: dict) -> dict:
    """Sizes that follow from the fields (no method arithmetic)."""
    L = cfg["prompt_len"] + cfg["gen_length"]
    nb = cfg["gen_length"] // cfg["block_size"]
    steps = cfg["steps"] or cfg["gen_length"]
    return dict(L=L, n_blocks=nb, steps=steps)


def weight_names(n_layers: int) -> list[str]:
    """Tensor names in generator order; the index in this list is the tensor id."""
    names = ["embed", "final_norm", "lm_head"]
    for l in range(n_layers):
        names += [f"layers.{l}.{n}" for n in LAYER_TENSORS]
    return names


LAYER_TENSORS = ["attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up", "w_down"]


def weight_shapes(cfg: dict) -> dict[str, tuple[int, ...]]:
    """Shapes in torch ``Linear`` layout ``[out_features, in_features]``."""
    d, H, Hkv, hd, F, V = (cfg["d_model"], cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"],
                           cfg["ffn_dim"], cfg["vocab"])
    shapes = {"embed": (V, d), "final_norm": (d,), "lm_head": (V, d)}
    for l in range(cfg["n_layers"]):
        p = f"layers.{l}."
        shapes.update({p + "attn_norm": (d,), p + "wq": (H * hd, d), p + "wk": (Hkv * hd, d),
                       p + "wv": (Hkv * hd, d), p + "wo": (d, H * hd), p + "ffn_norm": (d,),
                       p + "w_gate": (F, d), p + "w_up": (F, d), p + "w_down": (d, F)})
    return shapes
