"""The C ABI without a GPU: the library loads, exports every function include/dllm.h declares,
the ctypes structs match the C layout, and the host-only calls reject bad configurations."""

import ctypes as C
import os
import re
import subprocess

import pytest

import synth
from diffusion_block_denoise_amd import dllm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dllm.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dllm_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = dllm.load()
    declared = header_functions()
    assert len(declared) >= 15
    for name in declared:
        assert hasattr(lib, name), name
    assert sorted(dllm.EXPORTS) == declared


def test_struct_layout_matches_header(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text(f"""
#include <stdio.h>
#include <stddef.h>
#include "{HEADER}"
int main(void) {{
  printf("%zu %zu %zu %zu %zu\\n", sizeof(dllm_cfg), offsetof(dllm_cfg, threshold),
         offsetof(dllm_cfg, stream), sizeof(dllm_weights), sizeof(dllm_stats));
  printf("%zu %zu %zu %zu %zu\\n", offsetof(dllm_stats, commits_hist), offsetof(dllm_stats, ms_step),
         offsetof(dllm_cfg, suffix_window), offsetof(dllm_cfg, attention),
         offsetof(dllm_stats, nan_count));
  printf("%zu %zu %zu\\n", offsetof(dllm_cfg, exit_floor), offsetof(dllm_cfg, first_threshold),
         offsetof(dllm_stats, early_exits));
  return 0;
}}
""")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()
    got = [int(v) for v in out]
    want = [C.sizeof(dllm.dllm_cfg), dllm.dllm_cfg.threshold.offset, dllm.dllm_cfg.stream.offset,
            C.sizeof(dllm.dllm_weights), C.sizeof(dllm.dllm_stats),
            dllm.dllm_stats.commits_hist.offset, dllm.dllm_stats.ms_step.offset,
            dllm.dllm_cfg.suffix_window.offset, dllm.dllm_cfg.attention.offset,
            dllm.dllm_stats.nan_count.offset, dllm.dllm_cfg.exit_floor.offset,
            dllm.dllm_cfg.first_threshold.offset, dllm.dllm_stats.early_exits.offset]
    assert got == want


@pytest.mark.parametrize("name", synth.configs.ORDER)
def test_workloads_validate_and_size(name):
    c = dllm.make_cfg(synth.configs.get(name))
    assert dllm.dllm_validate_cfg(c) == 0
    n = dllm.dllm_workspace_bytes(c)
    cfg = synth.configs.get(name)
    L = cfg["prompt_len"] + cfg["gen_length"]
    Lp = (L + 31) // 32 * 32
    # K and V: fp32, or bf16 hi + lo planes: 4 bytes per cached element either way
    kv = 2 * cfg["n_layers"] * cfg["batch"] * cfg["n_kv_heads"] * Lp * cfg["head_dim"] * 4
    # bf16: a copy of every linear weight packed into 128-row panels (rows padded to 128)
    wp = 0
    if cfg["dtype"] == "bf16":
        pad = lambda n: (n + 127) // 128 * 128  # noqa: E731
        d, nq = cfg["d_model"], cfg["n_heads"] * cfg["head_dim"]
        nkv, F = cfg["n_kv_heads"] * cfg["head_dim"], cfg["ffn_dim"]
        per_layer = pad(nq + 2 * nkv) * d + pad(d) * nq + pad(2 * ((F + 63) // 64) * 64) * d + pad(d) * F
        wp = 2 * (cfg["n_layers"] * per_layer + pad(cfg["vocab"]) * d)
    assert kv + wp < n < kv + wp + 40 * 2 ** 30


def test_long_context_workspace_fits_one_gpu():
    n = dllm.dllm_workspace_bytes(dllm.make_cfg(synth.configs.get("llada8b_long")))
    assert 86e9 < n < 200e9     # ~86 GB of K/V (hi/lo pairs) plus activations, within 288 GB


BAD = [
    ("dtype", 7), ("n_layers", 0), ("n_heads", 6), ("head_dim", 48), ("mask_id", 512),
    ("mask_id", -1), ("vocab", 1), ("gen_length", 60), ("block_size", 0), ("block_size", 512),
    ("steps", 6), ("steps", -4), ("use_cache", 3), ("batch", 0), ("prompt_len", -1),
    ("threshold", float("nan")), ("rms_eps", -1.0), ("rope_base", 0.0), ("attention", 2),
    ("exit_steps", -1), ("exit_floor", float("nan")), ("first_threshold", float("nan")),
]


@pytest.mark.parametrize("field,value", BAD)
def test_validate_rejects(field, value):
    cfg = synth.configs.get("tiny_f32")
    c = dllm.make_cfg(cfg)
    setattr(c, field, value)
    assert dllm.dllm_validate_cfg(c) == dllm.DLLM_EINVAL
    with pytest.raises(dllm.DllmError):
        dllm.dllm_workspace_bytes(c)


def test_bf16_requires_64_multiples():
    cfg = synth.configs.get("tiny_f32", dtype="bf16")   # ffn_dim 344 is not a multiple of 64
    assert dllm.dllm_validate_cfg(dllm.make_cfg(cfg)) == dllm.DLLM_EINVAL
    cfg = synth.configs.get("tiny_f32", dtype="bf16", ffn_dim=384)
    assert dllm.dllm_validate_cfg(dllm.make_cfg(cfg)) == 0


def test_create_rejects_without_touching_gpu():
    lib = dllm.load()
    cfg = dllm.make_cfg(synth.configs.get("tiny_f32"))
    h = C.c_void_p()
    w = dllm.dllm_weights()
    assert lib.dllm_create(C.byref(w), C.byref(cfg), None, 0, C.byref(h)) == dllm.DLLM_EINVAL
    assert b"NULL" in lib.dllm_last_error(None)
    assert lib.dllm_create(None, C.byref(cfg), None, 0, None) == dllm.DLLM_EINVAL
    # NULL handle calls fail cleanly
    assert lib.dllm_block_begin(None, 0) == dllm.DLLM_EINVAL
    assert lib.dllm_denoise_step(None, None, None) == dllm.DLLM_EINVAL
    lib.dllm_destroy(None)


def test_steps_knob_accepts_block_multiples():
    cfg = synth.configs.get("tiny_f32", steps=8)      # 4 blocks -> 2 steps per block
    assert dllm.dllm_validate_cfg(dllm.make_cfg(cfg)) == 0
