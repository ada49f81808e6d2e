"""Approximate suffix pruning on the GPU against the oracle, through the C ABI (Streaming-dLLM
README, figure caption on approximated suffix pruning).  Needs an MI355X and a built
libdllm.so."""

import numpy as np
import pytest

import synth
from parity import Report, assert_report, oracle_decoder, teacher_forced_block

pytestmark = pytest.mark.gpu


def _handle(cfg, **kw):
    import torch
    from diffusion_block_denoise_amd import dllm
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    W = synth.weights_torch(cfg, device="cuda")
    return dllm.Handle(cfg, W, **kw)


def _log(*a):
    print(*a, flush=True)


def small_bf16(**kw):
    base = dict(n_layers=2, d_model=256, n_heads=8, n_kv_heads=2, head_dim=32, ffn_dim=512,
                vocab=1000, mask_id=999, batch=2, prompt_len=40, gen_length=64, block_size=16,
                use_cache=2, random_gains=True)
    base.update(kw)
    return synth.configs.get("small_bf16", **base)


@pytest.mark.parametrize("window", [0, 6])
def test_tiny_f32_pruned_generate_exact_sequence(window):
    cfg = synth.configs.get("tiny_f32", suffix_window=window)
    _log("case tiny_f32 pruned generate, window", window)
    h = _handle(cfg)
    x_gpu, st = h.generate(synth.prompt_np(cfg))
    x_ref, recs = oracle_decoder(cfg, keep_logits=False).generate(synth.prompt_np(cfg))
    assert np.array_equal(x_gpu, x_ref)
    assert st["steps"] == len(recs)


@pytest.mark.parametrize("variant", [
    dict(suffix_window=0),                                        # dual, GQA 8/2, hd 32, batch 2
    dict(suffix_window=16, use_cache=1, n_kv_heads=4, head_dim=64, n_heads=4),  # prefix, MHA
    dict(suffix_window=5, use_cache=0, head_dim=128, n_heads=2, n_kv_heads=1, batch=1),
    dict(suffix_window=7, batch=3, prompt_len=17),                 # ragged context lengths
])
def test_bf16_pruned_teacher_forced(variant):
    cfg = small_bf16(**variant)
    _log("case bf16 pruned teacher-forced", variant)
    h = _handle(cfg)
    dec = oracle_decoder(cfg)
    rep = Report()
    for b in range(cfg["gen_length"] // cfg["block_size"]):
        teacher_forced_block(cfg, h, dec, synth.block_state_np(cfg, b), b, rep)
    _log(rep)
    assert_report(cfg, rep)


def test_window_reaching_the_end_is_bit_identical_to_no_pruning():
    base = small_bf16(threshold=0.7)
    _log("case window to the end")
    outs = []
    for cfg in (base, dict(base, suffix_window=base["gen_length"])):
        h = _handle(cfg)
        x, st = h.generate(synth.prompt_np(cfg))
        outs.append((x, st["steps"], h.get_step_info()))
    (x0, n0, i0), (x1, n1, i1) = outs
    assert np.array_equal(x0, x1) and n0 == n1
    for k in ("tok", "conf", "p2"):
        assert np.array_equal(i0[k], i1[k])
