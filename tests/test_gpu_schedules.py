"""The schedule rules of the commit on the GPU, through the C ABI, against the oracle: early exit
for converged tokens (exit_steps, exit_floor) and first-step confidence scheduling
(first_threshold).  The fp32 tiny model must reproduce the oracle's decode exactly (tokens, step
count, early exits); bf16 models are teacher-forced step by step."""

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


RULES = [dict(exit_steps=2, exit_floor=0.3),
         dict(exit_steps=3, exit_floor=0.5),
         dict(first_threshold=0.5, steps=32),
         dict(exit_steps=2, exit_floor=0.4, first_threshold=0.7, steps=16)]


@pytest.mark.parametrize("kw", RULES)
def test_tiny_f32_schedule_rules_exact(kw):
    cfg = synth.configs.get("tiny_f32", **kw)
    _log("case tiny_f32 schedule", kw)
    x_gpu, st = _handle(cfg).generate(synth.prompt_np(cfg))
    dec = oracle_decoder(cfg, keep_logits=False)
    x_ref, recs = dec.generate(synth.prompt_np(cfg))
    assert np.array_equal(x_gpu, x_ref)
    assert st["steps"] == len(recs)
    assert st["early_exits"] == dec.early_exits
    if kw.get("exit_steps"):
        assert dec.early_exits > 0          # the rule fires in this decode


def _small_bf16(**kw):
    base = dict(n_layers=2, d_model=256, n_heads=8, n_kv_heads=2, head_dim=32, ffn_dim=512,
                vocab=1000, mask_id=999, batch=3, prompt_len=40, gen_length=64, block_size=16,
                use_cache=2, random_gains=True)
    base.update(kw)
    return synth.configs.get("small_bf16", **base)


@pytest.mark.parametrize("kw", RULES)
def test_bf16_schedule_rules_teacher_forced(kw):
    cfg = _small_bf16(**kw)
    _log("case bf16 schedule teacher-forced", kw)
    h = _handle(cfg)
    dec = oracle_decoder(cfg)
    rep = Report()
    for b in range(cfg["gen_length"] // cfg["block_size"]):
        teacher_forced_block(cfg, h, dec, synth.block_state_np(cfg, b), b, rep)
    _log(rep, "oracle early exits", dec.early_exits)
    assert_report(cfg, rep)


@pytest.mark.parametrize("kw", [dict(exit_steps=1, exit_floor=-1.0), dict(first_threshold=0.0)])
def test_rules_that_always_fire_take_one_step_per_block(kw):
    cfg = _small_bf16(**kw)
    x, st = _handle(cfg).generate(synth.prompt_np(cfg))
    nb = cfg["gen_length"] // cfg["block_size"]
    assert st["steps"] == nb and st["cached_forwards"] == 0
    assert (x[:, cfg["prompt_len"]:] != cfg["mask_id"]).all()
    x0, _ = _handle(_small_bf16(threshold=0.0)).generate(synth.prompt_np(cfg))
    assert np.array_equal(x, x0)
