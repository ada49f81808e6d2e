"""GPU library against the oracle, through the C ABI (teacher-forced per step, and free-running
invariants).  Needs an MI355X and a built libdllm.so."""

import numpy as np
import pytest

import synth
from parity import Report, assert_report, compare_step, oracle_decoder, teacher_forced_block

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
                vocab=1000, mask_id=999, batch=2, prompt_len=40, gen_length=32, block_size=16,
                use_cache=2, random_gains=True)
    base.update(kw)
    return synth.configs.get("small_bf16", **base)


# ------------------------------------------------------------------------------ fp32 tiny model
def test_tiny_f32_generate_exact_sequence():
    cfg = synth.configs.get("tiny_f32")
    _log("case tiny_f32 generate")
    h = _handle(cfg)
    x_gpu, st = h.generate(synth.prompt_np(cfg))
    dec = oracle_decoder(cfg, keep_logits=False)
    x_ref, recs = dec.generate(synth.prompt_np(cfg))
    assert np.array_equal(x_gpu, x_ref)
    assert st["steps"] == len(recs)
    assert st["full_forwards"] == cfg["gen_length"] // cfg["block_size"]


def test_tiny_f32_teacher_forced_all_blocks():
    cfg = synth.configs.get("tiny_f32", random_gains=True)
    _log("case tiny_f32 teacher-forced")
    h = _handle(cfg)
    dec = oracle_decoder(cfg)
    rep = Report()
    for b in range(cfg["gen_length"] // cfg["block_size"]):
        teacher_forced_block(cfg, h, dec, synth.block_state_np(cfg, b), b, rep)
    _log(rep)
    assert_report(cfg, rep)


@pytest.mark.parametrize("kw", [
    dict(prompt_len=0),                                   # no prompt: the first block starts at 0
    dict(prompt_len=0, use_cache=1),
    dict(prompt_len=0, use_cache=0),
    dict(block_size=1, gen_length=8),                     # one position per block
    dict(gen_length=16, block_size=16),                   # a single block
    dict(block_size=64, gen_length=64, use_cache=1),      # the whole generation in one block
    dict(steps=16),                                       # 4 steps per 16-wide block: floor 4
])
def test_tiny_f32_edge_configs_exact(kw):
    """Degenerate shapes of the decode: the GPU's token sequence and step count equal the
    oracle's exactly."""
    cfg = synth.configs.get("tiny_f32", **kw)
    _log("case tiny_f32 edge", kw)
    x_gpu, st = _handle(cfg).generate(synth.prompt_np(cfg))
    dec = oracle_decoder(cfg, keep_logits=False)
    x_ref, recs = dec.generate(synth.prompt_np(cfg))
    assert np.array_equal(x_gpu, x_ref)
    assert st["steps"] == len(recs)
    assert (x_gpu[:, cfg["prompt_len"]:] != cfg["mask_id"]).all()


# ------------------------------------------------------------------------------ bf16
@pytest.mark.parametrize("variant", [
    dict(),                                                  # GQA 8/2, hd 32, dual, batch 2
    dict(use_cache=1, n_kv_heads=4, head_dim=64, n_heads=4),  # prefix cache, hd 64, MHA
    dict(use_cache=0, head_dim=128, n_heads=2, n_kv_heads=1, batch=1),  # no cache, hd 128
    dict(batch=5, block_size=32, gen_length=64, prompt_len=17),  # M = 160 rows, ragged L
    dict(block_size=64, gen_length=64, batch=1, threshold=0.5),  # 64-wide block
    dict(vocab=1001, mask_id=1000),  # vocabulary not a multiple of 4: ragged split-K partials
    dict(prompt_len=0, batch=3),  # no prompt
    dict(block_size=256, gen_length=256, prompt_len=8, batch=1),  # the widest block, one block
    dict(n_heads=16, n_kv_heads=2),  # GQA ratio 8 (q width 512 over d_model 256)
    dict(block_size=1, gen_length=8, batch=1),  # one row in the cached step's GEMMs
])
def test_bf16_teacher_forced(variant):
    cfg = small_bf16(**variant)
    _log("case bf16 teacher-forced", variant)
    h = _handle(cfg)
    dec = oracle_decoder(cfg)
    rep = Report()
    for b in range(cfg["gen_length"] // cfg["block_size"]):
        teacher_forced_block(cfg, h, dec, synth.block_state_np(cfg, b), b, rep)
    _log(rep)
    assert_report(cfg, rep)


def test_small_bf16_workload_teacher_forced():
    """The 8-layer d=1024 vocab-32000 workload, prefix-only cache, blocks 0, 3 and 7."""
    cfg = synth.configs.get("small_bf16")
    _log("case small_bf16 workload")
    h = _handle(cfg)
    dec = oracle_decoder(cfg)
    rep = Report()
    for b in (0, 3, 7):
        teacher_forced_block(cfg, h, dec, synth.block_state_np(cfg, b), b, rep)
        _log("block", b, rep)
    assert_report(cfg, rep)


def test_bf16_split_tail_plans_rows():
    """1536-row refresh (batch 4 x 384 positions, d 2048, ffn 5632): the q/k/v and gate/up GEMMs
    run whole columns XCD by XCD and split the remaining columns K-wise, the down projection
    splits every tile, and the last layer continues with the block rows only.  The refresh
    statistics are bit-exact under a batch-row permutation (every row of a column is summed in
    the same order wherever its tile lands), and batch row 0 is teacher-forced against the
    oracle over one block."""
    cfg = small_bf16(d_model=2048, n_heads=16, n_kv_heads=16, head_dim=128, ffn_dim=5632,
                     vocab=4096, mask_id=4095, batch=4, prompt_len=320, gen_length=64,
                     block_size=32)
    _log("case split-tail plans, batch 4 x 384")
    h = _handle(cfg)
    b = 1
    x0 = synth.block_state_np(cfg, b)
    h.set_tokens(x0)
    h.block_begin(b)
    a = h.get_step_info()
    perm = np.random.default_rng(5).permutation(cfg["batch"])
    h.set_tokens(x0[perm])
    h.block_begin(b)
    p = h.get_step_info()
    for k in ("tok", "conf", "p2"):
        assert np.array_equal(p[k], a[k][perm]), k
    ocfg = dict(cfg, batch=1)
    dec = oracle_decoder(ocfg)
    rep = Report()
    dec.set_tokens(x0[:1])
    h.set_tokens(x0)
    dec.block_begin(b)
    h.block_begin(b)
    for _ in range(cfg["block_size"]):
        x_before = dec.x.copy()
        rec, done = dec.step()
        h.denoise_step()
        info = {k: v[:1] for k, v in h.get_step_info().items()}
        lg = h.debug_block_logits()[:1].cpu().numpy()
        compare_step(ocfg, rec, x_before, info, lg, rep)
        xg = h.get_tokens()
        xg[:1] = dec.x
        h.set_tokens(xg)
        if done:
            break
    _log(rep)
    assert_report(ocfg, rep)


# ------------------------------------------------------------------------------ invariants
def test_threshold_above_one_commits_one_per_step():
    cfg = small_bf16(threshold=1.5)
    h = _handle(cfg)
    x, st = h.generate(synth.prompt_np(cfg))
    assert st["steps"] == cfg["gen_length"]
    assert st["commits_hist"][1] == cfg["gen_length"] * cfg["batch"]
    assert (x[:, cfg["prompt_len"]:] != cfg["mask_id"]).all()


def test_threshold_zero_commits_whole_block():
    cfg = small_bf16(threshold=0.0)
    h = _handle(cfg)
    x, st = h.generate(synth.prompt_np(cfg))
    nb = cfg["gen_length"] // cfg["block_size"]
    assert st["steps"] == nb and st["cached_forwards"] == 0
    assert st["committed"] == cfg["gen_length"] * cfg["batch"]


def test_refresh_every_step_equals_no_cache():
    cfg2 = small_bf16(use_cache=2, threshold=0.9)
    cfg0 = small_bf16(use_cache=0, threshold=0.9)
    xa, sa = _handle(cfg2, refresh_every_step=True).generate(synth.prompt_np(cfg2))
    xb, sb = _handle(cfg0).generate(synth.prompt_np(cfg0))
    assert np.array_equal(xa, xb)
    assert sa["steps"] == sb["steps"]


def test_commits_are_never_revised_and_write_argmax():
    cfg = small_bf16(threshold=0.7, batch=3)
    h = _handle(cfg)
    h.prefill(synth.prompt_np(cfg))
    P, Bs, mask = cfg["prompt_len"], cfg["block_size"], cfg["mask_id"]
    prev = h.get_tokens()
    total = 0
    for b in range(cfg["gen_length"] // Bs):
        if b:
            h.block_begin(b)
        done = False
        while not done:
            n, done = h.denoise_step()
            total += 1
            x = h.get_tokens()
            info = h.get_step_info()
            was = prev != mask
            assert np.array_equal(x[was], prev[was])
            s = P + b * Bs
            assert np.array_equal(x[:, s:s + Bs][info["committed"]], info["tok"][info["committed"]])
            assert (n == info["committed"].sum(axis=1)).all()
            assert (x[:, s + Bs:] == mask).all()
            prev = x
    assert total <= cfg["gen_length"]
    assert (prev[:, P:] != mask).all()


def test_deterministic_repeat():
    cfg = small_bf16(batch=5, block_size=32, gen_length=64)
    h = _handle(cfg)
    xa, _ = h.generate(synth.prompt_np(cfg))
    xb, _ = h.generate(synth.prompt_np(cfg))
    assert np.array_equal(xa, xb)


def test_call_order_errors():
    from diffusion_block_denoise_amd import dllm
    cfg = small_bf16()
    h = _handle(cfg)
    with pytest.raises(dllm.DllmError) as e:
        h.block_begin(0)
    assert e.value.code == dllm.DLLM_ESTATE
    with pytest.raises(dllm.DllmError) as e:
        h.denoise_step()
    assert e.value.code == dllm.DLLM_ESTATE
    bad = synth.prompt_np(cfg).copy()
    bad[0, 0] = cfg["vocab"]
    with pytest.raises(dllm.DllmError) as e:
        h.prefill(bad)
    assert e.value.code == dllm.DLLM_EINVAL


def test_profiling_counts_launches():
    from diffusion_block_denoise_amd import dllm
    cfg = small_bf16(batch=5, block_size=32, gen_length=64)   # M = 160: tiled GEMM at refresh
    h = _handle(cfg)
    h.set_profiling((1 << dllm.DLLM_KC_COUNT) - 1)
    _, st = h.generate(synth.prompt_np(cfg))
    prof = h.get_profile()
    L = cfg["n_layers"]
    fwd = st["full_forwards"] + st["cached_forwards"]
    assert prof["attention"]["launches"] == L * fwd
    # 4 GEMMs per layer and the lm_head per forward; every row count here is above 64
    assert prof["gemm_tiled"]["launches"] == (4 * L + 1) * fwd
    assert prof["gemm_skinny"]["launches"] == 0
    for k in ("attention", "gemm_tiled"):
        assert prof[k]["ms"] > 0 and prof[k]["bytes"] > 0 and prof[k]["flops"] > 0
    h.set_profiling(0)
    assert h.get_profile()["attention"]["launches"] == 0


# ------------------------------------------------------------------------------ resume
@pytest.mark.parametrize("name", ["tiny_f32", "bf16"])
def test_resume_after_destroy_is_identical(name):
    """Checkpoint / resume: the decode state is the token state plus the block index, and the
    cache is a function of the token state at a block start.  A run stopped after two blocks,
    its handle destroyed, and resumed on a new handle from dllm_set_tokens + dllm_block_begin
    ends with the same tokens as an uninterrupted run."""
    cfg = synth.configs.get("tiny_f32") if name == "tiny_f32" else small_bf16(
        batch=3, gen_length=64, block_size=16, threshold=0.7)
    prompt = synth.prompt_np(cfg)
    nb = cfg["gen_length"] // cfg["block_size"]
    h = _handle(cfg)
    x_full, st_full = h.generate(prompt)
    h.destroy()

    def run_blocks(hh, blocks, begun):
        """Steps through `blocks`; the first one's refresh has already run (`begun`)."""
        steps = 0
        for i, b in enumerate(blocks):
            if i or not begun:
                hh.block_begin(b)
            done = False
            while not done:
                _, done = hh.denoise_step()
                steps += 1
        return steps

    h1 = _handle(cfg)
    h1.prefill(prompt)
    s1 = run_blocks(h1, [0, 1], begun=True)
    x_mid = h1.get_tokens()
    assert h1.get_position()[0] == 1
    h1.destroy()
    h2 = _handle(cfg)
    h2.set_tokens(x_mid)
    h2.block_begin(2)
    assert h2.get_position() == (2, 0)
    s2 = run_blocks(h2, list(range(2, nb)), begun=True)
    assert np.array_equal(h2.get_tokens(), x_full)
    assert s1 + s2 == st_full["steps"]
    assert h2.get_stats()["nan_count"] == 0


def test_stats_reset_by_prefill_and_gpu_times():
    """dllm_prefill resets the counters; the phase times are GPU times that add up."""
    cfg = small_bf16(batch=2, gen_length=64, block_size=16)
    h = _handle(cfg)
    _, st = h.generate(synth.prompt_np(cfg))
    h.prefill(synth.prompt_np(cfg))
    st2 = h.get_stats()
    assert st2["steps"] == 0 and st2["committed"] == 0 and st2["full_forwards"] == 1
    assert st2["ms_refresh"] > 0 and st2["ms_step"] == 0
    nb = cfg["gen_length"] // cfg["block_size"]
    assert st["full_forwards"] == nb and st["ms_refresh"] > 0 and st["ms_step"] > 0
    assert st["nan_count"] == 0
