"""The GPU library at the full sizes of the benchmark workloads, in the launch configuration the
benchmark uses.

* LLaDA-8B shape (batch 1, 768 positions, dual cache): one block teacher-forced against the
  oracle for its refresh and two cached steps.
* Dream-7B shape (28/4 grouped heads, batch 8, 1536 positions): the GPU runs all 8 rows; the
  oracle recomputes batch row 0 (rows are independent) for the refresh and one cached step.
* Long-context LLaDA-8B shape (batch 16, 5120 positions, block 64): properties that hold at
  any size (refresh determinism, batch-row permutation equivariance, commit invariants);
  the oracle is too slow for a full forward there.

The oracle's weights are the generator's values copied from the device tensors; a sample of
every tensor is first checked against the host generator so that they are the same data.
"""

import numpy as np
import pytest

import synth
from parity import Report, assert_report, compare_step

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _log(*a):
    print(*a, flush=True)


def _weights(cfg):
    import torch
    W = synth.weights_torch(cfg, device="cuda")
    torch.cuda.synchronize()
    return W


def _host_weights_checked(cfg, W, rows=None):
    """fp32 host copies of the device weights, each spot-checked against the host generator."""
    names = synth.configs.weight_names(cfg["n_layers"])
    out = {}
    rng = np.random.default_rng(0)
    for tid, n in enumerate(names):
        t = W[n].float().cpu().numpy()
        flat = t.reshape(-1)
        if not n.endswith("norm"):
            start = int(rng.integers(0, max(1, flat.size - 4096)))
            cnt = min(4096, flat.size - start)
            table = synth.gen.normal_table(cfg["weight_std"], cfg["dtype"])
            ref = table[(synth.gen.words_np(start, cnt, cfg["weight_seed"], tid) >> np.uint64(16))
                        .astype(np.int64)]
            assert np.array_equal(flat[start:start + cnt], ref), n
        out[n] = t
    return out


def _teacher_forced(cfg, h, dec, block, n_steps, rep, rows=None):
    x0 = synth.block_state_np(cfg, block)
    dec.set_tokens(x0[:dec.B])
    h.set_tokens(x0)
    dec.block_begin(block)
    h.block_begin(block)
    for j in range(n_steps):
        x_before = dec.x.copy()
        rec, done = dec.step()
        h.denoise_step()
        info = h.get_step_info()
        info = {k: v[:dec.B] for k, v in info.items()}
        lg = h.debug_block_logits()[:dec.B].cpu().numpy()
        ocfg = dict(cfg, batch=dec.B)
        compare_step(ocfg, rec, x_before, info, lg, rep)
        _log(f"block {block} step {j}: {rep}")
        xg = h.get_tokens()
        xg[:dec.B] = dec.x
        h.set_tokens(xg)
        if done:
            break


def test_llada8b_teacher_forced_block():
    from diffusion_block_denoise_amd import dllm
    from oracle import decode as od
    from oracle import model as om
    cfg = synth.configs.get("llada8b")
    _log("case llada8b: weights")
    W = _weights(cfg)
    h = dllm.Handle(cfg, W)
    Wh = _host_weights_checked(cfg, W)
    dec = od.Decoder(om.Model(cfg, Wh), keep_logits=True)
    rep = Report()
    _teacher_forced(cfg, h, dec, 3, 3, rep)
    assert_report(cfg, rep)


def test_dream7b_teacher_forced_row0():
    from diffusion_block_denoise_amd import dllm
    from oracle import decode as od
    from oracle import model as om
    cfg = synth.configs.get("dream7b")
    _log("case dream7b: weights")
    W = _weights(cfg)
    h = dllm.Handle(cfg, W)
    Wh = _host_weights_checked(cfg, W)
    ocfg = dict(cfg, batch=1)
    dec = od.Decoder(om.Model(ocfg, Wh), keep_logits=True)
    rep = Report()
    _teacher_forced(cfg, h, dec, 5, 2, rep)
    assert_report(ocfg, rep)


def test_long_context_properties():
    """Batch 16 x 5120 positions x block 64: refresh determinism, row permutation, commits."""
    from diffusion_block_denoise_amd import dllm
    cfg = synth.configs.get("llada8b_long")
    _log("case llada8b_long: weights")
    W = _weights(cfg)
    h = dllm.Handle(cfg, W)
    b = 7
    x0 = synth.block_state_np(cfg, b)
    h.set_tokens(x0)
    h.block_begin(b)
    a = h.get_step_info()
    h.block_begin(b)                      # same state, same refresh: bit-identical
    a2 = h.get_step_info()
    for k in ("tok", "conf", "p2"):
        assert np.array_equal(a[k], a2[k])
    perm = np.random.default_rng(3).permutation(cfg["batch"])
    h.set_tokens(x0[perm])
    h.block_begin(b)
    p = h.get_step_info()
    for k in ("tok", "conf", "p2"):
        assert np.array_equal(p[k], a[k][perm]), k
    _log("permutation ok")
    # a few steps of the block: commits only masked block positions with the step's argmax
    h.set_tokens(x0)
    h.block_begin(b)
    s = cfg["prompt_len"] + b * cfg["block_size"]
    prev = h.get_tokens()
    for _ in range(3):
        n, done = h.denoise_step()
        x = h.get_tokens()
        info = h.get_step_info()
        blk = x[:, s:s + cfg["block_size"]]
        assert np.array_equal(blk[info["committed"]], info["tok"][info["committed"]])
        assert (n >= 1).all() or done
        was = prev != cfg["mask_id"]
        assert np.array_equal(x[was], prev[was])
        assert np.array_equal(x[:, :s], prev[:, :s]) and np.array_equal(
            x[:, s + cfg["block_size"]:], prev[:, s + cfg["block_size"]:])
        prev = x
        if done:
            break
