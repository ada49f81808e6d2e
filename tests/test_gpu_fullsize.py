"""The GPU library at the full sizes of the benchmark workloads, in the launch configuration the
benchmark uses, teacher-forced against the oracle.

* LLaDA-8B shape (batch 1, 768 positions, dual cache): blocks 0, 4 and 7 (the first, a middle
  and the last block: the longest suffix and the longest prefix), the refresh and every cached
  step until the block is committed; block 4 again with early exit for converged tokens and
  first-step confidence scheduling on.
* Dream-7B shape (28/4 grouped heads, batch 8, 1536 positions): the GPU runs all 8 rows; the
  oracle follows batch rows 0 and 7 (rows are independent) at blocks 0, 8 and 15, for the
  refresh and one cached step.
* Long-context LLaDA-8B shape (batch 16, 5120 positions, block 64, the batch-16 refresh of
  81920 rows, the 5120-key refresh attention, the 1024-row cached step):
  - at the full 32-layer depth, batch row 15 at the last block: refresh and two cached steps;
  - with the depth cut to 2 layers (the kernels and their plans depend on the row counts and
    widths, not on the depth), batch rows 0 and 15 at the first and the last block;
  - properties that hold at any size: refresh determinism, batch-row permutation, commits.

The oracle's weights are the generator's values copied from the device tensors; a sample of
every tensor is first checked against the host generator so that they are the same data.
"""

import gc

import numpy as np
import pytest

import synth
from parity import Report, assert_report, compare_step

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _log(*a):
    print(*a, flush=True)


@pytest.fixture(autouse=True)
def _free_device_memory():
    """Each test holds tens of GB of weights and workspace: release them before the next."""
    yield
    import torch
    gc.collect()
    torch.cuda.empty_cache()


def _weights(cfg):
    import torch
    W = synth.weights_torch(cfg, device="cuda")
    torch.cuda.synchronize()
    return W


def _host_weights_checked(cfg, W):
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
        if tid % 36 == 35:
            _log(f"  host weights: {tid + 1}/{len(names)} tensors copied and checked")
    return out


def _teacher_forced(cfg, h, Wh, rows, block, n_steps, rep):
    """Refresh of `block` and up to n_steps steps (None: until the block is committed); the
    oracle follows the batch rows `rows` of the GPU handle and feeds them its token state after
    every step (the other rows run free on the GPU)."""
    from oracle import decode as od
    from oracle import model as om
    rows = list(rows)
    ocfg = dict(cfg, batch=len(rows))

    def progress(layer, n_layers, n_rows):
        if n_rows > 256 and (layer % 4 == 3 or layer == n_layers - 1):
            _log(f"  oracle forward over {n_rows} rows: layer {layer + 1}/{n_layers}")

    dec = od.Decoder(om.Model(ocfg, Wh, progress=progress), keep_logits=True)
    x0 = synth.block_state_np(cfg, block)
    dec.set_tokens(x0[rows])
    h.set_tokens(x0)
    dec.block_begin(block)
    h.block_begin(block)
    j = 0
    while True:
        x_before = dec.x.copy()
        rec, done = dec.step()
        h.denoise_step()
        info = {k: v[rows] for k, v in h.get_step_info().items()}
        lg = h.debug_block_logits()[rows].cpu().numpy()
        compare_step(ocfg, rec, x_before, info, lg, rep)
        _log(f"rows {rows} block {block} step {j}: {rep}")
        xg = h.get_tokens()
        xg[rows] = dec.x
        h.set_tokens(xg)
        j += 1
        if done or (n_steps is not None and j >= n_steps):
            break
    return dec


def _run(cfg, cases, decoders=None):
    """cases: (rows, block, n_steps) each; one handle, one report.  `decoders` (a list) receives
    each case's oracle decoder."""
    from diffusion_block_denoise_amd import dllm
    _log(f"case {cfg['name']} ({cfg['n_layers']} layers): weights")
    W = _weights(cfg)
    h = dllm.Handle(cfg, W)
    Wh = _host_weights_checked(cfg, W)
    rep = Report()
    for rows, block, n_steps in cases:
        dec = _teacher_forced(cfg, h, Wh, rows, block, n_steps, rep)
        if decoders is not None:
            decoders.append(dec)
    h.destroy()
    return rep


def test_llada8b_first_middle_last_blocks():
    cfg = synth.configs.get("llada8b")
    rep = _run(cfg, [((0,), 0, None), ((0,), 4, None), ((0,), 7, None)])
    assert_report(cfg, rep)


@pytest.mark.parametrize("kw,exits", [(dict(exit_steps=2, exit_floor=0.5, first_threshold=0.7), 0),
                                      (dict(threshold=0.999, exit_steps=2, exit_floor=0.0), 1)])
def test_llada8b_schedule_rules_middle_block(kw, exits):
    """Early exit for converged tokens and first-step confidence scheduling at the full LLaDA-8B
    shape: block 4 until it is committed.  With first-step scheduling the block ends in three
    steps, before any run of unchanged argmaxes completes; with threshold 0.999 (two or three
    commits a step) the early exit ends it (`exits`: the oracle's count in this seeded case)."""
    cfg = synth.configs.get("llada8b", **kw)
    decs = []
    rep = _run(cfg, [((0,), 4, None)], decs)
    _log(f"oracle early exits: {decs[0].early_exits}")
    assert_report(cfg, rep)
    assert decs[0].early_exits == exits


def test_dream7b_rows_0_and_7():
    cfg = synth.configs.get("dream7b")
    rep = _run(cfg, [((0, 7), 0, 2), ((0, 7), 8, 2), ((0, 7), 15, 2)])
    assert_report(dict(cfg, batch=2), rep)


def test_long_context_full_depth_last_block():
    cfg = synth.configs.get("llada8b_long")
    nb = cfg["gen_length"] // cfg["block_size"]
    rep = _run(cfg, [((15,), nb - 1, 3)])
    assert_report(dict(cfg, batch=1), rep)


def test_long_context_two_layers_rows_0_and_15():
    cfg = synth.configs.get("llada8b_long", n_layers=2)
    nb = cfg["gen_length"] // cfg["block_size"]
    rep = _run(cfg, [((0, 15), 0, 3), ((0, 15), nb - 1, 3)])
    assert_report(dict(cfg, batch=2), rep)


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
    assert h.get_stats()["nan_count"] == 0
    h.destroy()
