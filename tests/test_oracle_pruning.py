"""Pins for approximate suffix pruning in the oracle (Streaming-dLLM README, figure caption
on approximated suffix pruning; ES-dLLM paper card, Streaming-dLLM abstract).

Reading: while block [s, e) is decoded the model sees only the prefix, the block, the
``suffix_window`` positions after the block and the trailing position L-1, each at its own
rotary position; ``suffix_window < 0`` keeps the whole context.

* the pure-Python reference, which runs the model on the explicitly shortened sequence with
  a cache indexed by that sequence, reproduces the oracle's decode (which keeps a cache by
  position and restricts the rows and keys) in every cache mode;
* a window reaching the end equals no pruning, bit for bit;
* the pruned positions are absent: their token ids do not affect any statistic, while the
  trailing position's does.
"""

import numpy as np
import pytest

import synth
from brute import Brute
from oracle import decode as od
from oracle import model as om


def small(**kw):
    base = dict(n_layers=2, d_model=8, n_heads=2, n_kv_heads=1, head_dim=4, ffn_dim=12, vocab=6,
                mask_id=5, prompt_len=2, gen_length=9, block_size=3, random_gains=True,
                weight_std=0.5, threshold=0.6)
    base.update(kw)
    return synth.configs.get("tiny_f32", **base)


@pytest.mark.parametrize("use_cache", [0, 1, 2])
@pytest.mark.parametrize("window", [0, 1, 3])
def test_pruned_decode_matches_shortened_sequence_brute_force(use_cache, window):
    cfg = small(use_cache=use_cache, suffix_window=window)
    W = synth.weights_np(cfg)
    prompt = synth.prompt_np(cfg)
    x_or, recs = od.Decoder(om.Model(cfg, W)).generate(prompt)
    x_br, steps = Brute(cfg, W).generate(list(prompt[0]))
    assert list(x_or[0]) == x_br
    assert len(recs) == len(steps)
    P, Bs = cfg["prompt_len"], cfg["block_size"]
    for r, s in zip(recs, steps):
        assert (r["block"], r["j"]) == (s["block"], s["j"])
        base = P + r["block"] * Bs
        for i in range(Bs):
            tok, conf, p2 = s["stats"][base + i]
            assert r["tok"][0, i] == tok
            assert abs(r["conf"][0, i] - conf) < 1e-12
            assert abs(r["p2"][0, i] - p2) < 1e-12
        assert sorted(base + np.flatnonzero(r["committed"][0])) == s["chosen"]


def test_active_positions():
    dec = od.Decoder(om.Model(small(suffix_window=1), synth.weights_np(small())))
    L = 11
    assert list(dec.active(0)) == [0, 1, 2, 3, 4, 5, L - 1]        # e = 5: window {5}, tail 10
    assert list(dec.active(1)) == list(range(9)) + [L - 1]          # e = 8: window {8}
    assert list(dec.active(2)) == list(range(L))                    # last block: everything


@pytest.mark.parametrize("use_cache", [1, 2])
def test_window_reaching_the_end_is_no_pruning(use_cache):
    cfg = small(use_cache=use_cache)
    W = synth.weights_np(cfg)
    prompt = synth.prompt_np(cfg)
    _, ref = od.Decoder(om.Model(cfg, W)).generate(prompt)
    _, big = od.Decoder(om.Model(dict(cfg, suffix_window=cfg["gen_length"]), W)).generate(prompt)
    assert len(ref) == len(big)
    for a, b in zip(ref, big):
        for k in ("tok", "conf", "p2", "committed"):
            assert np.array_equal(a[k], b[k])


def _block_stats(cfg, W, x, b):
    dec = od.Decoder(om.Model(cfg, W))
    dec.set_tokens(x)
    dec.block_begin(b)
    out = []
    for _ in range(3):
        rec, done = dec.step()
        out.append((rec["tok"].copy(), rec["conf"].copy()))
        if done:
            break
    return out


def test_pruned_positions_are_absent_and_the_tail_is_present():
    cfg = small(use_cache=2, suffix_window=1, threshold=1.5)  # one commit per step
    W = synth.weights_np(cfg)
    L, P = cfg["prompt_len"] + cfg["gen_length"], cfg["prompt_len"]
    x = np.full((1, L), cfg["mask_id"], dtype=np.int64)
    x[0, :P] = synth.prompt_np(cfg)[0]
    base = _block_stats(cfg, W, x, 0)
    pruned = [p for p in range(L) if p not in (0, 1, 2, 3, 4, 5, L - 1)]
    y = x.copy()
    y[0, pruned] = 0                       # any other ids at the pruned positions
    for (t0, c0), (t1, c1) in zip(base, _block_stats(cfg, W, y, 0)):
        assert np.array_equal(t0, t1) and np.array_equal(c0, c1)
    z = x.copy()
    z[0, L - 1] = 0                        # the trailing position is in the context
    changed = [not np.array_equal(c0, c1) for (_, c0), (_, c1) in zip(base, _block_stats(cfg, W, z, 0))]
    assert any(changed)
