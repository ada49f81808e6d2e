"""Pins for block-causal decoding in the oracle (Fast-dLLM README track table, v2 "Block
Diffusion"; Streaming-dLLM README, the note on block-causal diffusion models).

Reading: the prompt is one block, the generation blocks of ``block_size``; a query sees its own
block and every block before it.  The oracle refreshes only the previous and the current block
and reuses every other K/V from its cache.

* a pure-Python decode that recomputes every position from scratch at every step, with the
  per-row key limits spelled out, reproduces the oracle's decode in every cache mode;
* the short refresh equals a full block-causal recompute bit for bit;
* positions after the current block are invisible; a finished block's K/V never change again
  after the refresh that follows it.
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
                weight_std=0.5, threshold=0.6, attention="block_causal")
    base.update(kw)
    return synth.configs.get("tiny_f32", **base)


@pytest.mark.parametrize("use_cache", [0, 2])
@pytest.mark.parametrize("threshold", [0.6, 1.5])
def test_block_causal_decode_matches_from_scratch_brute_force(use_cache, threshold):
    cfg = small(use_cache=use_cache, threshold=threshold)
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


def test_short_refresh_equals_full_recompute():
    cfg = small(prompt_len=4, gen_length=12, block_size=4)
    W = synth.weights_np(cfg)
    m = om.Model(cfg, W)
    dec = od.Decoder(m)
    x = synth.block_state_np(cfg, 2)            # blocks 0 and 1 filled, block 2 masked
    dec.set_tokens(x)
    dec.block_begin(0)
    dec.block_begin(1)
    dec.block_begin(2)                          # refreshes blocks 1 and 2 only
    rec, _ = dec.step()
    e = cfg["prompt_len"] + 3 * cfg["block_size"]
    rows = np.arange(e)
    full = m.forward_rows(x[0], rows, rows, m.new_cache(), dec._limits(rows))
    st = m.stats(full[e - cfg["block_size"]:])
    for k in ("tok", "conf", "p2"):
        assert np.array_equal(rec[k][0], st[k])


def test_later_positions_are_invisible_and_finished_blocks_are_final():
    cfg = small(prompt_len=4, gen_length=12, block_size=4, threshold=1.5)
    W = synth.weights_np(cfg)
    L, P, Bs = 16, 4, 4
    x = synth.block_state_np(cfg, 1)
    runs = []
    for later in (cfg["mask_id"], 0):
        y = x.copy()
        y[0, P + 2 * Bs:] = later                # anything after block 1
        dec = od.Decoder(om.Model(cfg, W))
        dec.set_tokens(y)
        dec.block_begin(0)
        dec.block_begin(1)
        recs = [dec.step()[0] for _ in range(2)]
        runs.append((recs, dec))
    for a, b in zip(runs[0][0], runs[1][0]):
        for k in ("tok", "conf", "p2"):
            assert np.array_equal(a[k], b[k])
    # block 0 is final once block 1's refresh has run: block 1's steps leave it alone
    dec = runs[0][1]
    k0 = [c.copy() for c in dec.caches[0][0]]
    while dec.step()[1] is False:
        pass
    for l, c in enumerate(dec.caches[0][0]):
        assert np.array_equal(c[:P + Bs], k0[l][:P + Bs])
