"""Pins for the oracle's commit rule, step schedule and cache policy.

The invariants come from the method itself: a threshold above 1 leaves only
the one-per-step floor (gen_length steps); a threshold of 0 commits a whole
block per step; commits are never revised; each commit writes that step's
argmax; the mask id is never committed; refreshing the cache every step is
exactly no-cache decoding; the first step of a block does not depend on the
cache mode.
"""

import itertools
import json
import os

import numpy as np
import pytest

import synth
from oracle import decode as od
from oracle import model as om

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def small(**kw):
    base = dict(n_layers=2, d_model=32, n_heads=4, n_kv_heads=2, head_dim=8, ffn_dim=40,
                vocab=50, mask_id=49, prompt_len=6, gen_length=12, block_size=4)
    base.update(kw)
    return synth.configs.get("tiny_f32", **base)


def run(cfg, refresh_every_step=False):
    m = om.Model(cfg, synth.weights_np(cfg))
    d = od.Decoder(m, refresh_every_step=refresh_every_step)
    x, recs = d.generate(synth.prompt_np(cfg))
    return x, recs, d


# ----------------------------------------------------------------------------- commit rule
def _rule_by_enumeration(masked, conf, tau, k):
    """Smallest subset of the masked positions that holds every position above the threshold
    and is closed under 'more confident (ties: lower position)', with at least min(k, |M|)
    members."""
    M = [i for i in range(len(masked)) if masked[i]]
    best = None
    for r in range(len(M) + 1):
        for S in itertools.combinations(M, r):
            S = set(S)
            if any(conf[i] > tau and i not in S for i in M):
                continue
            if len(S) < min(k, len(M)):
                continue
            closed = all(j in S for i in S for j in M
                         if (conf[j], -j) > (conf[i], -i))
            if closed and (best is None or len(S) < len(best)):
                best = S
    return best


def test_commit_set_matches_enumeration():
    rng = np.random.default_rng(1)
    for _ in range(300):
        n = int(rng.integers(1, 7))
        masked = rng.random(n) < 0.7
        conf = np.round(rng.random(n), 1)          # rounding makes ties common
        tau = float(rng.choice([0.0, 0.5, 0.9, 1.5]))
        k = int(rng.integers(1, 4))
        got = set(np.flatnonzero(od.commit_set(masked, conf, tau, k)))
        assert got == _rule_by_enumeration(masked, conf, tau, k)


def test_commit_set_edge_cases():
    m = np.array([True, True, True])
    assert not od.commit_set(np.zeros(3, bool), np.ones(3), 0.0, 1).any()
    # ties go to the lower position
    assert list(od.commit_set(m, np.array([0.5, 0.5, 0.5]), 0.9, 1)) == [True, False, False]
    # strictly greater than the threshold
    assert list(od.commit_set(m, np.array([0.9, 0.2, 0.1]), 0.9, 1)) == [True, False, False]
    assert list(od.commit_set(m, np.array([0.9, 0.95, 0.1]), 0.9, 1)) == [False, True, False]
    # NaN confidence ranks last and never clears the threshold
    got = od.commit_set(m, np.array([np.nan, 0.3, 0.2]), 0.1, 1)
    assert list(got) == [False, True, True]
    assert list(od.commit_set(m, np.array([np.nan, np.nan, np.nan]), 0.1, 1)) == [True, False, False]
    # floor larger than the masked count commits all of them
    assert od.commit_set(m, np.array([0.1, 0.2, 0.3]), 0.9, 5).all()


def test_floor_schedule_spreads_block_over_its_steps():
    for Bs in (1, 2, 5, 16, 32, 64):
        for spb in range(1, Bs + 1):
            ks = [od.floor_count(Bs, spb, j) for j in range(spb)]
            assert sum(ks) == Bs and max(ks) - min(ks) <= 1
    assert od.steps_per_block(256, 32, 0) == 32           # default steps = gen_length
    with pytest.raises(ValueError):
        od.steps_per_block(100, 32, 0)
    with pytest.raises(ValueError):
        od.steps_per_block(64, 16, 6)


def test_quickstart_knobs():
    """The Quick Start chat command's knobs give one commit floor per step."""
    with open(os.path.join(GOLDEN, "quickstart_knobs.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        spb = od.steps_per_block(case["gen_length"], case["block_size"], case["steps"])
        assert spb == case["steps_per_block"]
        assert [od.floor_count(case["block_size"], spb, j) for j in range(3)] == case["floor_first3"]


# ----------------------------------------------------------------------------- decode invariants
def _check_common(cfg, x, recs):
    P, G, Bs, mask = cfg["prompt_len"], cfg["gen_length"], cfg["block_size"], cfg["mask_id"]
    assert len(recs) <= G
    assert (x[:, P:] != mask).all()
    prev = None
    for r in recs:
        s = P + r["block"] * Bs
        blk = r["x"][:, s:s + Bs]
        # every commit wrote that step's argmax, never the mask id
        assert np.array_equal(blk[r["committed"]], r["tok"][r["committed"]])
        assert (r["tok"] != mask).all()
        if prev is not None:
            # a committed token never changes or reverts to the mask
            was = prev != mask
            assert np.array_equal(r["x"][was], prev[was])
        # the set holds the most confident masked position
        before = prev if prev is not None else None
        prev = r["x"]


def test_threshold_above_one_commits_exactly_one_per_step():
    cfg = small(threshold=1.5)
    x, recs, _ = run(cfg)
    assert len(recs) == cfg["gen_length"]
    assert all(int(r["committed"].sum()) == 1 for r in recs)
    for r in recs:   # the one commit is the most confident masked position (ties: lowest)
        i = int(np.flatnonzero(r["committed"][0])[0])
        s = cfg["prompt_len"] + r["block"] * cfg["block_size"]
        prev_x = r["x"][0].copy()
        prev_x[s + i] = cfg["mask_id"]
        masked = np.flatnonzero(prev_x[s:s + cfg["block_size"]] == cfg["mask_id"])
        order = sorted(masked, key=lambda t: (-r["conf"][0, t], t))
        assert order[0] == i
    _check_common(cfg, x, recs)


def test_threshold_zero_commits_whole_block_per_step():
    cfg = small(threshold=0.0, batch=2)
    x, recs, _ = run(cfg)
    nb = cfg["gen_length"] // cfg["block_size"]
    assert len(recs) == nb
    assert all(r["committed"].all() for r in recs)
    for r in recs:
        s = cfg["prompt_len"] + r["block"] * cfg["block_size"]
        assert np.array_equal(x[:, s:s + cfg["block_size"]], r["tok"])
    _check_common(cfg, x, recs)


@pytest.mark.parametrize("use_cache", [0, 1, 2])
def test_default_threshold_invariants(use_cache):
    cfg = small(threshold=0.9, use_cache=use_cache, batch=2, weight_std=0.08)
    x, recs, _ = run(cfg)
    _check_common(cfg, x, recs)
    for r in recs:
        for b in range(cfg["batch"]):
            c = r["committed"][b]
            if c.any():  # the most confident of the positions committed or still masked
                s = cfg["prompt_len"] + r["block"] * cfg["block_size"]
                cand = c | (r["x"][b, s:s + cfg["block_size"]] == cfg["mask_id"])
                top = max(np.flatnonzero(cand), key=lambda t: (r["conf"][b, t], -t))
                assert c[top]


def test_refresh_every_step_equals_no_cache_exactly():
    a = run(small(use_cache=2, weight_std=0.08), refresh_every_step=True)
    b = run(small(use_cache=0, weight_std=0.08))
    assert np.array_equal(a[0], b[0])
    assert len(a[1]) == len(b[1])
    for ra, rb in zip(a[1], b[1]):
        for key in ("tok", "conf", "p2", "committed", "x"):
            assert np.array_equal(ra[key], rb[key])


def test_first_step_of_block_independent_of_cache_mode():
    outs = []
    for uc in (0, 1, 2):
        cfg = small(use_cache=uc)
        d = od.Decoder(om.Model(cfg, synth.weights_np(cfg)))
        d.set_tokens(synth.block_state_np(cfg, 1))
        d.block_begin(1)
        rec, _ = d.step()
        outs.append(rec)
    for r in outs[1:]:
        for key in ("tok", "conf", "p2", "committed"):
            assert np.array_equal(r[key], outs[0][key])


def test_cache_modes_differ_after_first_step():
    """Stale cached K/V make later steps differ from no-cache decoding (the approximation)."""
    cfg0 = small(use_cache=0, weight_std=0.08)
    cfg2 = small(use_cache=2, weight_std=0.08)
    ra = run(cfg0)[1]
    rb = run(cfg2)[1]
    diffs = [np.abs(a["conf"] - b["conf"]).max() for a, b in zip(ra, rb) if a["j"] > 0]
    assert diffs and max(diffs) > 1e-9


def test_init_reading_spreads_confidence():
    """Weights of standard deviation 0.02 with logits x20 spread the tiny model's max-probs
    from about 0.3 up to about 1.0 over its decode; a variance reading (std 0.141) would not."""
    cfg = synth.configs.get("tiny_f32")
    _, recs, _ = run(cfg)
    c = np.concatenate([r["conf"].ravel() for r in recs])
    assert np.percentile(c, 10) < 0.35 and np.percentile(c, 90) > 0.85
    assert c.min() < 0.3 and c.max() > 0.95
    _, recs2, _ = run(synth.configs.get("tiny_f32", weight_std=0.141))
    c2 = np.concatenate([r["conf"].ravel() for r in recs2])
    assert np.percentile(c2, 10) > 0.5
