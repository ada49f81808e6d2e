"""Oracle pins for the two schedule rules of the decode: early exit for converged tokens and
first-step confidence scheduling (oracle/decode.py docstring gives both readings).

* Hand-worked step sequences (tests/golden/schedule_rules.json): the model is replaced by a
  script that reports given argmax tokens and confidences, and the decoder's commits must be
  the ones derived by hand from the rule text.
* Special cases that reduce to known decodes, on the tiny fp32 model: either rule switched off,
  or set so that it can never fire, reproduces the plain decode; an exit after one step with no
  confidence floor, and a first-step threshold of 0, both commit every block in one step, as a
  threshold of 0 does.
"""

import json
import os

import numpy as np
import pytest

import synth
from oracle import decode as od
from oracle import model as om

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = json.load(open(os.path.join(HERE, "golden", "schedule_rules.json")))


class ScriptedModel:
    """Stands in for the transformer: every forward reports the next scripted step's block
    statistics (tokens and confidences), whatever the input."""

    def __init__(self, cfg, steps):
        self.cfg = cfg
        self.steps = list(steps)
        self.calls = 0

    def new_cache(self):
        return None

    def forward_rows(self, x, rows, keys, cache, limits=None):
        return np.zeros((len(rows), 1))

    def stats(self, hidden):
        st = self.steps[self.calls]
        self.calls += 1
        conf = np.array(st["conf"], dtype=np.float64)
        return dict(tok=np.array(st["tok"], dtype=np.int64), conf=conf,
                    p2=np.zeros_like(conf), logits=None)


def scripted_cfg(sc):
    Bs, nb = sc["block_size"], sc["blocks"]
    return dict(batch=1, prompt_len=2, gen_length=Bs * nb, block_size=Bs,
                steps=sc["spb"] * nb, threshold=sc["threshold"], use_cache=2, mask_id=99,
                vocab=100, exit_steps=sc["exit_steps"], exit_floor=sc["exit_floor"],
                first_threshold=sc["first_threshold"])


@pytest.mark.parametrize("sc", GOLDEN["scenarios"], ids=lambda sc: sc["name"])
def test_hand_worked_scenarios(sc):
    cfg = scripted_cfg(sc)
    dec = od.Decoder(ScriptedModel(cfg, sc["steps"]))
    x = np.full((1, cfg["prompt_len"] + cfg["gen_length"]), cfg["mask_id"])
    x[0, :2] = [1, 2]
    dec.set_tokens(x)
    got = []
    for b in range(sc["blocks"]):
        dec.block_begin(b)
        done = False
        while not done:
            rec, done = dec.step()
            got.append(sorted(np.flatnonzero(rec["committed"][0]).tolist()))
    assert got == [st["commit"] for st in sc["steps"]], sc["why"]
    # every committed position took the token that its step reported
    s = cfg["prompt_len"]
    flat = [(b, st) for b, st in enumerate(sc["steps"])]
    assert len(flat) == len(got)
    assert (dec.x[0, s:] != cfg["mask_id"]).all()


def test_run_update_rules():
    masked = np.array([True, True, True, False])
    prev = np.array([4, 4, -1, 7])
    run = np.array([2, 3, 0, 5])
    tok = np.array([4, 5, 6, 7])
    conf = np.array([0.8, 0.8, np.nan, 0.99])
    p2, r2 = od.run_update(masked, tok, conf, prev, run, 0.5)
    assert r2.tolist() == [3, 1, 0, 5]         # same token: +1; new token: 1; NaN: 0; unmasked: kept
    assert p2.tolist() == [4, 5, 6, 7]
    _, r3 = od.run_update(masked, tok, np.array([0.5, 0.51, 0.9, 0.1]), prev, run, 0.5)
    assert r3.tolist() == [0, 1, 1, 5]         # at the floor is not above it


def test_hard_floor_spreads_hard_positions_over_remaining_steps():
    assert [od.hard_floor(3, 3, j) for j in (1, 2)] == [2, 1]
    assert [od.hard_floor(10, 5, j) for j in (1, 2, 3, 4)] == [3, 3, 2, 2]
    assert sum(od.hard_floor(29, 32, j) for j in range(1, 32)) >= 29
    assert od.hard_floor(0, 4, 1) == 1 and od.hard_floor(5, 1, 1) == 5


def _decode(**kw):
    cfg = synth.configs.get("tiny_f32", **kw)
    dec = od.Decoder(om.Model(cfg, synth.weights_np(cfg)))
    x, recs = dec.generate(synth.prompt_np(cfg))
    return x, recs, dec


@pytest.fixture(scope="module")
def plain():
    return _decode()


@pytest.mark.parametrize("kw", [dict(exit_steps=0, first_threshold=-1.0),
                                dict(exit_steps=2, exit_floor=1.0),       # no confidence is above 1
                                dict(exit_steps=1000, exit_floor=0.0),    # runs never get that long
                                dict(first_threshold=0.9)])               # same threshold, 1 per step
def test_rules_that_cannot_fire_reproduce_the_plain_decode(plain, kw):
    x, recs, dec = _decode(**kw)
    assert np.array_equal(x, plain[0])
    assert len(recs) == len(plain[1])
    assert dec.early_exits == 0
    for a, b in zip(recs, plain[1]):
        assert np.array_equal(a["committed"], b["committed"])


@pytest.mark.parametrize("kw", [dict(exit_steps=1, exit_floor=-1.0), dict(first_threshold=0.0)])
def test_rules_that_always_fire_commit_whole_blocks(kw):
    x, recs, _ = _decode(**kw)
    x0, recs0, _ = _decode(threshold=0.0)
    nb = 64 // 16
    assert len(recs) == nb and len(recs0) == nb
    assert np.array_equal(x, x0)


def test_early_exit_shortens_blocks_and_commits_argmax():
    x, recs, dec = _decode(exit_steps=2, exit_floor=0.3)
    _, plain_recs, _ = _decode()
    assert dec.early_exits > 0
    for rec in recs:
        c = rec["committed"][0]
        s = 32 + rec["block"] * 16
        assert np.array_equal(rec["x"][0, s:s + 16][c], rec["tok"][0][c])
        if rec["exited"][0]:
            assert (rec["x"][0, s:s + 16] != 511).all()   # the block is finished by the exit
    assert len(recs) < len(plain_recs)


def test_first_step_threshold_commits_easy_tokens_at_once():
    x, recs, dec = _decode(first_threshold=0.5)
    for rec in recs:
        if rec["j"] == 0:
            easy = rec["conf"][0] > 0.5
            assert rec["committed"][0][easy].all()
