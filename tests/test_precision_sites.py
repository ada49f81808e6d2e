"""The precision diagnostic (tests/precision_sites.py) on a small model: the hi/lo pairs that the
GPU path stores keep the step statistics at fp32-like accuracy, a single bf16 value at every site
does not.  The full-size table (LLaDA-8B shape, every site on its own) is produced by running the
script itself; it takes about 25 minutes of fp64 work on 8 cores."""

import precision_sites as ps
import synth


def test_pairs_keep_fp32_accuracy_and_single_bf16_does_not():
    cfg = synth.configs.get("small_bf16", n_layers=2)
    exps = [ps.Experiment("exact", {}),
            ps.Experiment("all pairs", {s: "pair" for s in ps.SITES}),
            ps.Experiment("all bf16", {s: "bf16" for s in ps.SITES})]
    rows = {r["name"]: r for r in ps.summarize(ps.run(cfg, 0, exps, log=lambda *a: None))}
    assert rows["exact"]["conf_rel_max"] == 0.0
    assert rows["all pairs"]["conf_rel_max"] < 1e-3
    assert rows["all bf16"]["conf_rel_max"] > 2e-2


def test_rounding_helpers():
    import numpy as np
    x = np.array([1.0 + 2.0 ** -8 + 2.0 ** -10, -3.0, 1e-3, 0.0])
    b = ps.bf16_round(x)
    # 8 significant bits: 1 + 2^-8 + 2^-10 rounds up to 1 + 2^-7 (above the halfway point)
    assert b[0] == 1.0 + 2.0 ** -7 and b[1] == -3.0 and b[3] == 0.0
    assert abs(b[2] - 1e-3) <= 1e-3 * 2.0 ** -8
    p = ps.pair_round(x)
    assert np.all(np.abs(p - x.astype(np.float32)) <= np.abs(x) * 2.0 ** -16)
