"""Teacher-forced step comparison of the GPU library against the oracle.

Per step the GPU gets the oracle's token state, so a disagreement cannot cascade.  Bars:
  * logits: per row max|dl| / max|l_ref| <= tol (fp32 1e-4, bf16 2e-2), finite entries;
  * confidence: |dc| <= tol * c_ref;
  * runner-up probability: |dp2| <= tol * max(p2_ref, c_ref);
  * argmax token and commit decisions bit-exact, except where the decision sits on a boundary
    that the tolerance cannot resolve: confidence within 1e-2 of the threshold, a top-2 margin
    (conf - p2) below 1e-2, or, for the floor's pick, another masked position whose
    confidence is within 1e-2 of the last position the floor takes.  The last kind is counted
    on its own (``exempt_floor``) so that it cannot widen the bar unseen.
"""

from __future__ import annotations

import numpy as np

import synth
from oracle import decode as od
from oracle import model as om

EDGE = 1e-2


def tol_for(cfg):
    return 1e-4 if cfg["dtype"] == "f32" else 2e-2


def exempt_masks(cfg, x_before_row, s, conf, p2, k):
    """Block positions whose decision the comparison does not hold to bit-exactness: (threshold
    or top-2 margin boundary, floor-pick tie)."""
    Bs = cfg["block_size"]
    tau = cfg["threshold"]
    masked = x_before_row[s:s + Bs] == cfg["mask_id"]
    ex = (np.abs(conf - tau) < EDGE) | ((conf - p2) < EDGE)
    floor = np.zeros_like(ex)
    idx = np.flatnonzero(masked)
    if idx.size:
        order = sorted(idx, key=lambda i: (-conf[i], i))
        kk = min(k, len(order))
        ck = conf[order[kk - 1]]
        near = masked & (np.abs(conf - ck) < EDGE) & ~(conf > tau + EDGE)
        if near.sum() > 1:
            floor = near & ~ex
    return ex, floor


def exempt_mask(cfg, x_before_row, s, conf, p2, k):
    ex, floor = exempt_masks(cfg, x_before_row, s, conf, p2, k)
    return ex | floor


class Report:
    def __init__(self):
        self.steps = 0
        self.max_logit_rel = 0.0
        self.max_conf_rel = 0.0
        self.max_p2_rel = 0.0
        self.tok_mismatch = 0
        self.commit_mismatch = 0
        self.exempt = 0
        self.exempt_floor = 0
        self.positions = 0

    def __repr__(self):
        return (f"steps={self.steps} logit_rel={self.max_logit_rel:.2e} conf_rel="
                f"{self.max_conf_rel:.2e} p2_rel={self.max_p2_rel:.2e} tok_mis={self.tok_mismatch} "
                f"commit_mis={self.commit_mismatch} exempt={self.exempt}/{self.positions} "
                f"floor_ties={self.exempt_floor}")


def compare_step(cfg, rec, x_before, info, logits_gpu, rep: Report, check_logits=True):
    tol = tol_for(cfg)
    B, Bs = cfg["batch"], cfg["block_size"]
    s = cfg["prompt_len"] + rec["block"] * Bs
    rep.steps += 1
    for b in range(B):
        c_ref, p2_ref = rec["conf"][b], rec["p2"][b]
        k = int(rec["ks"][b]) if "ks" in rec else rec["k"]
        ex_b, ex_f = exempt_masks(cfg, x_before[b], s, c_ref, p2_ref, k)
        ex = ex_b | ex_f
        rep.exempt += int(ex_b.sum())
        rep.exempt_floor += int(ex_f.sum())
        rep.positions += Bs
        crel = np.abs(info["conf"][b] - c_ref) / c_ref
        rep.max_conf_rel = max(rep.max_conf_rel, float(crel.max()))
        p2rel = np.abs(info["p2"][b] - p2_ref) / np.maximum(p2_ref, c_ref)
        rep.max_p2_rel = max(rep.max_p2_rel, float(p2rel.max()))
        tok_bad = (info["tok"][b] != rec["tok"][b]) & ~ex
        rep.tok_mismatch += int(tok_bad.sum())
        com_bad = (info["committed"][b] != rec["committed"][b]) & ~ex
        rep.commit_mismatch += int(com_bad.sum())
        if check_logits and logits_gpu is not None and "logits" in rec:
            lr = rec["logits"][b]
            lg = logits_gpu[b]
            fin = np.isfinite(lr)
            assert np.array_equal(fin, np.isfinite(lg)), "mask column handling differs"
            d = np.where(fin, np.abs(lg - np.where(fin, lr, 0)), 0).max(axis=1)
            rel = d / np.abs(np.where(fin, lr, 0)).max(axis=1)
            rep.max_logit_rel = max(rep.max_logit_rel, float(rel.max()))


def teacher_forced_block(cfg, handle, decoder, x0, block, rep: Report, logits=True,
                         max_steps=None):
    """Run one block on both sides from token state x0, feeding the GPU the oracle's state."""
    decoder.set_tokens(x0)
    handle.set_tokens(x0)
    decoder.block_begin(block)
    handle.block_begin(block)
    n = 0
    while True:
        x_before = decoder.x.copy()
        rec, done = decoder.step()
        handle.denoise_step()
        info = handle.get_step_info()
        lg = handle.debug_block_logits().cpu().numpy() if logits else None
        compare_step(cfg, rec, x_before, info, lg, rep, check_logits=logits)
        handle.set_tokens(decoder.x)
        n += 1
        if done or (max_steps is not None and n >= max_steps):
            return


def assert_report(cfg, rep: Report):
    tol = tol_for(cfg)
    assert rep.max_conf_rel <= tol, rep
    assert rep.max_p2_rel <= tol, rep
    assert rep.max_logit_rel <= tol, rep
    assert rep.tok_mismatch == 0, rep
    assert rep.commit_mismatch == 0, rep


def oracle_decoder(cfg, weights_np=None, keep_logits=True, refresh_every_step=False):
    W = weights_np if weights_np is not None else synth.weights_np(cfg)
    return od.Decoder(om.Model(cfg, W), keep_logits=keep_logits,
                      refresh_every_step=refresh_every_step)
