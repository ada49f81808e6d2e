"""Pins for the oracle's building blocks against library routines, closed forms and invariants.

Each check is chosen so that a plausible slip (dropped term, wrong sign or
index, transposed operand, wrong group mapping) fails it.
"""

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from scipy.special import softmax as sp_softmax

from oracle import model as om

RNG = np.random.default_rng(0)


def test_rms_norm_matches_torch():
    h = RNG.standard_normal((7, 48)) * 3.0
    g = RNG.standard_normal(48)
    ref = F.rms_norm(torch.from_numpy(h), (48,), torch.from_numpy(g), eps=1e-5).numpy()
    assert np.abs(om.rms_norm(h, g, 1e-5) - ref).max() < 1e-12


def test_rms_norm_unit_rms_and_eps():
    h = RNG.standard_normal((5, 64))
    out = om.rms_norm(h, np.ones(64), 0.0)
    assert np.allclose(np.sqrt((out ** 2).mean(-1)), 1.0, atol=1e-14)
    # eps sits inside the square root: a zero row stays zero, a tiny row is damped
    z = om.rms_norm(np.full((1, 4), 1e-4), np.ones(4), 1e-5)
    assert np.allclose(z, 1e-4 / np.sqrt(1e-8 + 1e-5))


def test_silu_matches_torch():
    z = RNG.standard_normal(1000) * 6
    assert np.abs(om.silu(z) - F.silu(torch.from_numpy(z)).numpy()).max() < 1e-14


def _rope_complex(u, positions, base):
    """Rotary embedding as complex multiplication: (u_i + i u_{i+hd/2}) * exp(i p theta_i)."""
    hd = u.shape[-1]
    half = hd // 2
    theta = np.outer(positions, base ** (-np.arange(0, hd, 2) / hd))
    zc = (u[..., :half] + 1j * u[..., half:]) * np.exp(1j * theta)[:, None, :]
    return np.concatenate([zc.real, zc.imag], axis=-1)


@pytest.mark.parametrize("hd", [4, 32, 128])
def test_rope_matches_complex_form(hd):
    pos = np.array([0, 1, 5, 97, 4095])
    u = RNG.standard_normal((5, 3, hd))
    c, s = om.rope_tables(pos, hd, 10000.0)
    assert np.abs(om.apply_rope(u, c, s) - _rope_complex(u, pos, 10000.0)).max() < 1e-12


def test_rope_invariants():
    hd = 64
    u = RNG.standard_normal((1, 2, hd))
    c, s = om.rope_tables(np.array([0]), hd, 10000.0)
    assert np.array_equal(om.apply_rope(u, c, s), u)                       # identity at p = 0
    pos = np.arange(10)
    uu = np.repeat(u, 10, axis=0)
    c, s = om.rope_tables(pos, hd, 10000.0)
    r = om.apply_rope(uu, c, s)
    assert np.allclose(np.linalg.norm(r, axis=-1), np.linalg.norm(uu, axis=-1))  # norm kept
    q = RNG.standard_normal((1, 1, hd))
    k = RNG.standard_normal((1, 1, hd))
    def dot(m, n):
        cm, sm = om.rope_tables(np.array([m]), hd, 10000.0)
        cn, sn = om.rope_tables(np.array([n]), hd, 10000.0)
        return float((om.apply_rope(q, cm, sm) * om.apply_rope(k, cn, sn)).sum())
    # <R_m q, R_n k> depends only on m - n
    assert abs(dot(7, 3) - dot(104, 100)) < 1e-10
    assert abs(dot(3, 7) - dot(0, 4)) < 1e-10
    assert abs(dot(7, 3) - dot(3, 7)) > 1e-6


@pytest.mark.parametrize("H,Hkv", [(4, 4), (4, 2), (7, 1), (8, 2)])
def test_attention_matches_torch_sdpa(H, Hkv):
    nq, L, hd = 5, 11, 16
    q = RNG.standard_normal((nq, H, hd))
    k = RNG.standard_normal((L, Hkv, hd))
    v = RNG.standard_normal((L, Hkv, hd))
    tq = torch.from_numpy(q).permute(1, 0, 2)[None]
    tk = torch.from_numpy(k).permute(1, 0, 2)[None]
    tv = torch.from_numpy(v).permute(1, 0, 2)[None]
    ref = F.scaled_dot_product_attention(tq, tk, tv, is_causal=False, enable_gqa=True)
    ref = ref[0].permute(1, 0, 2).numpy()
    assert np.abs(om.attention(q, k, v) - ref).max() < 1e-12
    # grouped heads equal plain multi-head attention with each K/V head repeated per group
    rep = H // Hkv
    mha = om.attention(q, np.repeat(k, rep, axis=1), np.repeat(v, rep, axis=1))
    assert np.abs(om.attention(q, k, v) - mha).max() < 1e-12


def test_attention_is_key_permutation_invariant():
    q = RNG.standard_normal((3, 2, 8))
    k = RNG.standard_normal((9, 2, 8))
    v = RNG.standard_normal((9, 2, 8))
    perm = RNG.permutation(9)
    assert np.abs(om.attention(q, k, v) - om.attention(q, k[perm], v[perm])).max() < 1e-12


def test_head_stats_matches_softmax_and_excludes_mask():
    n, d, V, mask_id = 6, 16, 40, 39
    z = RNG.standard_normal((n, d))
    w = RNG.standard_normal((V, d)) * 0.3
    st = om.head_stats(z, w, 20.0, mask_id)
    logits = 20.0 * z @ w.T
    assert np.allclose(st["logits"][:, :mask_id], logits[:, :mask_id])
    assert np.all(np.isneginf(st["logits"][:, mask_id]))
    p = sp_softmax(logits[:, :mask_id], axis=1)
    assert np.array_equal(st["tok"], p.argmax(1))
    assert np.allclose(st["conf"], p.max(1), rtol=1e-12)
    ps = np.sort(p, axis=1)
    assert np.allclose(st["p2"], ps[:, -2], rtol=1e-12)


def test_head_stats_mask_never_wins_and_ties_go_low():
    z = np.ones((1, 2))
    w = np.array([[0.0, 0.0], [1.0, 1.0], [1.0, 1.0], [5.0, 5.0]])  # id 3 is the mask and largest
    st = om.head_stats(z, w, 1.0, 3)
    assert st["tok"][0] == 1                       # tie between 1 and 2 goes to the lower id
    assert np.isclose(st["conf"][0], st["p2"][0])  # the runner-up is the tied id
    e = np.exp([0.0, 2.0, 2.0])
    assert np.isclose(st["conf"][0], e[1] / e.sum())
