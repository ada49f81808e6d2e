"""Pins for the oracle's forward pass and cache bookkeeping.

* the full forward equals the same block composed from torch's fp64 library
  routines (linear, rms_norm, scaled_dot_product_attention with grouped heads,
  silu) with rotary embedding written as complex multiplication;
* brute-force pure-Python loops on tiny shapes;
* structural facts: attention is bidirectional, batch rows are independent,
  and a cached forward right after a refresh reproduces the refresh.
"""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import synth
from brute import Brute
from oracle import decode as od
from oracle import model as om


def tiny(**kw):
    base = dict(n_layers=2, d_model=32, n_heads=4, n_kv_heads=2, head_dim=8, ffn_dim=40,
                vocab=50, mask_id=49, prompt_len=6, gen_length=8, block_size=4,
                random_gains=True)
    base.update(kw)
    return synth.configs.get("tiny_f32", **base)


def torch_reference(cfg, W, x):
    """Full no-cache forward composed of torch fp64 library routines."""
    T = {k: torch.from_numpy(np.asarray(v, dtype=np.float64)) for k, v in W.items()}
    d, H, Hkv, hd, eps = (cfg["d_model"], cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"],
                          cfg["rms_eps"])
    L = len(x)
    pos = torch.arange(L, dtype=torch.float64)
    inv = cfg["rope_base"] ** (-torch.arange(0, hd, 2, dtype=torch.float64) / hd)
    rot = torch.polar(torch.ones(L, hd // 2, dtype=torch.float64), torch.outer(pos, inv))

    def rope(u):  # u [L, heads, hd]
        c = torch.complex(u[..., :hd // 2], u[..., hd // 2:]) * rot[:, None, :]
        return torch.cat([c.real, c.imag], dim=-1)

    h = F.embedding(torch.from_numpy(np.asarray(x)), T["embed"])
    for l in range(cfg["n_layers"]):
        p = f"layers.{l}."
        a = F.rms_norm(h, (d,), T[p + "attn_norm"], eps)
        q = rope(F.linear(a, T[p + "wq"]).view(L, H, hd))
        k = rope(F.linear(a, T[p + "wk"]).view(L, Hkv, hd))
        v = F.linear(a, T[p + "wv"]).view(L, Hkv, hd)
        o = F.scaled_dot_product_attention(q.transpose(0, 1)[None], k.transpose(0, 1)[None],
                                           v.transpose(0, 1)[None], is_causal=False,
                                           enable_gqa=True)
        o = o[0].transpose(0, 1).reshape(L, H * hd)
        h = h + F.linear(o, T[p + "wo"])
        f = F.rms_norm(h, (d,), T[p + "ffn_norm"], eps)
        h = h + F.linear(F.silu(F.linear(f, T[p + "w_gate"])) * F.linear(f, T[p + "w_up"]),
                         T[p + "w_down"])
    z = F.rms_norm(h, (d,), T["final_norm"], eps)
    logits = cfg["logit_scale"] * F.linear(z, T["lm_head"])
    return h.numpy(), logits.numpy()


@pytest.mark.parametrize("H,Hkv,dtype", [(4, 4, "f32"), (4, 2, "f32"), (4, 1, "bf16")])
def test_full_forward_matches_torch_composition(H, Hkv, dtype):
    cfg = tiny(n_heads=H, n_kv_heads=Hkv, dtype=dtype)
    W = synth.weights_np(cfg)
    m = om.Model(cfg, W)
    x = synth.prompt_np(dict(cfg, prompt_len=cfg["prompt_len"] + cfg["gen_length"]))[0]
    cache = m.new_cache()
    h = m.forward(x, 0, len(x), cache)
    href, lref = torch_reference(cfg, W, x)
    assert np.abs(h - href).max() < 1e-11 * max(1.0, np.abs(href).max())
    st = m.stats(h)
    lref[:, cfg["mask_id"]] = -np.inf
    fin = np.isfinite(lref)
    assert np.abs(st["logits"][fin] - lref[fin]).max() < 1e-10


@pytest.mark.parametrize("threshold", [0.6, 1.5])
def test_oracle_matches_brute_force_decode(threshold):
    for use_cache in (0, 1, 2):
        cfg = synth.configs.get("tiny_f32", n_layers=2, d_model=8, n_heads=2, n_kv_heads=1,
                                head_dim=4, ffn_dim=12, vocab=6, mask_id=5, prompt_len=2,
                                gen_length=6, block_size=3, use_cache=use_cache,
                                random_gains=True, weight_std=0.5, threshold=threshold)
        W = synth.weights_np(cfg)
        prompt = synth.prompt_np(cfg)
        x_or, recs = od.Decoder(om.Model(cfg, W)).generate(prompt)
        x_br, steps = Brute(cfg, W).generate(list(prompt[0]))
        assert list(x_or[0]) == x_br
        assert len(recs) == len(steps)
        for r, s in zip(recs, steps):
            assert (r["block"], r["j"]) == (s["block"], s["j"])
            P, Bs = cfg["prompt_len"], cfg["block_size"]
            base = P + r["block"] * Bs
            for i in range(Bs):
                tok, conf, p2 = s["stats"][base + i]
                assert r["tok"][0, i] == tok
                assert abs(r["conf"][0, i] - conf) < 1e-12
                assert abs(r["p2"][0, i] - p2) < 1e-12
            assert sorted(base + np.flatnonzero(r["committed"][0])) == s["chosen"]


def test_attention_is_bidirectional():
    """Changing a later token changes the outputs at every earlier position."""
    cfg = tiny()
    m = om.Model(cfg, synth.weights_np(cfg))
    L = cfg["prompt_len"] + cfg["gen_length"]
    x = synth.prompt_np(dict(cfg, prompt_len=L))[0].copy()
    h1 = m.forward(x, 0, L, m.new_cache())
    x[-1] = (x[-1] + 1) % cfg["mask_id"]
    h2 = m.forward(x, 0, L, m.new_cache())
    assert np.all(np.abs(h1[:-1] - h2[:-1]).max(axis=1) > 1e-9)


def test_batch_rows_are_independent():
    cfg = tiny(batch=3)
    W = synth.weights_np(cfg)
    prompt = synth.prompt_np(cfg)
    xb, _ = od.Decoder(om.Model(cfg, W)).generate(prompt)
    for r in range(3):
        c1 = dict(cfg, batch=1)
        x1, _ = od.Decoder(om.Model(c1, W)).generate(prompt[r:r + 1])
        assert np.array_equal(xb[r], x1[0])


@pytest.mark.parametrize("use_cache", [1, 2])
def test_cached_forward_after_refresh_equals_refresh(use_cache):
    """With the cache refreshed from the same tokens, a cached step's rows equal the full forward."""
    cfg = tiny(use_cache=use_cache)
    m = om.Model(cfg, synth.weights_np(cfg))
    L = cfg["prompt_len"] + cfg["gen_length"]
    x = synth.block_state_np(cfg, 1)[0]
    cache = m.new_cache()
    full = m.forward(x, 0, L, cache)
    s = cfg["prompt_len"] + cfg["block_size"]
    stop = L if use_cache == 1 else s + cfg["block_size"]
    part = m.forward(x, s, stop, cache)
    assert np.abs(part - full[s:stop]).max() < 1e-12


def test_cached_rows_see_stale_cache():
    """Rows outside the recomputed range contribute their cached K/V, not fresh ones."""
    cfg = tiny(use_cache=2)
    m = om.Model(cfg, synth.weights_np(cfg))
    L = cfg["prompt_len"] + cfg["gen_length"]
    x = synth.block_state_np(cfg, 0)[0]
    cache = m.new_cache()
    m.forward(x, 0, L, cache)
    x2 = x.copy()
    x2[0] = (x2[0] + 1) % cfg["mask_id"]          # change a prefix token after the refresh
    s = cfg["prompt_len"]
    stale = m.forward(x2, s, s + cfg["block_size"], tuple([a.copy() for a in c] for c in cache))
    fresh = m.forward(x2, 0, L, m.new_cache())[s:s + cfg["block_size"]]
    same = m.forward(x, s, s + cfg["block_size"], tuple([a.copy() for a in c] for c in cache))
    assert np.abs(stale - same).max() < 1e-12     # the cached step cannot see the change
    assert np.abs(stale - fresh).max() > 1e-9
