"""Oracle forward pass: LLaDA/Dream-style bidirectional transformer in fp64 NumPy.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What it follows
---------------
* The backbones are the bidirectional diffusion LLMs Dream and LLaDA (Fast-dLLM
  README, track table, "Backbone: Dream, LLaDA"; ES-dLLM paper card, first
  abstract: dLLMs rely on bidirectional attention).  Every query attends to
  every key: there is no causal mask.
* A pre-norm block: RMSNorm, Q/K/V projections, rotary position embedding
  (rotate-half form, base 10^4), attention with grouped K/V heads, output
  projection plus residual, RMSNorm, SwiGLU feed-forward plus residual.  The
  pages do not spell the block out; this is the plainest LLaDA/Dream-style
  reading (no biases, untied embedding and lm_head).
* The KV cache: K (after rotation) and V of every position and layer are kept
  and reused for positions that a step does not recompute (Fast-dLLM README
  track table, "KV Cache + Parallel Decoding"; "Fast-dLLM: Four Acceleration
  Tracks ...", section "The v1 Mechanism").  A forward over a row set R writes
  the K/V of rows R into the cache and lets every query in R attend to all
  cached positions.
* The step's per-position statistics are those of a softmax over the scaled
  lm_head logits with the mask id excluded: argmax token, its probability
  (the confidence) and the runner-up's probability.

Conventions: weights are in torch ``Linear`` layout ``[out, in]``, so a
projection is ``a @ W.T``.  Arrays are fp64.
"""

from __future__ import annotations

import numpy as np

__all__ = ["rms_norm", "rope_tables", "apply_rope", "attention", "attention_limited", "silu",
           "swiglu_ffn", "head_stats", "Model"]


def rms_norm(h: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """h / sqrt(mean(h^2 over the last axis) + eps) * g."""
    ms = np.mean(h * h, axis=-1, keepdims=True)
    return h / np.sqrt(ms + eps) * g


def rope_tables(positions: np.ndarray, head_dim: int, base: float):
    """cos and sin of theta[p, i] = p * base^(-2i/head_dim), i < head_dim/2, shape [n, head_dim/2]."""
    half = head_dim // 2
    i = np.arange(half, dtype=np.float64)
    inv_freq = base ** (-2.0 * i / head_dim)
    theta = np.asarray(positions, dtype=np.float64)[:, None] * inv_freq[None, :]
    return np.cos(theta), np.sin(theta)


def apply_rope(u: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate-half rotary embedding of u [n, heads, head_dim] at the positions of cos/sin [n, hd/2].

    The pair (u_i, u_{i+hd/2}) is rotated by theta_i:
    (u_i cos - u_{i+hd/2} sin, u_{i+hd/2} cos + u_i sin).
    """
    half = u.shape[-1] // 2
    a, b = u[..., :half], u[..., half:]
    c, s = cos[:, None, :], sin[:, None, :]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Non-causal attention with grouped K/V heads.

    q [nq, H, hd]; k, v [L, Hkv, hd]; query head j reads K/V head j // (H / Hkv).
    Returns [nq, H, hd] = softmax(q k^T / sqrt(hd)) v per head, over all L keys.
    """
    nq, H, hd = q.shape
    Hkv = k.shape[1]
    group = H // Hkv
    out = np.empty_like(q)
    for j in range(H):
        g = j // group
        s = q[:, j, :] @ k[:, g, :].T / np.sqrt(hd)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        out[:, j, :] = p @ v[:, g, :]
    return out


def attention_limited(q: np.ndarray, k: np.ndarray, v: np.ndarray, key_pos, limits) -> np.ndarray:
    """attention() where query i sees only the keys whose position is below limits[i].

    q [nq, H, hd]; k, v [nk, Hkv, hd] at positions key_pos [nk]; limits [nq].
    """
    nq, H, hd = q.shape
    Hkv = k.shape[1]
    group = H // Hkv
    key_pos = np.asarray(key_pos)
    out = np.empty_like(q)
    for i in range(nq):
        sel = key_pos < limits[i]
        for j in range(H):
            g = j // group
            s = q[i, j, :] @ k[sel, g, :].T / np.sqrt(hd)
            p = np.exp(s - s.max())
            out[i, j, :] = (p / p.sum()) @ v[sel, g, :]
    return out


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def swiglu_ffn(f, w_gate, w_up, w_down):
    """(silu(f Wg^T) * (f Wu^T)) Wd^T."""
    return (silu(f @ w_gate.T) * (f @ w_up.T)) @ w_down.T


def head_stats(z: np.ndarray, w_lm: np.ndarray, logit_scale: float, mask_id: int) -> dict:
    """Scaled logits and softmax statistics of each row of z [n, d].

    logits = logit_scale * z W^T with the mask id set to -inf, so the mask token
    can never be chosen nor carry probability.  tok = lowest id of the maximum;
    conf = p(tok); p2 = probability of the best other id.
    """
    logits = logit_scale * (z @ w_lm.T)
    logits[:, mask_id] = -np.inf
    n = logits.shape[0]
    tok = np.argmax(logits, axis=1)  # first (lowest) index among equal maxima
    l1 = logits[np.arange(n), tok]
    other = logits.copy()
    other[np.arange(n), tok] = -np.inf
    l2 = other.max(axis=1)
    Z = np.exp(logits - l1[:, None]).sum(axis=1)
    conf = 1.0 / Z
    p2 = np.exp(l2 - l1) / Z
    return dict(logits=logits, tok=tok.astype(np.int64), conf=conf, p2=p2)


class Model:
    """The transformer for one workload, with weights given as a name -> array mapping.

    ``weights`` holds the storage-rounded values (fp32 arrays are fine: they are
    widened to fp64 at use).  Names follow ``synth.configs.weight_names``.
    ``progress`` (optional) is called with (layer, n_layers, rows) after each layer of a
    forward; it only reports, it takes no part in the arithmetic.
    """

    def __init__(self, cfg: dict, weights, progress=None):
        self.cfg = cfg
        self.w = weights
        self.progress = progress
        self.d = cfg["d_model"]
        self.H = cfg["n_heads"]
        self.Hkv = cfg["n_kv_heads"]
        self.hd = cfg["head_dim"]
        self.L = cfg["prompt_len"] + cfg["gen_length"]

    def _W(self, name: str) -> np.ndarray:
        return np.asarray(self.w[name], dtype=np.float64)

    def new_cache(self):
        """Empty K and V caches for one sequence: per layer [L, Hkv, hd]."""
        shp = (self.L, self.Hkv, self.hd)
        return ([np.zeros(shp) for _ in range(self.cfg["n_layers"])],
                [np.zeros(shp) for _ in range(self.cfg["n_layers"])])

    def forward(self, x: np.ndarray, start: int, stop: int, cache) -> np.ndarray:
        """Forward of rows [start, stop) of one sequence x [L], attending to all L positions.

        Rows outside [start, stop) contribute their cached K/V only.  K/V of the
        rows in the range are written to ``cache`` first, so the queries see the
        fresh values for their own rows.  Returns the final hidden states
        (before the final norm) of the rows, [stop - start, d].
        """
        return self.forward_rows(x, np.arange(start, stop), np.arange(self.L), cache)

    def forward_rows(self, x: np.ndarray, rows, keys, cache, limits=None) -> np.ndarray:
        """Forward of the row positions ``rows`` of one sequence x [L], whose queries attend
        to the positions ``keys`` only (``rows`` must be among them).

        Every position keeps its own index as its rotary position.  With
        ``keys = range(L)`` this is the full-context forward; a shorter ``keys``
        is the pruned context of approximate suffix pruning (the positions not in
        ``keys`` are absent for the model).  ``limits`` (one per row) narrows each
        row's keys further to the positions below its limit (block-causal
        attention).  K/V of the rows are written to the cache at their positions
        first.  Returns the final hidden states of the rows, [len(rows), d].
        """
        cfg = self.cfg
        eps = cfg["rms_eps"]
        ck, cv = cache
        rows = np.asarray(rows, dtype=np.int64)
        keys = np.asarray(keys, dtype=np.int64)
        n = len(rows)
        h = self._W("embed")[x[rows]]
        cos, sin = rope_tables(rows, self.hd, cfg["rope_base"])
        for l in range(cfg["n_layers"]):
            p = f"layers.{l}."
            a = rms_norm(h, self._W(p + "attn_norm"), eps)
            q = (a @ self._W(p + "wq").T).reshape(n, self.H, self.hd)
            k = (a @ self._W(p + "wk").T).reshape(n, self.Hkv, self.hd)
            v = (a @ self._W(p + "wv").T).reshape(n, self.Hkv, self.hd)
            q = apply_rope(q, cos, sin)
            k = apply_rope(k, cos, sin)
            ck[l][rows] = k
            cv[l][rows] = v
            if limits is None:
                o = attention(q, ck[l][keys], cv[l][keys])
            else:
                o = attention_limited(q, ck[l][keys], cv[l][keys], keys, limits)
            o = o.reshape(n, self.H * self.hd)
            h = h + o @ self._W(p + "wo").T
            f = rms_norm(h, self._W(p + "ffn_norm"), eps)
            h = h + swiglu_ffn(f, self._W(p + "w_gate"), self._W(p + "w_up"),
                               self._W(p + "w_down"))
            if self.progress is not None:
                self.progress(l, cfg["n_layers"], n)
        return h

    def stats(self, hidden: np.ndarray) -> dict:
        """Final RMSNorm, scaled lm_head and softmax statistics of hidden rows [n, d]."""
        z = rms_norm(hidden, self._W("final_norm"), self.cfg["rms_eps"])
        return head_stats(z, self._W("lm_head"), self.cfg["logit_scale"], self.cfg["mask_id"])
