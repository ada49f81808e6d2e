"""Brute-force scalar reference for tiny shapes: pure Python loops over floats.

A second, independent spelling of the decode (no NumPy in the arithmetic) used
only to pin the oracle on tiny inputs.  The commit set is formed as a prefix of
the confidence ranking whose length is max(k, number above the threshold),
which is a different construction from the oracle's union of two sets.
"""

import math


def _matvec(W, a):
    # W [out][in] (torch Linear layout), a [in]
    return [sum(W[o][i] * a[i] for i in range(len(a))) for o in range(len(W))]


def _rms(h, g, eps):
    ms = sum(v * v for v in h) / len(h)
    r = 1.0 / math.sqrt(ms + eps)
    return [h[i] * r * g[i] for i in range(len(h))]


def _rope(u, p, base):
    hd = len(u)
    half = hd // 2
    out = list(u)
    for i in range(half):
        th = p * base ** (-2.0 * i / hd)
        c, s = math.cos(th), math.sin(th)
        out[i] = u[i] * c - u[i + half] * s
        out[i + half] = u[i + half] * c + u[i] * s
    return out


class Brute:
    def __init__(self, cfg, W):
        self.cfg = cfg
        self.W = {k: (v.tolist()) for k, v in W.items()}
        self.L = cfg["prompt_len"] + cfg["gen_length"]
        nl, Hkv = cfg["n_layers"], cfg["n_kv_heads"]
        self.K = [[[None] * Hkv for _ in range(self.L)] for _ in range(nl)]
        self.V = [[[None] * Hkv for _ in range(self.L)] for _ in range(nl)]

    def forward_rows(self, x, rows, pos=None, limit=None):
        """Forward of indices ``rows`` of the token list x; index i sits at rotary position
        pos[i] (default i).  A query at index p attends to indices m < limit(p) (default all
        len(x) indices)."""
        cfg = self.cfg
        H, Hkv, hd, eps = cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"], cfg["rms_eps"]
        W = self.W
        n = len(x)
        pos = list(range(n)) if pos is None else pos
        hs = {p: list(W["embed"][x[p]]) for p in rows}
        for l in range(cfg["n_layers"]):
            pre = f"layers.{l}."
            qs = {}
            for p in rows:
                a = _rms(hs[p], W[pre + "attn_norm"], eps)
                q = _matvec(W[pre + "wq"], a)
                k = _matvec(W[pre + "wk"], a)
                v = _matvec(W[pre + "wv"], a)
                qs[p] = [_rope(q[j * hd:(j + 1) * hd], pos[p], cfg["rope_base"]) for j in range(H)]
                for g in range(Hkv):
                    self.K[l][p][g] = _rope(k[g * hd:(g + 1) * hd], pos[p], cfg["rope_base"])
                    self.V[l][p][g] = v[g * hd:(g + 1) * hd]
            for p in rows:
                o = []
                for j in range(H):
                    g = j * Hkv // H
                    nk = n if limit is None else limit(p)
                    sc = [sum(qs[p][j][t] * self.K[l][m][g][t] for t in range(hd)) / math.sqrt(hd)
                          for m in range(nk)]
                    mx = max(sc)
                    e = [math.exp(v - mx) for v in sc]
                    tot = sum(e)
                    o += [sum(e[m] / tot * self.V[l][m][g][t] for m in range(nk)) for t in range(hd)]
                hs[p] = [a + b for a, b in zip(hs[p], _matvec(W[pre + "wo"], o))]
                f = _rms(hs[p], W[pre + "ffn_norm"], eps)
                gt = _matvec(W[pre + "w_gate"], f)
                up = _matvec(W[pre + "w_up"], f)
                act = [gt[i] / (1.0 + math.exp(-gt[i])) * up[i] for i in range(len(gt))]
                hs[p] = [a + b for a, b in zip(hs[p], _matvec(W[pre + "w_down"], act))]
        return hs

    def stats(self, h):
        cfg = self.cfg
        z = _rms(h, self.W["final_norm"], cfg["rms_eps"])
        logits = [cfg["logit_scale"] * v for v in _matvec(self.W["lm_head"], z)]
        ids = [i for i in range(len(logits)) if i != cfg["mask_id"]]
        best = ids[0]
        for i in ids:
            if logits[i] > logits[best]:
                best = i
        second = max(logits[i] for i in ids if i != best)
        Z = sum(math.exp(logits[i] - logits[best]) for i in ids)
        return best, 1.0 / Z, math.exp(second - logits[best]) / Z

    def generate(self, prompt, refresh_every_step=False):
        cfg = self.cfg
        P, G, Bs, mask = cfg["prompt_len"], cfg["gen_length"], cfg["block_size"], cfg["mask_id"]
        nb = G // Bs
        spb = (cfg["steps"] or G) // nb
        x = list(prompt) + [mask] * G
        steps = []
        win = cfg.get("suffix_window", -1)
        if cfg.get("attention", "full") == "block_causal":
            return self._generate_block_causal(x)
        for b in range(nb):
            s, e = P + b * Bs, P + (b + 1) * Bs
            # suffix pruning: the model runs on the shorter sequence of the kept positions
            # (prefix, block, the window after the block, the last position), each keeping its
            # rotary position; its cache is indexed by the short sequence
            if win < 0 or e + win >= self.L - 1:
                keep = list(range(self.L))
            else:
                keep = list(range(e + win)) + [self.L - 1]
            j = 0
            while any(x[i] == mask for i in range(s, e)):
                if j == 0 or refresh_every_step or cfg["use_cache"] == 0:
                    rows = list(range(len(keep)))
                elif cfg["use_cache"] == 1:
                    rows = list(range(s, len(keep)))
                else:
                    rows = list(range(s, e))
                hs = self.forward_rows([x[p] for p in keep], rows, keep)
                st = {p: self.stats(hs[p]) for p in range(s, e)}
                k = max(1, Bs // spb + (1 if j < Bs % spb else 0))
                masked = [p for p in range(s, e) if x[p] == mask]
                ranking = sorted(masked, key=lambda p: (-st[p][1], p))
                n_above = sum(1 for p in masked if st[p][1] > cfg["threshold"])
                chosen = ranking[:max(k, n_above)]
                for p in chosen:
                    x[p] = st[p][0]
                steps.append(dict(block=b, j=j, stats=st, chosen=sorted(chosen)))
                j += 1
        return x, steps

    def _generate_block_causal(self, x):
        """Block-causal decoding spelled without a cache: every step recomputes every position
        up to the block's end from scratch, a query at p attending to the indices below the end
        of p's block (the prompt being one block)."""
        cfg = self.cfg
        P, G, Bs, mask = cfg["prompt_len"], cfg["gen_length"], cfg["block_size"], cfg["mask_id"]
        nb = G // Bs
        spb = (cfg["steps"] or G) // nb

        def block_end(p):
            return P if p < P else P + ((p - P) // Bs + 1) * Bs

        steps = []
        for b in range(nb):
            s, e = P + b * Bs, P + (b + 1) * Bs
            j = 0
            while any(x[i] == mask for i in range(s, e)):
                hs = self.forward_rows(x[:e], list(range(e)), None, block_end)
                st = {p: self.stats(hs[p]) for p in range(s, e)}
                k = max(1, Bs // spb + (1 if j < Bs % spb else 0))
                masked = [p for p in range(s, e) if x[p] == mask]
                ranking = sorted(masked, key=lambda p: (-st[p][1], p))
                n_above = sum(1 for p in masked if st[p][1] > cfg["threshold"])
                chosen = ranking[:max(k, n_above)]
                for p in chosen:
                    x[p] = st[p][0]
                steps.append(dict(block=b, j=j, stats=st, chosen=sorted(chosen)))
                j += 1
        return x, steps
