"""Oracle decode: block loop, cache policy and confidence-threshold commit, in fp64 NumPy.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What it follows
---------------
* Generation is split into blocks of ``block_size`` that are denoised left to
  right; only the current block's masked positions can be committed
  (Fast-dLLM README, Quick Start: ``--gen_length --steps --block_size``;
  ES-dLLM paper card, Streaming-dLLM abstract: "block-wise diffusion process").
* Confidence-threshold parallel decoding: in one step every masked position of
  the block whose confidence clears the threshold is committed, and a
  committed token is never revised ("Fast-dLLM: Four Acceleration Tracks ...",
  section "The v1 Mechanism"; README Dream command ``alg=confidence_threshold,
  threshold=0.9``).  "Clears" is read as strictly greater.
* The fixed schedule stays as a floor: step j of a block commits at least
  k_j of the most confident masked positions, with the block's step budget
  ``steps / n_blocks`` split evenly over its positions ("... Four Acceleration
  Tracks ...", section "Fast-dLLM v1 Versus a Standard Diffusion Sampler": v1
  keeps the conventional schedule and commits confident positions before it
  ends).  With the default ``steps = gen_length`` the floor is one position per
  step.  Ties in confidence go to the lower position; NaN confidence ranks last.
* The cache is refreshed only at block boundaries: the first step of every
  block is a full forward that rewrites every cache slot and whose block-row
  statistics are that step's statistics.  Later steps of the block recompute
  only the block rows (dual cache) or the block and every later row (prefix
  cache), and attend to the cached K/V of the others.  With no cache every
  step is a full forward (Streaming-dLLM README tables: "Prefix-Cache" and
  "Fast-dLLM" columns against the no-cache backbone).
* Approximate suffix pruning (Streaming-dLLM README, figure caption on
  approximated suffix pruning; ES-dLLM paper card, Streaming-dLLM abstract:
  pruning redundant mask tokens of the suffix).  While block [s, e) is decoded
  the model sees only the prefix, the block, the window of the ``suffix_window``
  positions right after the block and the trailing position L-1; every other
  suffix position is absent, for the block's refresh as well as its steps.  The
  kept positions keep their own rotary positions.  ``suffix_window < 0`` keeps
  the whole context.
* Block-causal attention (``attention == "block_causal"``; Fast-dLLM README
  track table, v2 "Block Diffusion"; Streaming-dLLM README, the note on
  block-causal diffusion models and the Open Pangu table).  The prompt is one
  block and the generation is split into blocks of ``block_size``; a query sees
  every key of its own block and of the blocks before it, nothing after.  A
  finished block's K/V therefore never change: the refresh at block b computes
  only block b-1 (its tokens are now final; for b = 0 the prompt) and block b,
  and every later step recomputes block b.  Suffix pruning does not apply
  (nothing after the block is visible).
* Early exit for converged tokens (``exit_steps`` N > 0, ``exit_floor`` c;
  ES-dLLM paper card, Streaming-dLLM abstract: a dynamic confidence-aware
  strategy with an early exit mechanism that skips the iterations of converged
  tokens).  A masked position's run is the number of consecutive steps of the
  current block, ending at this one, in which its argmax token stayed the same
  and its confidence was above c (a step whose token differs from the previous
  one starts a new run of 1; a confidence of c or less ends the run at 0).
  After the step's commit rule, if every position of the row that is still
  masked has a run of at least N, they are all committed with their argmax:
  the row's block exits early.  N = 0 turns it off.
* First-step confidence scheduling (``first_threshold`` t1 >= 0; ES-dLLM paper
  card, CAI-DLLM abstract: first-step confidence commits easy tokens earlier,
  gives the harder ones more denoising steps and adjusts the schedule per
  output block).  The first step of a block commits with threshold t1 instead
  of the threshold: the easy tokens go at once.  The positions of the row still
  masked after it are the hard ones; the block's remaining spb - 1 steps of
  the step budget are spread over them, so the floor of step j >= 1 is the
  share of the hard positions for step j - 1 of spb - 1 steps (at least 1).
  Each block, and each batch row, gets its own schedule.  t1 < 0 turns it off.
"""

from __future__ import annotations

import numpy as np

from .model import Model

__all__ = ["steps_per_block", "floor_count", "commit_set", "run_update", "hard_floor",
           "Decoder"]

NO_CACHE, PREFIX_CACHE, DUAL_CACHE = 0, 1, 2


def steps_per_block(gen_length: int, block_size: int, steps: int) -> int:
    """Step budget of one block: steps / n_blocks (steps = 0 means gen_length)."""
    if gen_length % block_size:
        raise ValueError("gen_length must be a multiple of block_size")
    nb = gen_length // block_size
    steps = steps or gen_length
    if steps % nb:
        raise ValueError("steps must be a multiple of the number of blocks")
    return steps // nb


def floor_count(block_size: int, spb: int, j: int) -> int:
    """How many positions step j of a block commits at least: the block's positions
    spread evenly over its spb steps, the remainder going to the earliest steps."""
    base, extra = divmod(block_size, spb)
    return max(1, base + (1 if j < extra else 0))


def commit_set(masked: np.ndarray, conf: np.ndarray, threshold: float, k: int) -> np.ndarray:
    """Positions to commit: every masked one with conf > threshold, plus the k most
    confident masked ones (conf descending, then position ascending)."""
    n = masked.shape[0]
    out = np.zeros(n, dtype=bool)
    idx = [i for i in range(n) if masked[i]]
    if not idx:
        return out
    c = {i: (-np.inf if np.isnan(conf[i]) else float(conf[i])) for i in idx}
    for i in idx:
        if c[i] > threshold:
            out[i] = True
    ranked = sorted(idx, key=lambda i: (-c[i], i))
    for i in ranked[:k]:
        out[i] = True
    return out


def run_update(masked: np.ndarray, tok: np.ndarray, conf: np.ndarray, prev_tok: np.ndarray,
               run: np.ndarray, floor: float):
    """Convergence runs after one step: for each masked position, the run grows by one when the
    argmax equals the previous step's and the confidence is above ``floor``, restarts at 1 for
    a new argmax above the floor, and is 0 at or below it (NaN included).  Positions that are not
    masked keep their values.  Returns the new (prev_tok, run)."""
    prev_tok = prev_tok.copy()
    run = run.copy()
    for i in range(masked.shape[0]):
        if not masked[i]:
            continue
        above = bool(conf[i] > floor)  # False for NaN
        if not above:
            run[i] = 0
        elif tok[i] == prev_tok[i]:
            run[i] = run[i] + 1
        else:
            run[i] = 1
        prev_tok[i] = tok[i]
    return prev_tok, run


def hard_floor(n_hard: int, spb: int, j: int) -> int:
    """Floor of step j >= 1 of a block under first-step scheduling: the n_hard positions left
    after the first step spread evenly over the remaining spb - 1 steps (at least 1)."""
    return floor_count(n_hard, max(spb - 1, 1), j - 1)


class Decoder:
    """Block-wise cached decoding of a batch of independent sequences.

    State: tokens ``x`` [B, L], one KV cache per sequence, the current block and
    the step index inside it.  Batch rows advance in lockstep: a row whose block
    is finished commits nothing until every row has finished the block.
    """

    def __init__(self, model: Model, refresh_every_step: bool = False, keep_logits: bool = False):
        cfg = model.cfg
        self.m = model
        self.cfg = cfg
        self.B = cfg["batch"]
        self.P = cfg["prompt_len"]
        self.Bs = cfg["block_size"]
        self.L = cfg["prompt_len"] + cfg["gen_length"]
        self.nb = cfg["gen_length"] // cfg["block_size"]
        self.spb = steps_per_block(cfg["gen_length"], cfg["block_size"], cfg["steps"])
        self.mask_id = cfg["mask_id"]
        self.refresh_every_step = refresh_every_step
        self.keep_logits = keep_logits
        self.caches = [model.new_cache() for _ in range(self.B)]
        self.x = None
        self.block = -1
        self.j = 0
        self.pending = None
        self.forwards = {"full": 0, "cached": 0}
        self.exit_steps = int(cfg.get("exit_steps", 0))
        self.exit_floor = float(cfg.get("exit_floor", 0.9))
        self.first_threshold = float(cfg.get("first_threshold", -1.0))
        self.prev_tok = np.full((self.B, self.Bs), -1, dtype=np.int64)
        self.run = np.zeros((self.B, self.Bs), dtype=np.int64)
        self.n_hard = np.zeros(self.B, dtype=np.int64)
        self.early_exits = 0

    # -- state ---------------------------------------------------------------------------
    def set_tokens(self, x: np.ndarray) -> None:
        x = np.asarray(x, dtype=np.int64)
        assert x.shape == (self.B, self.L)
        self.x = x.copy()

    def block_range(self, b: int) -> tuple[int, int]:
        s = self.P + b * self.Bs
        return s, s + self.Bs

    def block_causal(self) -> bool:
        return self.cfg.get("attention", "full") == "block_causal"

    def block_end(self, p: int) -> int:
        """End of the block that position p belongs to (the prompt is one block)."""
        if p < self.P:
            return self.P
        return self.P + ((p - self.P) // self.Bs + 1) * self.Bs

    def _limits(self, rows) -> np.ndarray:
        return np.array([self.block_end(int(p)) for p in rows])

    def active(self, b: int) -> np.ndarray:
        """Positions the model sees while block b is decoded: all of them, or with suffix
        pruning [0, e + W) and the trailing position L-1."""
        _, e = self.block_range(b)
        W = self.cfg.get("suffix_window", -1)
        if W < 0 or e + W >= self.L - 1:
            return np.arange(self.L)
        return np.concatenate([np.arange(e + W), [self.L - 1]])

    # -- forwards ------------------------------------------------------------------------
    def _full(self) -> list:
        s, e = self.block_range(self.block)
        if self.block_causal():
            # block b-1 (now final; for b = 0 the prompt) and block b, each with its own keys
            rows = np.arange(s - self.Bs if self.block > 0 else 0, e)
            out = []
            for r in range(self.B):
                h = self.m.forward_rows(self.x[r], rows, np.arange(e), self.caches[r],
                                        self._limits(rows))
                out.append(self.m.stats(h[s - rows[0]:]))
            self.forwards["full"] += 1
            return out
        act = self.active(self.block)
        out = []
        for r in range(self.B):
            h = self.m.forward_rows(self.x[r], act, act, self.caches[r])
            out.append(self.m.stats(h[s:e]))  # act[i] == i for every i < e
        self.forwards["full"] += 1
        return out

    def _cached(self) -> list:
        s, e = self.block_range(self.block)
        if self.block_causal():
            rows = np.arange(s, e)
            out = []
            for r in range(self.B):
                h = self.m.forward_rows(self.x[r], rows, np.arange(e), self.caches[r],
                                        self._limits(rows))
                out.append(self.m.stats(h))
            self.forwards["cached"] += 1
            return out
        act = self.active(self.block)
        mode = self.cfg["use_cache"]
        rows = np.arange(s, e) if mode == DUAL_CACHE else act[act >= s]
        out = []
        for r in range(self.B):
            h = self.m.forward_rows(self.x[r], rows, act, self.caches[r])
            out.append(self.m.stats(h[:self.Bs]))
        self.forwards["cached"] += 1
        return out

    def block_begin(self, b: int) -> None:
        """Refresh at a block boundary: full forward, all cache slots rewritten;
        its block-row statistics serve the block's first step."""
        if not 0 <= b < self.nb:
            raise ValueError("block out of range")
        self.block, self.j = b, 0
        self.prev_tok[:] = -1
        self.run[:] = 0
        self.n_hard[:] = 0
        self.pending = self._full()

    def step(self) -> tuple[dict, bool]:
        """One denoising step of the current block: statistics, then commit.

        Returns the step record and whether every row's block is finished.
        """
        if self.pending is not None:
            stats, self.pending = self.pending, None
        elif self.refresh_every_step or self.cfg["use_cache"] == NO_CACHE:
            stats = self._full()
        else:
            stats = self._cached()
        s, e = self.block_range(self.block)
        first = self.first_threshold >= 0
        tau = self.first_threshold if first and self.j == 0 else self.cfg["threshold"]
        committed = np.zeros((self.B, self.Bs), dtype=bool)
        ks = np.zeros(self.B, dtype=np.int64)
        exited = np.zeros(self.B, dtype=bool)
        for r in range(self.B):
            masked = self.x[r, s:e] == self.mask_id
            tok, conf = stats[r]["tok"], stats[r]["conf"]
            if first and self.j >= 1:
                k = hard_floor(int(self.n_hard[r]), self.spb, self.j)
            else:
                k = floor_count(self.Bs, self.spb, self.j)
            ks[r] = k
            c = commit_set(masked, conf, tau, k)
            if self.exit_steps > 0:
                self.prev_tok[r], self.run[r] = run_update(masked, tok, conf, self.prev_tok[r],
                                                           self.run[r], self.exit_floor)
                rest = masked & ~c
                if rest.any() and (self.run[r][rest] >= self.exit_steps).all():
                    c = c | rest
                    exited[r] = True
                    self.early_exits += 1
            if first and self.j == 0:
                self.n_hard[r] = int((masked & ~c).sum())
            self.x[r, s:e][c] = tok[c]
            committed[r] = c
        rec = dict(block=self.block, j=self.j, k=int(ks.max()), ks=ks, exited=exited,
                   tok=np.stack([st["tok"] for st in stats]),
                   conf=np.stack([st["conf"] for st in stats]),
                   p2=np.stack([st["p2"] for st in stats]),
                   committed=committed, x=self.x.copy())
        if self.keep_logits:
            rec["logits"] = np.stack([st["logits"] for st in stats])
        self.j += 1
        done = not bool((self.x[:, s:e] == self.mask_id).any())
        return rec, done

    def run_block(self, b: int) -> list:
        """block_begin(b), then steps until the block is finished."""
        self.block_begin(b)
        recs = []
        while True:
            rec, done = self.step()
            recs.append(rec)
            if done:
                return recs

    def generate(self, prompt: np.ndarray):
        """x = [prompt | mask^G]; every block in order.  Returns (x, step records)."""
        prompt = np.asarray(prompt, dtype=np.int64)
        x = np.full((self.B, self.L), self.mask_id, dtype=np.int64)
        x[:, :self.P] = prompt
        self.set_tokens(x)
        recs = []
        for b in range(self.nb):
            recs += self.run_block(b)
        return self.x.copy(), recs
