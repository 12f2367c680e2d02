"""Plain fp64 NumPy oracle of Fast-dLLM v1-style decoding of a full-attention
diffusion LM with the block-wise approximate KV cache (DualCache).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``, never by the HIP product path.
It shares no code with the HIP path.  The one-layer model pieces and the
threshold rule are those of ``oracle.refine``.

Source: "Fast-dLLM: Training-free Acceleration of Diffusion LLM by Enabling
KV Cache and Parallel Decoding" (article), Core technique 1 (block-wise KV
cache for bidirectional attention: DualCache keeps the K/V of the prefix
(prompt and decoded blocks) and of the suffix (the masked positions after
the current block) and reuses them while the current block is refined;
activations of adjacent steps are nearly identical, so the reuse is an
approximation) and Core technique 2 (confidence-aware parallel decoding,
the same threshold rule as in v2).

The sequence is [prompt | generation region]; the generation region
(a multiple of D positions) starts fully masked and is decoded block by
block, left to right.  Attention is full (every position sees every
position, masked ones included).

Readings (the article gives the cache's contents, not its schedule):

* the cache is refreshed once per block: the first step of a block is an
  exact forward pass over the whole sequence; its K/V outside the block
  become the prefix and suffix caches, and later steps of the block
  recompute only the block's D rows, attending over prefix cache, the fresh
  block rows and suffix cache;
* the token shift of the one-layer model is kept (the prediction for
  position j is read from output row j - 1); the row feeding the block's
  first position comes from the refresh pass (like the v2 snapshot row);
* candidates are the masked positions of the current block; the threshold
  rule is the v2 one (strict ``>``, at least one token per step).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import refine as R

F64 = np.float64


def full_forward(model: R.Model, tokens, masked, plant=None):
    """Full-attention forward over all T positions: (H, K, V)."""
    X = R.embed(model, np.asarray(tokens), np.asarray(masked, dtype=bool))
    if plant is not None:
        X = X + np.asarray(plant, dtype=F64)
    Q, K, V = R.project(model, X)
    T = X.shape[0]
    O, _ = R.attention(Q, K, V, np.ones((T, T), dtype=bool), model.G)
    return R.output(model, X, O), K, V


@dataclass
class V1Seq:
    """tokens / masked [T]: prompt (unmasked) then the generation region.
    cache_k/v: K/V of every row outside the current block (prefix rows, then
    suffix rows) from the last refresh; carry: output row feeding the
    block's first position; plant: optional [T, hidden] input offset."""
    tokens: np.ndarray
    masked: np.ndarray
    P: int
    plant: np.ndarray | None = None
    block: int = -1
    cache_k: np.ndarray | None = None
    cache_v: np.ndarray | None = None
    carry: np.ndarray | None = None

    @property
    def T(self) -> int:
        return len(self.tokens)


@dataclass
class V1Step:
    src: np.ndarray         # [D, hidden] row feeding each block position
    argmax: np.ndarray
    maxlogit: np.ndarray
    lse: np.ndarray
    conf: np.ndarray
    picked: list


def new_sequence(prompt, gen_len: int, plant=None) -> V1Seq:
    prompt = np.asarray(prompt, dtype=np.int64)
    P = len(prompt)
    tokens = np.concatenate([prompt, np.zeros(gen_len, dtype=np.int64)])
    masked = np.concatenate([np.zeros(P, dtype=bool), np.ones(gen_len, dtype=bool)])
    return V1Seq(tokens, masked, P, plant)


def _bounds(seq: V1Seq, k: int, D: int):
    lo = seq.P + k * D
    return lo, lo + D


def _decide(model, seq, lo, D, src, tau) -> V1Step:
    logits = R.lm_logits(model.Wlm, src)
    am, mx, lse, conf = R.confidence(logits)
    blk_t, blk_m, picked = R.threshold_unmask(conf, am, seq.tokens[lo:lo + D], seq.masked[lo:lo + D], 0, tau)
    seq.tokens[lo:lo + D] = blk_t
    seq.masked[lo:lo + D] = blk_m
    return V1Step(src, am, mx, lse, conf, [lo + p for p in picked])


def exact_step(model: R.Model, seq: V1Seq, k: int, D: int, tau, refresh: bool = True) -> V1Step:
    """Exact step of block k: a full forward pass; predictions for block
    position j from output row j - 1.  With ``refresh`` the pass also
    refills the DualCache (prefix and suffix K/V, carry row)."""
    lo, hi = _bounds(seq, k, D)
    assert lo >= 1
    H, K, V = full_forward(model, seq.tokens, seq.masked, seq.plant)
    if refresh:
        seq.block = k
        seq.cache_k = np.concatenate([K[:lo], K[hi:]], axis=0)
        seq.cache_v = np.concatenate([V[:lo], V[hi:]], axis=0)
        seq.carry = H[lo - 1]
    src = H[lo - 1:hi - 1]
    return _decide(model, seq, lo, D, src, tau)


def dual_step(model: R.Model, seq: V1Seq, k: int, D: int, tau) -> V1Step:
    """DualCache step of block k: only the block's D rows are recomputed;
    they attend over the cached prefix and suffix K/V and the fresh block
    K/V (all visible); position j of the block reads row j - 1, the first
    position the carry row of the refresh."""
    assert seq.block == k and seq.cache_k is not None
    lo, hi = _bounds(seq, k, D)
    plant = None if seq.plant is None else seq.plant[lo:hi]
    X = R.embed(model, seq.tokens[lo:hi], seq.masked[lo:hi])
    if plant is not None:
        X = X + np.asarray(plant, dtype=F64)
    Q, Kb, Vb = R.project(model, X)
    K_all = np.concatenate([seq.cache_k, Kb], axis=0)
    V_all = np.concatenate([seq.cache_v, Vb], axis=0)
    O, _ = R.attention(Q, K_all, V_all, np.ones((D, K_all.shape[0]), dtype=bool), model.G)
    H = R.output(model, X, O)
    src = np.concatenate([seq.carry[None, :], H[:D - 1]], axis=0)
    return _decide(model, seq, lo, D, src, tau)


def decode(model: R.Model, seq: V1Seq, D: int, tau, mode: str = "dual", on_step=None) -> int:
    """Decode the whole generation region block by block.  mode 'dual':
    refresh step, then DualCache steps until the block is unmasked; mode
    'exact': a full forward pass every step.  Returns the number of steps."""
    n_blocks = (seq.T - seq.P) // D
    steps = 0
    for k in range(n_blocks):
        lo, hi = _bounds(seq, k, D)
        first = True
        while seq.masked[lo:hi].any():
            if first or mode == "exact":
                res = exact_step(model, seq, k, D, tau, refresh=True)
                kind = "E"
            else:
                res = dual_step(model, seq, k, D, tau)
                kind = "DC"
            if on_step is not None:
                on_step(k, kind, res)
            first = False
            steps += 1
    return steps
