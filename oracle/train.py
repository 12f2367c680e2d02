"""Plain fp64 NumPy oracle of the training form of block diffusion (forward
pass and loss value only).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``, never by the HIP product path.
It shares no code with the HIP path.  The one-layer model pieces (embedding
with the [MASK] row, projections, masked softmax attention, output
projection, LM-head logits) are those of ``oracle.refine``.

Source: "Fast-dLLM v2: Efficient Block-Diffusion LLM" (ICLR 2026 paper
notes), Key design 1 (every training sequence of length L is cut into
aligned blocks of D) and Key design 2:

* a binary mask m over the positions replaces masked tokens by the
  learnable [MASK] embedding (the noisy sequence x_t); each sample is put in
  the batch twice, with m and with its complement 1 - m, so every token is
  masked in exactly one of the two views;
* the prediction for masked position i is read from the logit of position
  i - 1 (token shift), and the loss is the cross-entropy on masked tokens
  only, of x_0^i given the clean earlier blocks x_{<i} and the whole own
  block x_block(i) (noisy);
* x_t and x_0 are concatenated along the sequence into 2L positions and
  attended under one hybrid mask A in {0, 1}^{2L x 2L}.

Readings (the pages print no matrix A and no rule for block starts):

* rows and columns 0 .. L-1 are x_t (noisy), L .. 2L-1 are x_0 (clean);
  block of position p = (p mod L) // D;
* a noisy query of block b sees the noisy keys of block b (bidirectional)
  and the clean keys of blocks < b; a clean query of block b sees the clean
  keys of blocks <= b; clean queries never see noisy keys.  These are the
  conditioning sets of the loss (x_{<i} clean, x_block(i) noisy), and the
  clean half alone is the block-causal forward used at inference;
* the logit for masked position i is taken from noisy row i - 1 when i - 1
  lies in the same block, and from clean row i - 1 when i starts a block:
  the only row of block b - 1 conditioned on exactly x_{<i}, the row that
  is the carry at inference (v2 notes, Key design 2 and 3).  Position 0 has
  no predecessor and is never supervised;
* the loss of a sample is the sum of the two views' masked-token
  cross-entropies (natural log); the mean divides by the number of
  supervised positions.
"""
from __future__ import annotations

import numpy as np

from . import refine as R

F64 = np.float64


def mask_2L(L: int, D: int) -> np.ndarray:
    """The hybrid mask A [2L, 2L] (True = key visible), written out region by
    region from the four rules above."""
    assert L % D == 0
    A = np.zeros((2 * L, 2 * L), dtype=bool)
    for p in range(2 * L):
        bp = (p % L) // D
        for c in range(2 * L):
            bc = (c % L) // D
            if p < L and c < L:          # noisy -> noisy: same block only
                A[p, c] = bc == bp
            elif p < L:                  # noisy -> clean: strictly earlier blocks
                A[p, c] = bc < bp
            elif c >= L:                 # clean -> clean: block-causal
                A[p, c] = bc <= bp
            else:                        # clean -> noisy: never
                A[p, c] = False
    return A


def complementary_views(m) -> tuple:
    """The two views of a sample: mask m and its complement."""
    m = np.asarray(m, dtype=bool)
    return m, ~m


def forward_2L(model: R.Model, x0, m, D: int, plant=None):
    """One-layer forward over [x_t | x_0] under A.  Returns (H, Q, K, V, O)
    for all 2L rows; plant [2L, hidden] is an optional additive offset of
    the input rows (synthetic workloads)."""
    x0 = np.asarray(x0, dtype=np.int64)
    L = len(x0)
    X = np.concatenate([R.embed(model, x0, np.asarray(m, dtype=bool)),
                        R.embed(model, x0, np.zeros(L, dtype=bool))], axis=0)
    if plant is not None:
        X = X + np.asarray(plant, dtype=F64)
    Q, K, V = R.project(model, X)
    O, _ = R.attention(Q, K, V, mask_2L(L, D), model.G)
    return R.output(model, X, O), Q, K, V, O


def source_row(i: int, L: int, D: int) -> int:
    """Row of the 2L layout whose logits predict position i (i >= 1)."""
    assert 1 <= i < L
    return i - 1 if i % D != 0 else L + i - 1


def supervised(m) -> np.ndarray:
    """Positions whose cross-entropy counts in a view: masked, and i >= 1."""
    m = np.asarray(m, dtype=bool)
    idx = np.flatnonzero(m)
    return idx[idx >= 1]


def token_nll(logits: np.ndarray, target) -> np.ndarray:
    """-log softmax(logits)[target] per row, natural log, in float64."""
    logits = np.atleast_2d(np.asarray(logits, dtype=F64))
    mx = logits.max(axis=1, keepdims=True)
    lse = (mx + np.log(np.exp(logits - mx).sum(axis=1, keepdims=True)))[:, 0]
    return lse - logits[np.arange(logits.shape[0]), np.asarray(target)]


def view_nll(model: R.Model, x0, m, D: int, plant=None):
    """Masked-token cross-entropy terms of one view.  Returns (positions,
    source rows, nll per position, H)."""
    x0 = np.asarray(x0, dtype=np.int64)
    L = len(x0)
    H = forward_2L(model, x0, m, D, plant)[0]
    pos = supervised(m)
    rows = np.array([source_row(int(i), L, D) for i in pos], dtype=np.int64)
    logits = R.lm_logits(model.Wlm, H[rows]) if len(rows) else np.zeros((0, model.V))
    return pos, rows, token_nll(logits, x0[pos]), H


def sample_loss(model: R.Model, x0, m, D: int):
    """Loss of one sample over its two complementary views: (sum of the
    masked-token cross-entropies, number of supervised positions)."""
    total, count = 0.0, 0
    for view in complementary_views(m):
        pos, _, nll, _ = view_nll(model, x0, view, D)
        total += float(nll.sum())
        count += len(pos)
    return total, count
