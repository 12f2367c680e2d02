"""Plain fp64 NumPy oracle of the multi-layer block-diffusion decode.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``, never by the HIP product path.
It shares no code with the HIP path.

The decoding procedure is the one of ``oracle.refine`` (exact refresh step at
each window start, DualCache steps, token shift, carry row, commit of the
clean block; "Fast-dLLM v2: Efficient Block-Diffusion LLM" notes, Framework
and Key designs 2-4; "Fast-dLLM" v1 article, Core techniques 1-2), applied to
a stack of transformer layers instead of one attention layer.  The pages name
the model family (Qwen2.5-style decoders adapted to block diffusion) but not
its layer equations; this module takes the plainest reading of that family,
listed here and in the design notes:

* pre-norm layers: x += attn(rmsnorm(x)); x += mlp(rmsnorm(x)); a final
  rmsnorm before the LM head;
* RMSNorm y = x / sqrt(mean(x^2) + eps) with unit gains (random-init model);
* rotary position embedding in the rotate-half form: for i < d/2 the pair
  (x_i, x_{i+d/2}) is rotated by the angle pos * theta^(-2i/d), applied to
  queries and keys (so the cached keys are rotated) at their absolute
  positions;
* SwiGLU MLP: down(silu(gate(h)) * up(h)), silu(z) = z * sigmoid(z);
* no biases; the softmax scale 1/sqrt(d);
* the LM head and the carry/snapshot rows use the final normalised hidden
  state.

With ``norm``, ``rope`` and ``mlp`` switched off and one layer the model is
exactly the one-layer model of ``oracle.refine`` (pinned by a test).  The
pieces (RMSNorm, rotary embedding, SwiGLU) and the exactness of the cached
steps are pinned; where the norms sit in a layer (pre-norm) is a reading of
the model family with no independent pin: parity unpinned for that choice.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

from .refine import (F64, attention, confidence, lm_logits, shift_row, threshold_unmask, visible)


# ==========================================================================
# layer pieces
# ==========================================================================
def rmsnorm(x, eps: float) -> np.ndarray:
    """RMSNorm with unit gains over the last axis."""
    x = np.asarray(x, dtype=F64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def rope(x, pos, theta: float) -> np.ndarray:
    """Rotary embedding, rotate-half form, of x [n, H, d] at positions pos [n]:
    dims i and i + d/2 (i < d/2) are rotated by pos * theta^(-2i/d)."""
    x = np.asarray(x, dtype=F64)
    n, H, d = x.shape
    half = d // 2
    inv = theta ** (-2.0 * np.arange(half) / d)
    ang = np.asarray(pos, dtype=F64)[:, None] * inv[None, :]          # [n, half]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def silu(z) -> np.ndarray:
    z = np.asarray(z, dtype=F64)
    return z / (1.0 + np.exp(-z))


@dataclass
class Layer:
    """Weights of one layer, out x in: Wq [Hq*d, hid], Wk/Wv [Hkv*d, hid],
    Wo [hid, Hq*d], Wg/Wu [I, hid], Wd [hid, I]."""
    Wq: np.ndarray
    Wk: np.ndarray
    Wv: np.ndarray
    Wo: np.ndarray
    Wg: np.ndarray | None = None
    Wu: np.ndarray | None = None
    Wd: np.ndarray | None = None


@dataclass
class LM:
    """Token embeddings E [V+1, hid] (row V = [MASK]), layers, LM head
    Wlm [V, hid]; switches for the pieces beyond the one-layer model."""
    E: np.ndarray
    layers: list
    Wlm: np.ndarray
    Hq: int
    Hkv: int
    d: int
    eps: float = 1e-6
    theta: float = 1e6
    norm: bool = True
    use_rope: bool = True
    mlp: bool = True

    @property
    def V(self) -> int:
        return self.Wlm.shape[0]

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @classmethod
    def from_weights(cls, w, cfg, **kw) -> "LM":
        f = lambda a: None if a is None else np.asarray(a, dtype=F64)
        layers = [Layer(f(l.Wq), f(l.Wk), f(l.Wv), f(l.Wo), f(l.Wg), f(l.Wu), f(l.Wd)) for l in w.layers]
        return cls(f(w.E), layers, f(w.Wlm), cfg.Hq, cfg.Hkv, cfg.d, cfg.eps, cfg.theta, **kw)


def embed(model: LM, tokens, masked) -> np.ndarray:
    """E[token] where unmasked, the [MASK] row E[V] where masked (v2 notes,
    Key design 2)."""
    rows = np.where(np.asarray(masked, dtype=bool), model.V, np.asarray(tokens))
    return model.E[rows].astype(F64)


def _norm(model: LM, x):
    return rmsnorm(x, model.eps) if model.norm else np.asarray(x, dtype=F64)


def mlp(model: LM, layer: Layer, h) -> np.ndarray:
    return (silu(h @ layer.Wg.T) * (h @ layer.Wu.T)) @ layer.Wd.T


def layer_qkv(model: LM, layer: Layer, X, pos):
    """Normalised input, projections and rotary embedding of rows X at
    positions pos.  Returns Q [n, Hq, d], K, V [n, Hkv, d]."""
    n = X.shape[0]
    h = _norm(model, X)
    Q = (h @ layer.Wq.T).reshape(n, model.Hq, model.d)
    K = (h @ layer.Wk.T).reshape(n, model.Hkv, model.d)
    V = (h @ layer.Wv.T).reshape(n, model.Hkv, model.d)
    if model.use_rope:
        Q, K = rope(Q, pos, model.theta), rope(K, pos, model.theta)
    return Q, K, V


def layer_rest(model: LM, layer: Layer, X, O) -> np.ndarray:
    """x += o Wo^T; then x += mlp(rmsnorm(x))."""
    n = X.shape[0]
    X = X + O.reshape(n, -1) @ layer.Wo.T
    if model.mlp:
        X = X + mlp(model, layer, _norm(model, X))
    return X


# ==========================================================================
# sequences, steps and the block loop
# ==========================================================================
@dataclass
class MSeq:
    """One sequence of the multi-layer model: per-layer block-level caches
    (cache_k[l] [L, Hkv, d], keys rotated), the carry (final normalised row
    of the last committed position), the current block and the per-layer
    DualCache snapshot."""
    cache_k: list
    cache_v: list
    carry: np.ndarray
    history: list
    tokens: np.ndarray
    masked: np.ndarray
    snap_k: list | None = None
    snap_v: list | None = None
    snap_h: np.ndarray | None = None
    window: int = 0

    @property
    def L(self) -> int:
        return self.cache_k[0].shape[0]


@dataclass
class MStep:
    H: np.ndarray       # final normalised rows of this step's fresh rows
    rows: np.ndarray
    src: np.ndarray     # [S, hid] row feeding each window position
    argmax: np.ndarray
    conf: np.ndarray
    picked: list
    K: list             # per layer: fresh K of this step (rotated)
    V: list


def forward_rows(model: LM, seq: MSeq | None, X, rows, D: int, snap_k=None, snap_v=None):
    """All layers over input rows X of block rows ``rows`` (positions
    L + rows).  Queries see every cached row and the in-block rows of blocks
    up to their own (hybrid mask); the in-block K/V are this pass's fresh
    rows, and in a DualCache pass the other rows come from the snapshot.
    With ``seq`` None there is no cache and the rows are a whole multi-block
    prompt (positions = rows).  Returns (final normalised rows, [K], [V])."""
    rows = np.asarray(rows)
    L = 0 if seq is None else seq.L
    pos = L + rows
    n_blk = D if seq is not None else len(rows)
    Ks, Vs = [], []
    for li, layer in enumerate(model.layers):
        Q, K, V = layer_qkv(model, layer, X, pos)
        if snap_k is None:
            assert len(rows) == n_blk and np.array_equal(rows, np.arange(n_blk))
            bk, bv = K, V
        else:
            bk, bv = snap_k[li].copy(), snap_v[li].copy()
            bk[rows], bv[rows] = K, V
        if seq is not None:
            Kc = np.concatenate([seq.cache_k[li], bk], axis=0)
            Vc = np.concatenate([seq.cache_v[li], bv], axis=0)
        else:
            Kc, Vc = bk, bv
        vis = visible(pos, np.arange(L + n_blk), D)
        O, _ = attention(Q, Kc, Vc, vis, model.G)
        X = layer_rest(model, layer, X, O)
        Ks.append(K)
        Vs.append(V)
    return _norm(model, X), Ks, Vs


def prefill(model: LM, prompt, D: int) -> MSeq:
    """A block-aligned prompt through all layers under the block-causal mask
    (the same hybrid mask as decoding; v2 notes, Framework).  Every prompt
    row's rotated K/V go to the caches; the carry is the last row."""
    prompt = np.asarray(prompt)
    P = len(prompt)
    assert P % D == 0 and P > 0
    X = embed(model, prompt, np.zeros(P, dtype=bool))
    H, Ks, Vs = forward_rows(model, None, X, np.arange(P), D)
    return MSeq(Ks, Vs, H[P - 1], list(prompt), np.zeros(D, dtype=np.int64), np.ones(D, dtype=bool))


def new_block(seq: MSeq, D: int) -> None:
    seq.tokens = np.zeros(D, dtype=np.int64)
    seq.masked = np.ones(D, dtype=bool)
    seq.window = 0
    seq.snap_k = seq.snap_v = seq.snap_h = None


def _decide(model: LM, seq: MSeq, s: int, S: int, tau, src):
    am, _, _, conf = confidence(lm_logits(model.Wlm, src))
    seq.tokens, seq.masked, picked = threshold_unmask(conf, am, seq.tokens, seq.masked, s * S, tau)
    return am, conf, picked


def e_step(model: LM, seq: MSeq, s: int, S: int, tau, D: int) -> MStep:
    """Exact step for window s: every block row recomputed through all
    layers; its per-layer K/V and the row feeding position s*S become the
    window's DualCache snapshot (refine.e_step, per layer)."""
    X = embed(model, seq.tokens, seq.masked)
    H, Ks, Vs = forward_rows(model, seq, X, np.arange(D), D)
    seq.snap_k, seq.snap_v = Ks, Vs
    seq.snap_h = H[shift_row(s * S)] if s > 0 else seq.carry
    src = np.stack([H[shift_row(j)] if shift_row(j) >= 0 else seq.carry for j in range(s * S, s * S + S)])
    am, conf, picked = _decide(model, seq, s, S, tau, src)
    seq.window = s
    return MStep(H, np.arange(D), src, am, conf, picked, Ks, Vs)


def dc_step(model: LM, seq: MSeq, s: int, S: int, tau, D: int) -> MStep:
    """DualCache step for window s: only the window rows go through the
    layers; every layer's other in-block K/V and the row feeding the first
    window position come from the snapshot (refine.dc_step, per layer)."""
    assert seq.snap_k is not None and seq.window == s
    lo = s * S
    rows = np.arange(lo, lo + S)
    X = embed(model, seq.tokens[rows], seq.masked[rows])
    H, Ks, Vs = forward_rows(model, seq, X, rows, D, seq.snap_k, seq.snap_v)
    src = np.stack([H[shift_row(j) - lo] if shift_row(j) >= lo else seq.snap_h for j in range(lo, lo + S)])
    am, conf, picked = _decide(model, seq, s, S, tau, src)
    return MStep(H, rows, src, am, conf, picked, Ks, Vs)


def commit(model: LM, seq: MSeq, D: int) -> np.ndarray:
    """Finished block -> per-layer caches; the new carry is the last row of
    a forward pass over the clean block (refine.commit, per layer)."""
    assert not seq.masked.any()
    X = embed(model, seq.tokens, seq.masked)
    H, Ks, Vs = forward_rows(model, seq, X, np.arange(D), D)
    seq.cache_k = [np.concatenate([c, k], axis=0) for c, k in zip(seq.cache_k, Ks)]
    seq.cache_v = [np.concatenate([c, v], axis=0) for c, v in zip(seq.cache_v, Vs)]
    seq.carry = H[D - 1]
    seq.history = list(seq.history) + [int(t) for t in seq.tokens]
    return H


def full_forward(model: LM, history, block_tokens, block_masked, D: int):
    """All layers over [committed clean tokens | current noisy block] with the
    hybrid mask and no cache (the cache-free definition the cached steps must
    reproduce).  Returns the final normalised rows of every position."""
    toks = np.concatenate([np.asarray(history, dtype=np.int64), np.asarray(block_tokens, dtype=np.int64)])
    msk = np.concatenate([np.zeros(len(history), dtype=bool), np.asarray(block_masked, dtype=bool)])
    X = embed(model, toks, msk)
    H, _, _ = forward_rows(model, None, X, np.arange(len(toks)), D)
    return H


def decode_block(model: LM, seqs: list, D: int, S: int, tau, mode: str = "dual", on_step=None,
                 max_steps: int = 10_000) -> int:
    """Decode the current block of every sequence in lockstep, then commit
    (refine.decode_block with lockstep=True).  Returns the number of steps."""
    assert D % S == 0
    step = 0
    for s in range(D // S):
        first = True
        while any(q.masked[s * S:(s + 1) * S].any() for q in seqs):
            kind = "E" if (first or mode == "exact") else "DC"
            fn = e_step if kind == "E" else dc_step
            res = [fn(model, q, s, S, tau, D) for q in seqs]
            if on_step is not None:
                on_step(step, s, kind, res)
            first = False
            step += 1
            assert step < max_steps
    for q in seqs:
        commit(model, q, D)
    return step


def generate(model: LM, prompts, n_blocks: int, D: int, S: int, tau, on_step=None) -> list:
    """Prefill every prompt, then decode n_blocks blocks in lockstep.
    Returns the sequences (history = prompt + generated tokens)."""
    seqs = [prefill(model, p, D) for p in prompts]
    for _ in range(n_blocks):
        for q in seqs:
            new_block(q, D)
        decode_block(model, seqs, D, S, tau, on_step=on_step)
    return seqs
