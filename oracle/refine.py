"""Plain fp64 NumPy oracle of block-diffusion decoding (Fast-dLLM v2 style).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``, never by the HIP product path.
It shares no code with the HIP path; the seeded inputs come from
``bd_inputs``, which holds no arithmetic of the method.

Everything is computed in float64 from the (float32-stored, possibly
bf16-representable) inputs, with no intermediate rounding, in the order the
method describes it.  Sources (page titles; see the sections named):

* "Fast-dLLM v2: Efficient Block-Diffusion LLM" (ICLR 2026 paper notes,
  cited below as *v2 notes*): Framework; flowchart; Key design 1 (block-
  aligned blocks of size D), Key design 2 (learnable [MASK] embedding, token
  shift: the prediction for masked position i uses the output at i-1;
  conditioning set = clean earlier blocks plus the whole own block), Key
  design 3 (block-level cache of finished blocks, confidence-threshold
  parallel unmasking, threshold 1.0 degenerates to ordinary decoding,
  DualCache prefix+suffix reuse inside the block), Key design 4 (sub-block
  decoding, block 32 / sub-block 8).
* "Fast-dLLM: Training-free Acceleration of Diffusion LLM" article (cited
  as *v1 article*), Core technique 1 (block-wise KV cache, DualCache) and 2
  (confidence = probability the model gives the token; threshold rule).
* "Fast-dLLM v2" news article (aigc.bar, *v2 news*), "hierarchical cache"
  and "block structure" paragraphs: bidirectional inside a block, causal
  across blocks; finished blocks' K/V reused like an AR KV cache.

Readings where the pages are silent or disagree (each is also listed in the
design notes of the repository):

* threshold test is strict ``conf > tau`` ("exceeds", v2 notes Key design 3);
* a step in which no candidate passes unmasks the single most confident
  candidate (so tau = 1.0 gives one token per step, v2 notes Key design 3);
* ties: argmax over the vocabulary takes the lowest id; the most confident
  position takes the lowest position;
* the row that feeds block position 0 is the *carry*: the output row of the
  last committed position, from the forward pass that committed it;
* in a DualCache step the row that feeds the first window position (row
  s*S-1) comes from the snapshot, like every other row outside the window;
* the K/V appended when a block completes come from a forward pass over the
  final clean block (commit), not from the last refinement step;
* the snapshot is refreshed by an exact step at the start of each window;
* windows advance left to right; only masked positions of the active window
  are candidates; no re-masking;
* softmax scale 1/sqrt(d); no RoPE, norm or bias in the one-layer model.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

F64 = np.float64
_VCHUNK = 8192          # LM-head rows converted to float64 at a time


# ==========================================================================
# model pieces
# ==========================================================================
@dataclass
class Model:
    """One attention layer + LM head (weights stored out x in, row-major).

    E [V+1, hidden]: token embeddings, row V is the learnable [MASK]
    embedding (v2 notes, Key design 2).  Wq [Hq*d, hidden], Wk/Wv
    [Hkv*d, hidden], Wo [hidden, Hq*d], Wlm [V, hidden].
    """
    E: np.ndarray
    Wq: np.ndarray
    Wk: np.ndarray
    Wv: np.ndarray
    Wo: np.ndarray
    Wlm: np.ndarray
    Hq: int
    Hkv: int
    d: int

    @property
    def V(self) -> int:
        return self.Wlm.shape[0]

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @classmethod
    def from_weights(cls, w, cfg) -> "Model":
        f = lambda a: np.asarray(a, dtype=F64)
        return cls(f(w.E), f(w.Wq), f(w.Wk), f(w.Wv), f(w.Wo), f(w.Wlm), cfg.Hq, cfg.Hkv, cfg.d)


def kv_head(h: int, G: int) -> int:
    """Grouped-query attention: query head h reads KV head h // G."""
    return h // G


def shift_row(j: int) -> int:
    """Token shift (v2 notes, Key design 2): the prediction for block
    position j is read from the output row of position j - 1."""
    return j - 1


def block_index(pos, D: int):
    return np.asarray(pos) // D


def visible(q_pos, k_pos, D: int) -> np.ndarray:
    """Hybrid block mask (v2 notes, Framework; v2 news, block structure).

    Key k is visible to query p iff block(k) <= block(p): bidirectional
    inside a block, causal across blocks.  [n_q, n_k] bool.
    """
    return block_index(k_pos, D)[None, :] <= block_index(q_pos, D)[:, None]


def embed(model: Model, tokens, masked, plant=None) -> np.ndarray:
    """Input rows: E[token] where unmasked, the [MASK] row E[V] where masked
    (v2 notes, Key design 2), plus an optional synthetic offset."""
    rows = np.where(np.asarray(masked, dtype=bool), model.V, np.asarray(tokens))
    X = model.E[rows].astype(F64)
    if plant is not None:
        X = X + np.asarray(plant, dtype=F64)
    return X


def project(model: Model, X: np.ndarray):
    """Q = X Wq^T, K = X Wk^T, V = X Wv^T, split into heads."""
    n = X.shape[0]
    Q = (X @ model.Wq.T).reshape(n, model.Hq, model.d)
    K = (X @ model.Wk.T).reshape(n, model.Hkv, model.d)
    V = (X @ model.Wv.T).reshape(n, model.Hkv, model.d)
    return Q, K, V


def attention(Q, K, V, vis, G: int):
    """Masked softmax attention, per query head, in float64.

    Q [n, Hq, d]; K, V [T, Hkv, d]; vis [n, T] bool.  Scores are q.k/sqrt(d);
    the softmax subtracts the row max.  Returns O [n, Hq, d] and the natural
    log-sum-exp of the visible scores, lse [Hq, n].
    """
    n, Hq, d = Q.shape
    O = np.empty((n, Hq, d), dtype=F64)
    lse = np.empty((Hq, n), dtype=F64)
    scale = 1.0 / math.sqrt(d)
    for h in range(Hq):
        g = kv_head(h, G)
        s = (Q[:, h, :] @ K[:, g, :].T) * scale
        s = np.where(vis, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        p = np.exp(s - m)
        z = p.sum(axis=1, keepdims=True)
        O[:, h, :] = (p / z) @ V[:, g, :]
        lse[h] = (m + np.log(z))[:, 0]
    return O, lse


def output(model: Model, X: np.ndarray, O: np.ndarray) -> np.ndarray:
    """H = X + concat_h(O) Wo^T (attention output projection with residual)."""
    n = X.shape[0]
    return X + O.reshape(n, -1) @ model.Wo.T


def lm_logits(Wlm: np.ndarray, h: np.ndarray) -> np.ndarray:
    """logits = h Wlm^T in float64 (Wlm rows lifted to float64 chunk by chunk
    when they are stored in a narrower type)."""
    h = np.atleast_2d(np.asarray(h, dtype=F64))
    out = np.empty((h.shape[0], Wlm.shape[0]), dtype=F64)
    for v0 in range(0, Wlm.shape[0], _VCHUNK):
        w = np.asarray(Wlm[v0:v0 + _VCHUNK], dtype=F64)
        out[:, v0:v0 + w.shape[0]] = h @ w.T
    return out


def confidence(logits: np.ndarray):
    """Per row: argmax (lowest id on ties), max logit, log-sum-exp and the
    confidence = the softmax probability of the argmax token
    (v1 article, Core technique 2: confidence is the probability the model
    assigns to the token).  Returns (argmax int64, max, lse, conf)."""
    logits = np.atleast_2d(logits)
    am = np.argmax(logits, axis=1)
    mx = logits[np.arange(logits.shape[0]), am]
    z = np.exp(logits - mx[:, None]).sum(axis=1)
    lse = mx + np.log(z)
    conf = 1.0 / z
    return am, mx, lse, conf


def threshold_unmask(conf, argmax, tokens, masked, win_lo: int, tau):
    """Confidence-aware parallel unmasking inside the active window.

    Candidates are the masked positions win_lo + r, r < len(conf).  Every
    candidate whose confidence exceeds tau is unmasked to its argmax (v2
    notes, Key design 3; v1 article, Core technique 2).  If candidates exist
    and none passes, the single most confident one is unmasked (lowest
    position on ties), so tau = 1.0 decodes one token per step.  The
    comparison runs in the precision of ``conf``/``tau`` as given.
    Returns (tokens, masked, picked positions ascending).
    """
    tokens = np.array(tokens, copy=True)
    masked = np.array(masked, dtype=bool, copy=True)
    cand = [r for r in range(len(conf)) if masked[win_lo + r]]
    picked = [r for r in cand if conf[r] > tau]
    if not picked and cand:
        best = max(conf[r] for r in cand)
        picked = [min(r for r in cand if conf[r] == best)]
    for r in picked:
        tokens[win_lo + r] = argmax[r]
        masked[win_lo + r] = False
    return tokens, masked, [win_lo + r for r in picked]


# ==========================================================================
# per-sequence decoding state
# ==========================================================================
@dataclass
class Seq:
    """One sequence: block-level cache, carry row and current block.

    cache_k / cache_v [L, Hkv, d]: K/V of every committed position (the
    block-level cache, v2 notes Key design 3).  carry [hidden]: output row of
    the last committed position.  history: clean token ids of the committed
    positions, when known (None for a synthetic cache).  tokens / masked [D]:
    current block.  plant [D, hidden]: synthetic offset on the block's input
    rows (zeros unless a workload plants peaked logits).  snap_*: DualCache
    snapshot of the in-block K/V and of the row feeding the window's first
    position.
    """
    cache_k: np.ndarray
    cache_v: np.ndarray
    carry: np.ndarray
    history: list | None
    tokens: np.ndarray
    masked: np.ndarray
    plant: np.ndarray
    snap_k: np.ndarray | None = None
    snap_v: np.ndarray | None = None
    snap_h: np.ndarray | None = None
    window: int = 0

    @property
    def L(self) -> int:
        return self.cache_k.shape[0]


@dataclass
class StepResult:
    """What one refinement step computed for one sequence."""
    H: np.ndarray           # output rows computed in this step
    rows: np.ndarray        # block rows those outputs belong to
    src: np.ndarray         # [S, hidden] row feeding each window position
    argmax: np.ndarray
    maxlogit: np.ndarray
    lse: np.ndarray
    conf: np.ndarray
    picked: list
    K: np.ndarray           # fresh in-block K/V of this step
    V: np.ndarray


def new_block(seq: Seq, D: int, hidden: int, plant=None) -> None:
    seq.tokens = np.zeros(D, dtype=np.int64)
    seq.masked = np.ones(D, dtype=bool)
    seq.plant = np.zeros((D, hidden)) if plant is None else np.asarray(plant, dtype=F64)
    seq.window = 0
    seq.snap_k = seq.snap_v = seq.snap_h = None


def prefill(model: Model, prompt, D: int) -> Seq:
    """Process a block-aligned prompt under the same hybrid mask as decoding
    (v2 notes, Framework: the mask is the same in training and inference).
    The cache holds every prompt row's K/V; the carry is the last row."""
    prompt = np.asarray(prompt)
    P = len(prompt)
    assert P % D == 0 and P > 0
    X = embed(model, prompt, np.zeros(P, dtype=bool))
    Q, K, V = project(model, X)
    pos = np.arange(P)
    O, _ = attention(Q, K, V, visible(pos, pos, D), model.G)
    H = output(model, X, O)
    hidden = X.shape[1]
    return Seq(K, V, H[P - 1], list(prompt), np.zeros(D, dtype=np.int64),
               np.ones(D, dtype=bool), np.zeros((D, hidden)))


def _block_forward(model: Model, seq: Seq, rows, blk_k, blk_v, X_rows, D: int):
    """Queries at block rows ``rows`` (positions L + rows) attend over every
    committed row plus the D in-block rows ``blk_k/blk_v``."""
    L = seq.L
    Q, _, _ = project(model, X_rows)
    K_all = np.concatenate([seq.cache_k, blk_k], axis=0)
    V_all = np.concatenate([seq.cache_v, blk_v], axis=0)
    vis = visible(L + np.asarray(rows), np.arange(L + D), D)
    O, _ = attention(Q, K_all, V_all, vis, model.G)
    return output(model, X_rows, O)


def _decide(model: Model, seq: Seq, s: int, S: int, tau, src) -> tuple:
    logits = lm_logits(model.Wlm, src)
    am, mx, lse, conf = confidence(logits)
    seq.tokens, seq.masked, picked = threshold_unmask(conf, am, seq.tokens, seq.masked, s * S, tau)
    return am, mx, lse, conf, picked


def e_step(model: Model, seq: Seq, s: int, S: int, tau, D: int) -> StepResult:
    """Exact refinement step for window s.

    Every block row is recomputed from the current tokens (masked rows use
    the [MASK] embedding), attending over the block-level cache and the whole
    block.  The in-block K/V of all D rows and the row feeding position s*S
    become the DualCache snapshot for the window (refresh at the start of a
    sub-block).  Window position j is predicted from output row j-1 (token
    shift, v2 notes Key design 2); position 0 uses the carry.
    """
    assert seq.L % D == 0
    X = embed(model, seq.tokens, seq.masked, seq.plant)
    _, K, V = project(model, X)
    H = _block_forward(model, seq, np.arange(D), K, V, X, D)
    seq.snap_k, seq.snap_v = K, V
    seq.snap_h = H[shift_row(s * S)] if s > 0 else seq.carry
    src = np.stack([H[shift_row(j)] if shift_row(j) >= 0 else seq.carry
                    for j in range(s * S, s * S + S)])
    am, mx, lse, conf, picked = _decide(model, seq, s, S, tau, src)
    seq.window = s
    return StepResult(H, np.arange(D), src, am, mx, lse, conf, picked, K, V)


def dc_step(model: Model, seq: Seq, s: int, S: int, tau, D: int) -> StepResult:
    """DualCache refinement step for window s (v2 notes Key design 3; v1
    article Core technique 1).

    Only the S window rows are recomputed.  The K/V of every other in-block
    row (decoded prefix and masked suffix of the block) come from the
    snapshot taken by the window's exact step, and so does the row feeding
    the window's first position.
    """
    assert seq.snap_k is not None and seq.window == s
    lo = s * S
    rows = np.arange(lo, lo + S)
    X = embed(model, seq.tokens[rows], seq.masked[rows], seq.plant[rows])
    _, Kw, Vw = project(model, X)
    blk_k = seq.snap_k.copy()
    blk_v = seq.snap_v.copy()
    blk_k[rows] = Kw
    blk_v[rows] = Vw
    H = _block_forward(model, seq, rows, blk_k, blk_v, X, D)
    src = np.stack([H[shift_row(j) - lo] if shift_row(j) >= lo else seq.snap_h
                    for j in range(lo, lo + S)])
    am, mx, lse, conf, picked = _decide(model, seq, s, S, tau, src)
    return StepResult(H, rows, src, am, mx, lse, conf, picked, Kw, Vw)


def commit(model: Model, seq: Seq, D: int) -> np.ndarray:
    """Finished block -> block-level cache (v2 notes Key design 3; v2 news,
    hierarchical cache).  A forward pass over the final clean block gives the
    K/V appended to the cache and the new carry (its last output row)."""
    assert not seq.masked.any()
    X = embed(model, seq.tokens, seq.masked, seq.plant)
    _, K, V = project(model, X)
    H = _block_forward(model, seq, np.arange(D), K, V, X, D)
    seq.cache_k = np.concatenate([seq.cache_k, K], axis=0)
    seq.cache_v = np.concatenate([seq.cache_v, V], axis=0)
    seq.carry = H[D - 1]
    if seq.history is not None:
        seq.history = list(seq.history) + [int(t) for t in seq.tokens]
    return H


def full_recompute(model: Model, history, block_tokens, block_masked, D: int, block_plant=None):
    """The same model on the whole sequence [committed clean tokens | current
    noisy block] with the hybrid mask and no cache: the inference restriction
    of the 2L training layout (v2 notes, Key design 2), where the clean copy
    of the current block is never visible.  Returns (H, K, V) for all rows."""
    history = np.asarray(history, dtype=np.int64)
    L = len(history)
    toks = np.concatenate([history, np.asarray(block_tokens, dtype=np.int64)])
    msk = np.concatenate([np.zeros(L, dtype=bool), np.asarray(block_masked, dtype=bool)])
    X = embed(model, toks, msk)
    if block_plant is not None:
        X[L:] += np.asarray(block_plant, dtype=F64)
    Q, K, V = project(model, X)
    pos = np.arange(len(toks))
    O, _ = attention(Q, K, V, visible(pos, pos, D), model.G)
    return output(model, X, O), K, V


def decode_block(model: Model, seqs: list, D: int, S: int, tau, mode: str = "dual",
                 lockstep: bool = True, on_step=None, max_steps: int = 10_000) -> None:
    """Decode the current block of every sequence, then commit it.

    Windows of S positions go left to right (sub-block decoding, v2 notes
    Key design 4).  Each window starts with an exact step (which refreshes
    the DualCache snapshot); ``mode == 'dual'`` continues with DualCache
    steps, ``mode == 'exact'`` recomputes the whole block every step.  With
    ``lockstep`` the batch advances a window when every sequence has finished
    it (finished sequences keep stepping but have no candidates); otherwise
    each sequence runs its own loop.  ``on_step(step_idx, s, kind, results)``
    sees each batch step.
    """
    assert D % S == 0
    groups = [seqs] if lockstep else [[q] for q in seqs]
    for group in groups:
        step = 0
        for s in range(D // S):
            first = True
            while any(q.masked[s * S:(s + 1) * S].any() for q in group):
                kind = "E" if (first or mode == "exact") else "DC"
                fn = e_step if kind == "E" else dc_step
                res = [fn(model, q, s, S, tau, D) for q in group]
                if on_step is not None:
                    on_step(step, s, kind, res)
                first = False
                step += 1
                assert step < max_steps
        for q in group:
            commit(model, q, D)


# ==========================================================================
# the four library calls, in their array layouts
# ==========================================================================
def block_attn(q, k_cache, v_cache, kv_len, k_blk, v_blk, q_off: int, D: int):
    """Definition of the hybrid-mask block attention call.

    q [B, n_q, Hq, d]: rows q_off .. q_off+n_q-1 of the in-block buffer.
    k_cache/v_cache [B, Hkv, cap, d]: committed rows [0, kv_len[b]).
    k_blk/v_blk [B, n_blk, Hkv, d]: in-block rows (n_blk = D for a step,
    a multiple of D for a multi-block prefill).  In-block row r sits at
    position kv_len[b] + r.  Returns o [B, n_q, Hq, d] and lse [B, Hq, n_q].
    """
    q = np.asarray(q, dtype=F64)
    B, n_q, Hq, d = q.shape
    Hkv = k_cache.shape[1]
    n_blk = k_blk.shape[1]
    o = np.empty_like(q)
    lse = np.empty((B, Hq, n_q))
    for b in range(B):
        L = int(kv_len[b])
        K = np.concatenate([np.asarray(k_cache[b, :, :L, :], dtype=F64).transpose(1, 0, 2),
                            np.asarray(k_blk[b], dtype=F64)], axis=0)
        V = np.concatenate([np.asarray(v_cache[b, :, :L, :], dtype=F64).transpose(1, 0, 2),
                            np.asarray(v_blk[b], dtype=F64)], axis=0)
        # every committed row is visible; in-block rows follow the hybrid
        # mask by their block index inside the buffer (the committed length
        # is a whole number of blocks, so this is the positional mask)
        vis = np.concatenate([np.ones((n_q, L), dtype=bool),
                              visible(q_off + np.arange(n_q), np.arange(n_blk), D)], axis=1)
        o[b], lse[b] = attention(q[b], K, V, vis, Hq // Hkv)
    return o, lse


def lmhead_confidence(h_src, row_idx, w):
    """Definition of the LM-head + confidence call: output row m uses
    h_src[row_idx[m]] (token shift is expressed through row_idx).
    Returns (argmax, conf, max, lse, logits)."""
    h_src = np.asarray(h_src, dtype=F64).reshape(-1, np.asarray(h_src).shape[-1])
    rows = np.arange(h_src.shape[0]) if row_idx is None else np.asarray(row_idx)
    logits = lm_logits(w, h_src[rows])
    am, mx, lse, conf = confidence(logits)
    return am, conf, mx, lse, logits


def batch_threshold_unmask(conf, argmax, tokens, masked, win_lo: int, tau):
    """Batched form of ``threshold_unmask``: conf/argmax [B, win_len],
    tokens/masked [B, D].  Returns (tokens, masked, n_unmasked [B],
    unmasked_pos [B, win_len] ascending, -1 padded)."""
    B, W = np.asarray(conf).shape
    tokens = np.array(tokens, copy=True)
    masked = np.array(masked, dtype=bool, copy=True)
    n = np.zeros(B, dtype=np.int64)
    pos = -np.ones((B, W), dtype=np.int64)
    for b in range(B):
        tokens[b], masked[b], picked = threshold_unmask(conf[b], argmax[b], tokens[b], masked[b], win_lo, tau)
        n[b] = len(picked)
        pos[b, :len(picked)] = picked
    return tokens, masked, n, pos


def kv_append(k_cache, v_cache, kv_len, k_blk, v_blk, n_rows: int):
    """Definition of the append call: rows [0, n_rows) of the in-block K/V
    go to cache rows [kv_len[b], kv_len[b]+n_rows); kv_len[b] += n_rows."""
    k_cache = np.array(k_cache, copy=True)
    v_cache = np.array(v_cache, copy=True)
    kv_len = np.array(kv_len, copy=True)
    for b in range(k_cache.shape[0]):
        L = int(kv_len[b])
        k_cache[b, :, L:L + n_rows, :] = np.asarray(k_blk[b, :n_rows]).transpose(1, 0, 2)
        v_cache[b, :, L:L + n_rows, :] = np.asarray(v_blk[b, :n_rows]).transpose(1, 0, 2)
        kv_len[b] = L + n_rows
    return k_cache, v_cache, kv_len


# ==========================================================================
# building sequences from the seeded inputs
# ==========================================================================
def seqs_from_inputs(model: Model, cfg, prefix, state, plant=None, carry_plant=None) -> list:
    """Sequences for a workload: prefill+commit for a 'prefill' prefix, the
    synthetic cache/carry otherwise; the current block from ``state``."""
    B, D, hidden = cfg.B, cfg.D, cfg.hidden
    seqs = []
    for b in range(B):
        if prefix.kind == "prefill":
            q = prefill(model, prefix.prompt[b], D)
            comm = prefix.committed[b]
            for blk in range(len(comm) // D):
                q.tokens = np.asarray(comm[blk * D:(blk + 1) * D], dtype=np.int64)
                q.masked = np.zeros(D, dtype=bool)
                q.plant = np.zeros((D, hidden))
                commit(model, q, D)
        else:
            L = int(prefix.kv_len[b])
            q = Seq(np.asarray(prefix.cache_k[b, :, :L, :], dtype=F64).transpose(1, 0, 2).copy(),
                    np.asarray(prefix.cache_v[b, :, :L, :], dtype=F64).transpose(1, 0, 2).copy(),
                    np.asarray(prefix.carry[b], dtype=F64).copy(), None,
                    np.zeros(D, dtype=np.int64), np.ones(D, dtype=bool), np.zeros((D, hidden)))
        q.tokens = np.asarray(state.tokens[b], dtype=np.int64).copy()
        q.masked = np.asarray(state.masked[b], dtype=bool).copy()
        q.plant = np.zeros((D, hidden)) if plant is None else np.asarray(plant[b], dtype=F64)
        if carry_plant is not None:
            q.carry = q.carry + np.asarray(carry_plant[b], dtype=F64)
        q.window = state.window
        seqs.append(q)
    return seqs
