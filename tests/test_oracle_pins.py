"""Pins of the fp64 oracle against things other than itself (CPU only).

P1  block-cached decoding == full recomputation under the hybrid mask
P2  tau = 1.0 unmasks exactly one token per step; with D = S = 1 the whole
    procedure is textbook causal greedy decoding (written out independently
    below)
P3  attention against brute force; softmax rows sum to 1
P4  special cases reducing to a library routine (torch SDPA in float64):
    one block with no prefix = bidirectional attention, D = 1 = causal
    attention, Hkv = Hq = multi-head attention; DualCache step with a fresh
    snapshot == exact step; DualCache refreshed every step == exact mode
P5  LM-head statistics against scipy's logsumexp / softmax
P6  unmask rule against enumeration of every subset of a tiny window
P7  after a commit the cache rows equal the K/V of a full recomputation
P8  lockstep and per-sequence window progression give identical results
P9  permuting the committed keys leaves attention unchanged
P10 a masked position enters as the [MASK] embedding, whatever id it holds
P4 also covers the DualCache window rows: a DualCache step whose window is the
whole block equals the exact step on any token state, and in one layer every
window row of a DualCache step is exact (a row's K/V depend on its own token)
"""
import itertools
import math
from dataclasses import replace

import numpy as np
import pytest
import scipy.special
import torch

import bd_inputs as bi
from oracle import refine as R

TINY = bi.Config(name="tiny", dtype="f32", B=3, Hq=4, Hkv=2, d=8, hidden=32, V=64,
                 D=8, S=4, prefix="prefill", prompt_len=5, n_committed_blocks=1, cap=64)


def tiny_model(cfg=TINY, seed=0, lm_scale=1.0):
    w = bi.make_weights(replace(cfg, lm_scale=lm_scale), seed)
    return R.Model.from_weights(w, cfg)


def tiny_seqs(cfg=TINY, seed=0, lm_scale=1.0, window=0, all_masked=True):
    m = tiny_model(cfg, seed, lm_scale)
    pre = bi.make_prefix(cfg, seed)
    st = bi.make_block_state(cfg, seed, window, all_masked=all_masked)
    return m, R.seqs_from_inputs(m, cfg, pre, st)


def rel(a, b):
    a, b = np.asarray(a, float), np.asarray(b, float)
    return np.abs(a - b).max() / max(np.abs(b).max(), 1e-300)


def sdpa(q, k, v, mask=None, causal=False):
    """torch scaled_dot_product_attention in float64; q [n,H,d], k/v [T,H,d]."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.float64).transpose(1, 0, 2)))
    am = None if mask is None else torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=am, is_causal=causal)
    return o.numpy().transpose(1, 0, 2)


# --------------------------------------------------------------------------
# P3: brute force
# --------------------------------------------------------------------------
def brute_attention(q, k, v, allowed, G):
    n, Hq, d = q.shape
    out = np.zeros_like(q)
    for i in range(n):
        for h in range(Hq):
            g = h // G
            ws = []
            for t in range(k.shape[0]):
                if allowed(i, t):
                    s = sum(q[i, h, c] * k[t, g, c] for c in range(d)) / math.sqrt(d)
                    ws.append((t, s))
            mx = max(s for _, s in ws)
            den = sum(math.exp(s - mx) for _, s in ws)
            for t, s in ws:
                out[i, h] += math.exp(s - mx) / den * v[t, g]
    return out


def test_p3_attention_brute_force():
    rng = np.random.default_rng(3)
    D, n_blk, L = 4, 8, 6
    q = rng.normal(size=(n_blk, 4, 5))
    k = rng.normal(size=(L + n_blk, 2, 5))
    v = rng.normal(size=(L + n_blk, 2, 5))
    qpos = L + np.arange(n_blk)
    # reference: query i sees every cache row and in-block rows of blocks <= its own
    allowed = lambda i, t: t < L or (t - L) // D <= i // D
    ref = brute_attention(q, k, v, allowed, 2)
    vis = np.array([[allowed(i, t) for t in range(L + n_blk)] for i in range(n_blk)])
    o, lse = R.attention(q, k, v, vis, 2)
    assert rel(o, ref) < 1e-12
    # through the call-shaped definition (cache [B,Hkv,cap,d], blk [B,n,Hkv,d])
    kc = np.zeros((1, 2, 16, 5)); vc = np.zeros((1, 2, 16, 5))
    kc[0, :, :L] = k[:L].transpose(1, 0, 2); vc[0, :, :L] = v[:L].transpose(1, 0, 2)
    o2, lse2 = R.block_attn(q[None], kc, vc, np.array([L]), k[None, L:], v[None, L:], 0, D)
    assert rel(o2[0], ref) < 1e-12
    assert rel(lse2[0], lse) < 1e-12
    # closed form for the lse of one row: log sum exp of its visible scores
    h, i = 3, 1
    s = [q[i, h] @ k[t, 1] / math.sqrt(5) for t in range(L + n_blk) if allowed(i, t)]
    assert abs(lse[h, i] - math.log(sum(math.exp(x) for x in s))) < 1e-12


def test_p3_softmax_rows_sum_to_one():
    rng = np.random.default_rng(4)
    q = rng.normal(size=(6, 4, 8)) * 3
    k = rng.normal(size=(20, 2, 8)) * 3
    v = np.ones((20, 2, 8))
    vis = R.visible(np.arange(14, 20), np.arange(20), 4)
    o, _ = R.attention(q, k, v, vis, 2)
    assert np.abs(o - 1.0).max() < 1e-12


def test_p3_two_key_closed_form():
    # two visible keys with scores a, b: o = (e^a v0 + e^b v1) / (e^a + e^b)
    q = np.zeros((1, 1, 4)); q[0, 0, 0] = 2.0
    k = np.zeros((2, 1, 4)); k[0, 0, 0] = 1.0; k[1, 0, 0] = -1.0
    v = np.zeros((2, 1, 4)); v[0, 0, 1] = 1.0; v[1, 0, 2] = 1.0
    o, lse = R.attention(q, k, v, np.ones((1, 2), bool), 1)
    a, b = 2.0 / 2.0, -2.0 / 2.0            # q.k / sqrt(4)
    assert abs(o[0, 0, 1] - math.exp(a) / (math.exp(a) + math.exp(b))) < 1e-15
    assert abs(o[0, 0, 2] - math.exp(b) / (math.exp(a) + math.exp(b))) < 1e-15
    assert abs(lse[0, 0] - math.log(math.exp(a) + math.exp(b))) < 1e-15


# --------------------------------------------------------------------------
# P4: special cases against torch SDPA (float64)
# --------------------------------------------------------------------------
def test_p4_one_block_no_prefix_is_bidirectional():
    rng = np.random.default_rng(5)
    D = 8
    q = rng.normal(size=(1, D, 4, 8)); k = rng.normal(size=(1, D, 2, 8)); v = rng.normal(size=(1, D, 2, 8))
    empty = np.zeros((1, 2, 4, 8))
    o, _ = R.block_attn(q, empty, empty, np.array([0]), k, v, 0, D)
    ref = sdpa(q[0], np.repeat(k[0], 2, axis=1), np.repeat(v[0], 2, axis=1))
    assert rel(o[0], ref) < 1e-12


def test_p4_block_size_one_is_causal():
    rng = np.random.default_rng(6)
    T = 9
    q = rng.normal(size=(1, T, 4, 8)); k = rng.normal(size=(1, T, 2, 8)); v = rng.normal(size=(1, T, 2, 8))
    empty = np.zeros((1, 2, 4, 8))
    o, _ = R.block_attn(q, empty, empty, np.array([0]), k, v, 0, 1)
    ref = sdpa(q[0], np.repeat(k[0], 2, axis=1), np.repeat(v[0], 2, axis=1), causal=True)
    assert rel(o[0], ref) < 1e-12


def test_p4_multi_block_mask_is_causal_to_block_end():
    # a query in block b sees exactly the keys before the end of block b
    rng = np.random.default_rng(7)
    D, T = 4, 12
    q = rng.normal(size=(1, T, 2, 8)); k = rng.normal(size=(1, T, 2, 8)); v = rng.normal(size=(1, T, 2, 8))
    empty = np.zeros((1, 2, 4, 8))
    o, _ = R.block_attn(q, empty, empty, np.array([0]), k, v, 0, D)
    block_end = np.array([(i // D + 1) * D for i in range(T)])
    mask = np.arange(T)[None, :] < block_end[:, None]
    ref = sdpa(q[0], k[0], v[0], mask=mask)
    assert rel(o[0], ref) < 1e-12


def test_p4_gqa_equals_mha_with_shared_heads_and_mha_case():
    rng = np.random.default_rng(8)
    L, D = 8, 4
    q = rng.normal(size=(1, D, 6, 8))
    kc = np.zeros((1, 3, 16, 8)); vc = np.zeros((1, 3, 16, 8))
    kc[0, :, :L] = rng.normal(size=(3, L, 8)); vc[0, :, :L] = rng.normal(size=(3, L, 8))
    kb = rng.normal(size=(1, D, 3, 8)); vb = rng.normal(size=(1, D, 3, 8))
    o, _ = R.block_attn(q, kc, vc, np.array([L]), kb, vb, 0, D)
    K = np.concatenate([kc[0, :, :L].transpose(1, 0, 2), kb[0]])
    V = np.concatenate([vc[0, :, :L].transpose(1, 0, 2), vb[0]])
    # GQA (6 query heads over 3 KV heads): head h reads KV head h // 2
    ref = sdpa(q[0], np.repeat(K, 2, axis=1), np.repeat(V, 2, axis=1))
    assert rel(o[0], ref) < 1e-12
    # Hkv == Hq: plain multi-head attention
    q3 = q[:, :, :3]
    o3, _ = R.block_attn(q3, kc, vc, np.array([L]), kb, vb, 0, D)
    assert rel(o3[0], sdpa(q3[0], K, V)) < 1e-12


def test_p4_dualcache_with_fresh_snapshot_equals_exact_step():
    cfg = replace(TINY, B=2)
    m, seqs = tiny_seqs(cfg, seed=1, window=1, all_masked=False)
    for q in seqs:
        s = 1
        saved = (q.tokens.copy(), q.masked.copy())
        e = R.e_step(m, q, s, cfg.S, 2.0, cfg.D)      # tau 2: fallback only
        q.tokens, q.masked = saved[0].copy(), saved[1].copy()
        dc = R.dc_step(m, q, s, cfg.S, 2.0, cfg.D)
        assert rel(dc.src, e.src) < 1e-12
        assert rel(dc.H, e.H[s * cfg.S:(s + 1) * cfg.S]) < 1e-12
        assert np.array_equal(dc.argmax, e.argmax) and dc.picked == e.picked
        assert rel(dc.conf, e.conf) < 1e-12


def test_p4_dualcache_refreshed_every_step_equals_exact_mode():
    cfg = replace(TINY, B=2)
    m, exact = tiny_seqs(cfg, seed=2, lm_scale=150.0)
    _, dual = tiny_seqs(cfg, seed=2, lm_scale=150.0)
    R.decode_block(m, exact, cfg.D, cfg.S, 0.5, mode="exact")
    for s in range(cfg.D // cfg.S):
        while any(q.masked[s * cfg.S:(s + 1) * cfg.S].any() for q in dual):
            for q in dual:
                saved = (q.tokens.copy(), q.masked.copy())
                R.e_step(m, q, s, cfg.S, 0.5, cfg.D)          # refresh only
                q.tokens, q.masked = saved
                R.dc_step(m, q, s, cfg.S, 0.5, cfg.D)
    for q in dual:
        R.commit(m, q, cfg.D)
    for a, b in zip(exact, dual):
        assert np.array_equal(a.tokens, b.tokens)
        assert rel(a.cache_k, b.cache_k) < 1e-12 and rel(a.carry, b.carry) < 1e-12


def _decode_since_refresh(q, lo, hi, n, rng, V):
    """Unmask n masked positions of [lo, hi) to random ids, as the steps that
    follow a refresh would."""
    idx = rng.choice(np.flatnonzero(q.masked[lo:hi]) + lo, size=n, replace=False)
    q.tokens[idx] = rng.integers(0, V, size=n)
    q.masked[idx] = False


def test_p4_dualcache_whole_block_window_equals_exact_step_on_any_state():
    """S = D: the window is the whole block, so no in-block row lies outside
    it and a DualCache step recomputes all of them.  After any unmasking
    since the refresh it must equal the exact step on the current state."""
    cfg = replace(TINY, B=2, S=TINY.D)
    m, seqs = tiny_seqs(cfg, seed=6)
    rng = np.random.default_rng(13)
    for q in seqs:
        R.e_step(m, q, 0, cfg.S, 2.0, cfg.D)                 # refresh
        _decode_since_refresh(q, 0, cfg.D, 3, rng, cfg.V)
        state = (q.tokens.copy(), q.masked.copy())
        dc = R.dc_step(m, q, 0, cfg.S, 2.0, cfg.D)
        q.tokens, q.masked = state[0].copy(), state[1].copy()
        e = R.e_step(m, q, 0, cfg.S, 2.0, cfg.D)
        assert rel(dc.H, e.H) < 1e-12 and rel(dc.src, e.src) < 1e-12
        assert rel(dc.K, e.K) < 1e-12 and rel(dc.V, e.V) < 1e-12
        assert np.array_equal(dc.argmax, e.argmax) and dc.picked == e.picked


def test_p4_dualcache_window_rows_are_exact_in_one_layer():
    """In a one-layer model a row's K/V are a projection of its own input row,
    and between a refresh and a DualCache step only window positions change,
    so the snapshot K/V of the other rows still equal fresh ones.  The
    DualCache step must then equal the exact step on the current state at
    every window row; only the row feeding the window's first position
    differs: it is the snapshot row, taken before the window changed."""
    cfg = replace(TINY, B=2)
    m, seqs = tiny_seqs(cfg, seed=7, window=1)
    rng = np.random.default_rng(14)
    s, S, D = 1, cfg.S, cfg.D
    lo = s * S
    for q in seqs:
        refresh = R.e_step(m, q, s, S, 2.0, D)
        _decode_since_refresh(q, lo, lo + S, 2, rng, cfg.V)
        state = (q.tokens.copy(), q.masked.copy())
        dc = R.dc_step(m, q, s, S, 2.0, D)
        q.tokens, q.masked = state[0].copy(), state[1].copy()
        e = R.e_step(m, q, s, S, 2.0, D)
        assert rel(dc.H, e.H[lo:lo + S]) < 1e-12
        assert rel(dc.src[1:], e.src[1:]) < 1e-12
        assert rel(dc.src[0], refresh.H[lo - 1]) < 1e-12
        assert rel(dc.src[0], e.H[lo - 1]) > 1e-9


# --------------------------------------------------------------------------
# P10: a masked position enters as the [MASK] embedding
# --------------------------------------------------------------------------
def test_p10_masked_positions_take_the_mask_embedding():
    """v2 notes, Key design 2: a masked position's input is the learnable
    [MASK] embedding (row V of E), whatever id is stored at that position.
    Exact and DualCache steps are unchanged when the ids at masked positions
    change, and change when E[V] changes."""
    cfg = replace(TINY, B=1)
    m, (q0,) = tiny_seqs(cfg, seed=8, window=1, all_masked=False)
    assert q0.masked.sum() >= 2 and (~q0.masked).sum() >= 2
    rng = np.random.default_rng(15)

    def run(model, tokens):
        q = R.Seq(q0.cache_k, q0.cache_v, q0.carry, None, tokens.copy(), q0.masked.copy(), q0.plant)
        e = R.e_step(model, q, 1, cfg.S, 2.0, cfg.D)
        d = R.dc_step(model, q, 1, cfg.S, 2.0, cfg.D)
        return np.concatenate([e.H.ravel(), e.K.ravel(), d.H.ravel(), e.conf, d.conf])

    base = run(m, q0.tokens)
    t2 = q0.tokens.copy()
    t2[q0.masked] = rng.integers(0, cfg.V, int(q0.masked.sum()))
    assert np.array_equal(run(m, t2), base)
    E2 = m.E.copy()
    E2[cfg.V] += 0.05 * rng.standard_normal(cfg.hidden)
    assert rel(run(replace(m, E=E2), q0.tokens), base) > 1e-6
    # an unmasked position is a lookup of its own id
    t3 = q0.tokens.copy()
    j = int(np.flatnonzero(~q0.masked)[0])
    t3[j] = (t3[j] + 1) % cfg.V
    assert rel(run(m, t3), base) > 1e-6


# --------------------------------------------------------------------------
# P1 / P7: block cache is exact
# --------------------------------------------------------------------------
@pytest.mark.parametrize("cfg", [bi.C1, bi.C1_96, TINY], ids=["c1", "c1-96", "tiny"])
@pytest.mark.parametrize("mode", ["exact", "dual"])
def test_p1_block_cache_equals_full_recompute(cfg, mode):
    m = R.Model.from_weights(bi.make_weights(cfg, 0), cfg)
    seqs = R.seqs_from_inputs(m, cfg, bi.make_prefix(cfg, 0), bi.make_block_state(cfg, 0, 0, all_masked=True))
    n_checked = [0]

    def on_step(step, s, kind, results):
        if kind != "E":
            return                      # DualCache steps are approximate by design
        for q, r in zip(seqs, results):
            pre_tokens = q.tokens.copy(); pre_masked = q.masked.copy()
            for pos in r.picked:        # undo this step's unmasking to see its input
                pre_masked[pos] = True; pre_tokens[pos] = 0
            H, _, _ = R.full_recompute(m, q.history, pre_tokens, pre_masked, cfg.D)
            L = len(q.history)
            assert rel(r.H, H[L:]) < 1e-12
            src = np.stack([H[L + j - 1] for j in range(s * cfg.S, (s + 1) * cfg.S)])
            assert rel(r.src, src) < 1e-12
            am, mx, lse, conf = R.confidence(R.lm_logits(m.Wlm, src))
            assert np.array_equal(am, r.argmax) and rel(conf, r.conf) < 1e-12
            n_checked[0] += 1

    R.decode_block(m, seqs, cfg.D, cfg.S, cfg.tau, mode=mode, on_step=on_step)
    assert n_checked[0] > 0
    # P7 + carry: the committed cache and carry equal the clean full recomputation
    for q in seqs:
        H, K, V = R.full_recompute(m, q.history[:-cfg.D], q.tokens, np.zeros(cfg.D, bool), cfg.D)
        assert rel(q.cache_k, K) < 1e-12 and rel(q.cache_v, V) < 1e-12
        assert rel(q.carry, H[-1]) < 1e-12


def test_p7_prefill_then_commit_equals_multi_block_prefill():
    cfg = TINY
    m = tiny_model(cfg)
    pre = bi.make_prefix(cfg, 0)
    toks = np.concatenate([pre.prompt[0], pre.committed[0]])
    a = R.prefill(m, toks, cfg.D)
    b = R.prefill(m, pre.prompt[0], cfg.D)
    b.tokens = pre.committed[0].astype(np.int64); b.masked = np.zeros(cfg.D, bool)
    R.commit(m, b, cfg.D)
    assert rel(a.cache_k, b.cache_k) < 1e-12 and rel(a.cache_v, b.cache_v) < 1e-12
    assert rel(a.carry, b.carry) < 1e-12


# --------------------------------------------------------------------------
# P2: threshold 1.0 and textbook greedy decoding
# --------------------------------------------------------------------------
@pytest.mark.parametrize("mode", ["exact", "dual"])
def test_p2_threshold_one_unmasks_one_token_per_step(mode):
    m, seqs = tiny_seqs(seed=3, lm_scale=400.0)
    counts = []
    R.decode_block(m, seqs, TINY.D, TINY.S, 1.0, mode=mode,
                   on_step=lambda st, s, k, res: counts.extend(len(r.picked) for r in res))
    assert counts and set(counts) == {1}
    # the same inputs at a lower threshold decode several tokens in some step
    m, seqs = tiny_seqs(seed=3, lm_scale=400.0)
    counts = []
    R.decode_block(m, seqs, TINY.D, TINY.S, 0.1, mode=mode,
                   on_step=lambda st, s, k, res: counts.extend(len(r.picked) for r in res))
    assert max(counts) > 1


class TextbookCausalLM:
    """Independent one-layer causal LM with greedy decoding and no cache:
    every new token is the argmax of the LM head applied to the last
    position's output row, recomputed from scratch with a causal mask."""

    def __init__(self, E, Wq, Wk, Wv, Wo, Wlm, Hq, Hkv, d):
        self.__dict__.update(E=E, Wq=Wq, Wk=Wk, Wv=Wv, Wo=Wo, Wlm=np.asarray(Wlm, float),
                             Hq=Hq, Hkv=Hkv, d=d)

    def last_row(self, toks):
        T = len(toks)
        X = self.E[toks]
        q = X @ self.Wq.T; k = X @ self.Wk.T; v = X @ self.Wv.T
        att = np.zeros((self.Hq * self.d,))
        i = T - 1
        for h in range(self.Hq):
            g = h * self.Hkv // self.Hq
            qh = q[i, h * self.d:(h + 1) * self.d]
            sc = [qh @ k[t, g * self.d:(g + 1) * self.d] / math.sqrt(self.d) for t in range(i + 1)]
            mx = max(sc)
            e = [math.exp(x - mx) for x in sc]
            for t in range(i + 1):
                att[h * self.d:(h + 1) * self.d] += e[t] / sum(e) * v[t, g * self.d:(g + 1) * self.d]
        return X[i] + self.Wo @ att

    def greedy(self, prompt, n):
        toks = list(prompt)
        for _ in range(n):
            toks.append(int(np.argmax(self.Wlm @ self.last_row(toks))))
        return toks[len(prompt):]


def test_p2_block_and_subblock_of_one_is_textbook_greedy():
    cfg = replace(TINY, B=1, D=1, S=1)
    m = tiny_model(TINY, seed=4, lm_scale=50.0)
    prompt = bi.make_prefix(TINY, 4).prompt[0][-6:]
    q = R.prefill(m, prompt, 1)
    out = []
    for _ in range(7):
        R.new_block(q, 1, cfg.hidden)
        R.decode_block(m, [q], 1, 1, 0.9, mode="dual")
        out.append(int(q.tokens[0]))
    ref = TextbookCausalLM(m.E, m.Wq, m.Wk, m.Wv, m.Wo, m.Wlm, m.Hq, m.Hkv, m.d).greedy(prompt, 7)
    assert out == ref


# --------------------------------------------------------------------------
# P5: LM-head statistics
# --------------------------------------------------------------------------
def test_p5_lm_head_statistics():
    rng = np.random.default_rng(9)
    h = rng.normal(size=(5, 16))
    W = rng.normal(size=(40, 16)).astype(np.float32)
    logits = h @ W.astype(float).T
    am, conf, mx, lse, lg = R.lmhead_confidence(h, None, W)
    assert rel(lg, logits) < 1e-14
    assert np.array_equal(am, np.argmax(logits, axis=1))
    assert rel(lse, scipy.special.logsumexp(logits, axis=1)) < 1e-14
    assert rel(conf, scipy.special.softmax(logits, axis=1).max(axis=1)) < 1e-13
    assert np.all(conf >= 1 / 40) and np.all(conf <= 1) and np.all(lse >= mx)
    assert rel(-np.log(conf), lse - mx) < 1e-12
    # row selection (token shift through row_idx)
    am2, conf2, *_ = R.lmhead_confidence(h, np.array([4, 0, 0]), W)
    assert np.array_equal(am2, am[[4, 0, 0]])
    # tie: lowest id wins
    lg = np.array([[0.0, 3.0, 1.0, 3.0]])
    a, *_ = R.confidence(lg)
    assert a[0] == 1


# --------------------------------------------------------------------------
# P6: unmask rule against enumeration
# --------------------------------------------------------------------------
def _enumerated_unmask(conf, masked, tau):
    """The unique subset P of the window with: P within the candidates; P
    holds every candidate above tau and nothing else if one is above tau;
    otherwise P is one most-confident candidate, the lowest on ties; P is
    empty only without candidates."""
    W = len(conf)
    cand = {r for r in range(W) if masked[r]}
    ok = []
    for bits in range(1 << W):
        P = {r for r in range(W) if bits >> r & 1}
        if not P <= cand:
            continue
        above = {r for r in cand if conf[r] > tau}
        if above:
            good = P == above
        elif cand:
            good = (len(P) == 1 and conf[min(P)] == max(conf[r] for r in cand)
                    and all(conf[r] < conf[min(P)] for r in cand if r < min(P)))
        else:
            good = not P
        if good:
            ok.append(P)
    assert len(ok) == 1
    return sorted(ok[0])


def test_p6_unmask_against_enumeration():
    rng = np.random.default_rng(10)
    for trial in range(400):
        W = 6
        conf = rng.choice([0.1, 0.5, 0.9, 0.95, 0.99, rng.random()], size=W)
        masked = rng.random(W) < 0.6
        tau = rng.choice([0.9, 1.0, 0.5])
        toks = rng.integers(0, 100, W)
        am = rng.integers(0, 100, W)
        t2, m2, picked = R.threshold_unmask(conf, am, toks, masked, 0, tau)
        assert picked == _enumerated_unmask(conf, masked, tau)
        assert (len(picked) > 0) == bool(masked.any())
        for r in range(W):
            assert t2[r] == (am[r] if r in picked else toks[r])
            assert m2[r] == (masked[r] and r not in picked)
        # lowering the threshold gives a superset
        _, _, p_low = R.threshold_unmask(conf, am, toks, masked, 0, tau - 0.3)
        assert set(picked) <= set(p_low)


def test_p6_threshold_is_strict():
    conf = np.array([0.9, 0.5], dtype=np.float32)
    _, _, picked = R.threshold_unmask(conf, [1, 2], [0, 0], [True, True], 0, np.float32(0.9))
    assert picked == [0]       # not above tau: the fallback picks it alone
    conf = np.array([0.9, 0.95], dtype=np.float32)
    _, _, picked = R.threshold_unmask(conf, [1, 2], [0, 0], [True, True], 0, np.float32(0.9))
    assert picked == [1]


# --------------------------------------------------------------------------
# P8 / P9
# --------------------------------------------------------------------------
def test_p8_lockstep_equals_per_sequence():
    m, a = tiny_seqs(seed=5, lm_scale=300.0)
    _, b = tiny_seqs(seed=5, lm_scale=300.0)
    R.decode_block(m, a, TINY.D, TINY.S, 0.9, lockstep=True)
    R.decode_block(m, b, TINY.D, TINY.S, 0.9, lockstep=False)
    for x, y in zip(a, b):
        assert np.array_equal(x.tokens, y.tokens)
        assert rel(x.cache_k, y.cache_k) == 0 and rel(x.carry, y.carry) == 0


def test_p9_permuting_committed_keys():
    rng = np.random.default_rng(11)
    L, D = 24, 8
    q = rng.normal(size=(1, D, 4, 8))
    kc = np.zeros((1, 2, 32, 8)); vc = np.zeros((1, 2, 32, 8))
    kc[0, :, :L] = rng.normal(size=(2, L, 8)); vc[0, :, :L] = rng.normal(size=(2, L, 8))
    kb = rng.normal(size=(1, D, 2, 8)); vb = rng.normal(size=(1, D, 2, 8))
    o, lse = R.block_attn(q, kc, vc, np.array([L]), kb, vb, 0, D)
    perm = rng.permutation(L)
    kc2 = kc.copy(); vc2 = vc.copy()
    kc2[0, :, :L] = kc[0, :, perm].transpose(1, 0, 2); vc2[0, :, :L] = vc[0, :, perm].transpose(1, 0, 2)
    o2, lse2 = R.block_attn(q, kc2, vc2, np.array([L]), kb, vb, 0, D)
    assert rel(o2, o) < 1e-12 and rel(lse2, lse) < 1e-12


def test_kv_append_definition():
    rng = np.random.default_rng(12)
    kc = rng.normal(size=(2, 2, 16, 4)); vc = rng.normal(size=(2, 2, 16, 4))
    kb = rng.normal(size=(2, 4, 2, 4)); vb = rng.normal(size=(2, 4, 2, 4))
    k2, v2, n2 = R.kv_append(kc, vc, np.array([3, 8]), kb, vb, 4)
    assert list(n2) == [7, 12]
    assert np.array_equal(k2[1, 1, 8:12], kb[1, :, 1]) and np.array_equal(v2[0, 0, 3:7], vb[0, :, 0])
    assert np.array_equal(k2[0, :, :3], kc[0, :, :3]) and np.array_equal(k2[0, :, 7:], kc[0, :, 7:])


def test_tiny_lm_scale_is_the_frozen_one():
    """The tiny workload's LM-head scale is the one the committed golden
    script chose on the oracle: ~30% of candidate rows above tau, none near it."""
    import json, os, sys
    here = os.path.dirname(os.path.abspath(__file__))
    rec = json.load(open(os.path.join(here, "golden", "c1_lm_scale.json")))
    assert bi.C1.lm_scale == rec["lm_scale"]
    sys.path.insert(0, os.path.join(here, "golden"))
    from make_tiny_scale import candidate_confs
    c = candidate_confs(bi.C1.lm_scale)
    assert abs(np.mean(c > bi.C1.tau) - 0.30) <= 0.06
    assert np.min(np.abs(c - bi.C1.tau)) >= 2e-3
