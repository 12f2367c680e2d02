"""Pins of the multi-layer oracle (oracle/model.py) against facts that do not
come from the oracle itself: closed forms, a hand-worked rotation, library
routines, the already pinned one-layer oracle, and the exactness of the
block-level cache (a cached step must equal the cache-free forward pass)."""
import math

import numpy as np
import pytest
from scipy.special import expit

import bd_inputs as bi
from oracle import model as OM
from oracle import refine as R


# ---------------------------------------------------------------- RMSNorm
def test_rmsnorm_closed_form_and_scale_invariance():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 64)) * 3.0
    eps = 1e-3
    y = OM.rmsnorm(x, eps)
    m = np.mean(x * x, axis=1)
    np.testing.assert_allclose(np.mean(y * y, axis=1), m / (m + eps), rtol=1e-13)
    np.testing.assert_allclose(OM.rmsnorm(7.5 * x, 0.0), OM.rmsnorm(x, 0.0), rtol=1e-13)
    # one element: x / |x|
    np.testing.assert_allclose(OM.rmsnorm(np.array([[-4.0]]), 0.0), [[-1.0]])


# ----------------------------------------------------------------- rotary
def test_rope_hand_example_fixes_pairing_and_sign():
    """d = 4, theta = 1e4: frequencies 1 and 1e4^(-1/2) = 0.01.  Rotate-half
    pairs (x0, x2) and (x1, x3); at position pi/2 the first pair turns by a
    quarter turn: (1, 3) -> (1*0 - 3*1, 3*0 + 1*1) = (-3, 1)."""
    x = np.array([[[1.0, 2.0, 3.0, 4.0]]])
    y = OM.rope(x, [math.pi / 2], 1e4)[0, 0]
    a1 = math.pi / 2 * 0.01
    np.testing.assert_allclose(y[[0, 2]], [-3.0, 1.0], atol=1e-14)
    np.testing.assert_allclose(y[[1, 3]], [2 * math.cos(a1) - 4 * math.sin(a1), 4 * math.cos(a1) + 2 * math.sin(a1)],
                               rtol=1e-14)


def test_rope_identity_norms_relative_positions_and_composition():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((6, 3, 16))
    k = rng.standard_normal((6, 3, 16))
    pos_q = rng.integers(0, 1000, 6)
    pos_k = rng.integers(0, 1000, 6)
    th = 1e6
    np.testing.assert_allclose(OM.rope(q, np.zeros(6), th), q, atol=1e-15)
    rq = OM.rope(q, pos_q, th)
    pn = lambda a: a[..., :8] ** 2 + a[..., 8:] ** 2
    np.testing.assert_allclose(pn(rq), pn(q), rtol=1e-12)
    for t in (1, 17, 333):
        a = np.einsum("nhd,nhd->nh", OM.rope(q, pos_q, th), OM.rope(k, pos_k, th))
        b = np.einsum("nhd,nhd->nh", OM.rope(q, pos_q + t, th), OM.rope(k, pos_k + t, th))
        np.testing.assert_allclose(a, b, rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(OM.rope(OM.rope(q, pos_q, th), pos_k, th), OM.rope(q, pos_q + pos_k, th), atol=1e-11)


# ------------------------------------------------------------------- SiLU
def test_silu_matches_logistic():
    z = np.linspace(-30, 30, 601)
    np.testing.assert_allclose(OM.silu(z), z * expit(z), rtol=1e-13, atol=1e-300)
    assert OM.silu(0.0) == 0.0


# ------------------------------------------- reduction to the one-layer model
def _one_layer_pair(seed=3):
    cfg = bi.C1
    w = bi.make_weights(cfg, seed)
    one = R.Model.from_weights(w, cfg)
    lm = OM.LM(one.E, [OM.Layer(one.Wq, one.Wk, one.Wv, one.Wo)], one.Wlm, cfg.Hq, cfg.Hkv, cfg.d,
               norm=False, use_rope=False, mlp=False)
    return cfg, one, lm


def test_reduces_to_one_layer_oracle():
    """Norm, rotary and MLP off, one layer: prefill, exact and DualCache
    steps and commit equal the one-layer oracle's."""
    cfg, one, lm = _one_layer_pair()
    D, S = cfg.D, cfg.S
    prompt = bi._rng(3, bi.TID["prompt"]).integers(0, cfg.V, size=2 * D)
    a = R.prefill(one, prompt, D)
    b = OM.prefill(lm, prompt, D)
    np.testing.assert_allclose(b.cache_k[0], a.cache_k, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(b.carry, a.carry, rtol=1e-12, atol=1e-15)
    R.new_block(a, D, cfg.hidden)
    OM.new_block(b, D)
    for s in range(D // S):
        ra = R.e_step(one, a, s, S, 1.0, D)
        rb = OM.e_step(lm, b, s, S, 1.0, D)
        np.testing.assert_allclose(rb.H, ra.H, rtol=1e-11, atol=1e-14)
        np.testing.assert_allclose(rb.conf, ra.conf, rtol=1e-10)
        assert rb.picked == ra.picked
        while a.masked[s * S:(s + 1) * S].any():
            ra = R.dc_step(one, a, s, S, 1.0, D)
            rb = OM.dc_step(lm, b, s, S, 1.0, D)
            np.testing.assert_allclose(rb.H, ra.H, rtol=1e-11, atol=1e-14)
            assert rb.picked == ra.picked
    R.commit(one, a, D)
    OM.commit(lm, b, D)
    np.testing.assert_allclose(b.cache_v[0], a.cache_v, rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(b.carry, a.carry, rtol=1e-11, atol=1e-14)


# ----------------------------------------------------------- cache exactness
def _small(seed=4):
    cfg = bi.M1
    w = bi.make_model_weights(cfg, seed)
    return cfg, OM.LM.from_weights(w, cfg), bi.make_prompts(cfg, seed)


def test_exact_step_equals_cache_free_forward():
    """The exact step's final rows (cache of earlier blocks + the whole noisy
    block) equal the cache-free forward over [history | block]; so do the
    rows after a committed block."""
    cfg, m, prompts = _small()
    D, S = cfg.D, cfg.S
    q = OM.prefill(m, prompts[0], D)
    OM.new_block(q, D)
    q.masked[:5] = False
    q.tokens[:5] = [3, 1, 4, 1, 5]
    r = OM.e_step(m, q, 0, S, cfg.tau, D)
    full = OM.full_forward(m, q.history, np.where(np.arange(D) < 5, [3, 1, 4, 1, 5] + [0] * (D - 5), 0),
                           np.arange(D) >= 5, D)
    np.testing.assert_allclose(r.H, full[-D:], rtol=1e-10, atol=1e-13)
    # the carry (last prompt row) equals the cache-free row too
    np.testing.assert_allclose(q.carry, full[len(q.history) - 1], rtol=1e-10, atol=1e-13)


def test_dualcache_pass_with_current_snapshot_equals_exact_pass():
    cfg, m, prompts = _small(5)
    D, S = cfg.D, cfg.S
    q = OM.prefill(m, prompts[1], D)
    OM.new_block(q, D)
    X = OM.embed(m, q.tokens, q.masked)
    H, Ks, Vs = OM.forward_rows(m, q, X, np.arange(D), D)
    rows = np.arange(8, 16)
    Hw, _, _ = OM.forward_rows(m, q, X[rows], rows, D, Ks, Vs)
    np.testing.assert_allclose(Hw, H[rows], rtol=1e-11, atol=1e-14)


def test_dualcache_whole_block_window_equals_exact_step_on_any_state():
    """S = D: every in-block row is a window row, so a DualCache step
    recomputes all of them through every layer and must equal the exact step
    on the current state, including after unmasking since the refresh."""
    cfg, m, prompts = _small(8)
    D = cfg.D
    rng = np.random.default_rng(21)
    q = OM.prefill(m, prompts[0], D)
    OM.new_block(q, D)
    OM.e_step(m, q, 0, D, 2.0, D)                         # refresh
    idx = rng.choice(np.flatnonzero(q.masked), size=5, replace=False)
    q.tokens[idx] = rng.integers(0, cfg.V, size=5)
    q.masked[idx] = False
    state = (q.tokens.copy(), q.masked.copy())
    dc = OM.dc_step(m, q, 0, D, 2.0, D)
    q.tokens, q.masked = state[0].copy(), state[1].copy()
    e = OM.e_step(m, q, 0, D, 2.0, D)
    np.testing.assert_allclose(dc.H, e.H, rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(dc.src, e.src, rtol=1e-11, atol=1e-14)
    for l in range(cfg.n_layers):
        np.testing.assert_allclose(dc.K[l], e.K[l], rtol=1e-11, atol=1e-14)
    assert dc.picked == e.picked


def test_masked_positions_take_the_mask_embedding():
    """v2 notes, Key design 2: masked positions enter as row V of E whatever
    id they hold; the step changes when E[V] changes."""
    cfg, m, prompts = _small(9)
    D, S = cfg.D, cfg.S
    rng = np.random.default_rng(22)
    base_q = OM.prefill(m, prompts[0], D)
    OM.new_block(base_q, D)
    base_q.tokens[:S] = rng.integers(0, cfg.V, S)
    base_q.masked[:S] = False

    def run(model, tokens):
        q = OM.MSeq(base_q.cache_k, base_q.cache_v, base_q.carry, list(base_q.history), tokens.copy(),
                    base_q.masked.copy())
        e = OM.e_step(model, q, 1, S, 2.0, D)
        d = OM.dc_step(model, q, 1, S, 2.0, D)
        return np.concatenate([e.H.ravel(), d.H.ravel(), e.conf, d.conf])

    base = run(m, base_q.tokens)
    t2 = base_q.tokens.copy()
    t2[base_q.masked] = rng.integers(0, cfg.V, int(base_q.masked.sum()))
    np.testing.assert_array_equal(run(m, t2), base)
    E2 = m.E.copy()
    E2[cfg.V] += 0.05 * rng.standard_normal(E2.shape[1])
    m2 = OM.LM(E2, m.layers, m.Wlm, m.Hq, m.Hkv, m.d, m.eps, m.theta)
    assert np.abs(run(m2, base_q.tokens) - base).max() > 1e-6 * np.abs(base).max()


def test_prefill_of_longer_prompt_equals_prefill_then_commit():
    cfg, m, prompts = _small(6)
    D = cfg.D
    p = prompts[0]
    a = OM.prefill(m, p, D)
    b = OM.prefill(m, p[:D], D)
    OM.new_block(b, D)
    b.tokens = np.asarray(p[D:2 * D], dtype=np.int64)
    b.masked[:] = False
    OM.commit(m, b, D)
    for l in range(cfg.n_layers):
        np.testing.assert_allclose(b.cache_k[l], a.cache_k[l], rtol=1e-10, atol=1e-13)
        np.testing.assert_allclose(b.cache_v[l], a.cache_v[l], rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(b.carry, a.carry, rtol=1e-10, atol=1e-13)


def test_generate_runs_blocks_and_every_step_unmasks():
    cfg, m, prompts = _small(7)
    steps = []
    seqs = OM.generate(m, prompts, cfg.n_blocks, cfg.D, cfg.S, cfg.tau,
                       on_step=lambda i, s, kind, res: steps.append((kind, [len(r.picked) for r in res])))
    for q in seqs:
        assert len(q.history) == cfg.prompt_len + cfg.n_blocks * cfg.D
        assert q.L == cfg.cap
    assert all(min(n) >= 0 and max(n) >= 1 for _, n in steps)
    assert sum(1 for k, _ in steps if k == "E") == cfg.n_blocks * cfg.D // cfg.S
