"""Pins of the training-form oracle (oracle/train.py) against facts that do
not come from it: a mask worked out by hand, the already pinned inference
oracle (the clean half is the block-causal prefill; a noisy block is an
exact refinement step over the clean prefix, and its token-shift rows are
the step's source rows, carry included), a closed form of the loss and a
library log-softmax."""
import math
import os

import numpy as np
import pytest
from scipy.special import log_softmax

import bd_inputs as bi
from oracle import refine as R
from oracle import train as TR

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _model(seed=0):
    cfg = bi.C1
    return R.Model.from_weights(bi.make_weights(cfg, seed), cfg), cfg


def _sample(rng, L, V, p=0.5):
    return rng.integers(0, V, L), rng.random(L) < p


def test_mask_matches_the_hand_worked_example():
    want = np.loadtxt(os.path.join(GOLDEN, "mask_2L_L4_D2.txt"), dtype=int).astype(bool)
    assert np.array_equal(TR.mask_2L(4, 2), want)


@pytest.mark.parametrize("L,D", [(96, 32), (32, 8)])
def test_clean_half_is_the_block_causal_prefill(L, D):
    model, cfg = _model(1)
    rng = np.random.default_rng(2)
    x0, m = _sample(rng, L, cfg.V)
    H = TR.forward_2L(model, x0, m, D)[0]
    seq = R.prefill(model, x0, D)
    ref = R.full_recompute(model, x0[:L - D], x0[L - D:], np.zeros(D, bool), D)[0]
    np.testing.assert_allclose(H[L:], ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(H[2 * L - 1], seq.carry, rtol=1e-12, atol=1e-12)


def _exact_step_of_block(model, x0, m, b, D):
    """The inference oracle's exact step for block b of a sequence whose
    committed prefix is the clean x0 of blocks < b (window = whole block)."""
    hid = model.E.shape[1]
    if b == 0:
        seq = R.Seq(np.zeros((0, model.Hkv, model.d)), np.zeros((0, model.Hkv, model.d)), np.zeros(hid), [],
                    np.zeros(D, dtype=np.int64), np.ones(D, bool), np.zeros((D, hid)))
    else:
        seq = R.prefill(model, x0[:b * D], D)
    seq.tokens = np.where(m[b * D:(b + 1) * D], 0, x0[b * D:(b + 1) * D]).astype(np.int64)
    seq.masked = m[b * D:(b + 1) * D].copy()
    return R.e_step(model, seq, 0, D, 2.0, D)       # tau 2: nothing passes but the fallback


@pytest.mark.parametrize("L,D", [(96, 32), (32, 8)])
def test_noisy_block_is_an_exact_step_over_the_clean_prefix(L, D):
    model, cfg = _model(3)
    rng = np.random.default_rng(4)
    x0, m = _sample(rng, L, cfg.V)
    H = TR.forward_2L(model, x0, m, D)[0]
    for b in range(L // D):
        st = _exact_step_of_block(model, x0, m, b, D)
        np.testing.assert_allclose(H[b * D:(b + 1) * D], st.H, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("L,D", [(96, 32), (32, 8)])
def test_token_shift_rows_are_the_steps_source_rows(L, D):
    """Masked position i is predicted from the row the exact step uses for
    it: output row i-1 inside the block, the carry at a block start."""
    model, cfg = _model(5)
    rng = np.random.default_rng(6)
    x0, m = _sample(rng, L, cfg.V)
    pos, rows, _, H = TR.view_nll(model, x0, m, D)
    for b in range(L // D):
        st = _exact_step_of_block(model, x0, m, b, D)
        for k, i in enumerate(pos):
            if i // D == b:
                np.testing.assert_allclose(H[rows[k]], st.src[i - b * D], rtol=1e-12, atol=1e-12)


def test_a_single_masked_position_is_the_only_supervised_one():
    m = np.zeros(64, bool)
    m[37] = True
    assert list(TR.supervised(m)) == [37]
    m[0] = True                     # position 0 has no predecessor row
    assert list(TR.supervised(m)) == [37]


def test_complementary_views_supervise_every_position_once():
    model, cfg = _model(7)
    rng = np.random.default_rng(8)
    L, D = 64, 32
    x0, m = _sample(rng, L, cfg.V)
    seen = np.zeros(L, int)
    for v in TR.complementary_views(m):
        seen[TR.supervised(v)] += 1
    assert seen[0] == 0 and np.all(seen[1:] == 1)
    assert TR.sample_loss(model, x0, m, D)[1] == L - 1


def test_zero_head_gives_log_vocab_per_token():
    model, cfg = _model(9)
    model.Wlm = np.zeros_like(model.Wlm)
    rng = np.random.default_rng(10)
    L, D = 64, 32
    x0, m = _sample(rng, L, cfg.V)
    total, count = TR.sample_loss(model, x0, m, D)
    assert count == L - 1
    assert total == pytest.approx((L - 1) * math.log(cfg.V), rel=1e-13)


def test_token_nll_matches_library_log_softmax():
    rng = np.random.default_rng(11)
    logits = rng.standard_normal((7, 50)) * 4
    tgt = rng.integers(0, 50, 7)
    np.testing.assert_allclose(TR.token_nll(logits, tgt), -log_softmax(logits, axis=1)[np.arange(7), tgt],
                               rtol=1e-13, atol=1e-13)
