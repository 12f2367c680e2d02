"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins
in test_oracle_pins.py catch each one.  Nothing here touches the HIP path."""
import math

import numpy as np
import pytest

import test_oracle_pins as P
from oracle import refine as R

_orig_attention = R.attention
_orig_confidence = R.confidence
_orig_threshold = R.threshold_unmask
_orig_output = R.output
_orig_embed = R.embed


def _attention_no_scale(Q, K, V, vis, G):
    return _orig_attention(Q * math.sqrt(Q.shape[2]), K, V, vis, G)


def _attention_no_max_shift_wrong_lse(Q, K, V, vis, G):
    o, lse = _orig_attention(Q, K, V, vis, G)
    return o, lse - 1.0


def _confidence_inverted(logits):
    am, mx, lse, conf = _orig_confidence(logits)
    return am, mx, lse, np.exp(lse - mx)


def _confidence_argmax_last(logits):
    am, mx, lse, conf = _orig_confidence(logits)
    lg = np.atleast_2d(logits)
    am = lg.shape[1] - 1 - np.argmax(lg[:, ::-1], axis=1)
    return am, mx, lse, conf


def _threshold_ge(conf, argmax, tokens, masked, win_lo, tau):
    return _orig_threshold(conf, argmax, tokens, masked, win_lo, np.nextafter(tau, -np.inf))


def _threshold_no_fallback(conf, argmax, tokens, masked, win_lo, tau):
    tokens = np.array(tokens, copy=True); masked = np.array(masked, dtype=bool, copy=True)
    picked = [r for r in range(len(conf)) if masked[win_lo + r] and conf[r] > tau]
    for r in picked:
        tokens[win_lo + r] = argmax[r]; masked[win_lo + r] = False
    return tokens, masked, [win_lo + r for r in picked]


def _threshold_fallback_highest_index(conf, argmax, tokens, masked, win_lo, tau):
    t, m, picked = _orig_threshold(conf, argmax, tokens, masked, win_lo, tau)
    cand = [r for r in range(len(conf)) if masked[win_lo + r]]
    if cand and not any(conf[r] > tau for r in cand):
        best = max(conf[r] for r in cand)
        r = max(r for r in cand if conf[r] == best)
        t = np.array(tokens, copy=True); m = np.array(masked, dtype=bool, copy=True)
        t[win_lo + r] = argmax[r]; m[win_lo + r] = False
        picked = [win_lo + r]
    return t, m, picked


def _output_no_residual(model, X, O):
    return _orig_output(model, X, O) - X


def _commit_stale(model, seq, D):
    # appends the K/V of the block as it looked with every position masked
    X = _orig_embed(model, seq.tokens, np.ones(D, bool), seq.plant)
    _, K, V = R.project(model, X)
    H = R._block_forward(model, seq, np.arange(D), K, V, X, D)
    seq.cache_k = np.concatenate([seq.cache_k, K]); seq.cache_v = np.concatenate([seq.cache_v, V])
    seq.carry = H[D - 1]
    seq.history = list(seq.history) + [int(t) for t in seq.tokens]
    return H


def _dc_step_window_keeps_snapshot_kv(model, seq, s, S, tau, D):
    """DualCache step whose window rows attend with the snapshot's K/V
    instead of the K/V of their current tokens."""
    lo = s * S
    rows = np.arange(lo, lo + S)
    X = R.embed(model, seq.tokens[rows], seq.masked[rows], seq.plant[rows])
    _, Kw, Vw = R.project(model, X)
    H = R._block_forward(model, seq, rows, seq.snap_k, seq.snap_v, X, D)
    src = np.stack([H[j - 1 - lo] if j - 1 >= lo else seq.snap_h for j in range(lo, lo + S)])
    am, mx, lse, conf, picked = R._decide(model, seq, s, S, tau, src)
    return R.StepResult(H, rows, src, am, mx, lse, conf, picked, Kw, Vw)


def _embed_token_id_when_masked(model, tokens, masked, plant=None):
    X = model.E[np.asarray(tokens)].astype(np.float64)
    return X if plant is None else X + np.asarray(plant, dtype=np.float64)


MUTATIONS = {
    "dualcache_window_keeps_snapshot_kv": ("dc_step", _dc_step_window_keeps_snapshot_kv),
    "masked_rows_embed_their_token_id": ("embed", _embed_token_id_when_masked),
    "gqa_head_modulo": ("kv_head", lambda h, G: h % G),
    "mask_causal_inside_block": ("visible", lambda q, k, D: np.asarray(k)[None, :] <= np.asarray(q)[:, None]),
    "mask_everything_visible": ("visible", lambda q, k, D: np.ones((len(q), len(k)), bool)),
    "mask_strictly_earlier_blocks": ("visible", lambda q, k, D: (np.asarray(k)[None, :] // D) < (np.asarray(q)[:, None] // D) + (np.asarray(k)[None, :] == np.asarray(q)[:, None])),
    "no_token_shift": ("shift_row", lambda j: j),
    "shift_by_two": ("shift_row", lambda j: j - 2),
    "attention_without_scale": ("attention", _attention_no_scale),
    "attention_lse_off": ("attention", _attention_no_max_shift_wrong_lse),
    "confidence_inverted": ("confidence", _confidence_inverted),
    "argmax_highest_id_on_ties": ("confidence", _confidence_argmax_last),
    "threshold_ge": ("threshold_unmask", _threshold_ge),
    "no_fallback": ("threshold_unmask", _threshold_no_fallback),
    "fallback_highest_position": ("threshold_unmask", _threshold_fallback_highest_index),
    "no_residual": ("output", _output_no_residual),
    "commit_stale_kv": ("commit", _commit_stale),
}

PINS = [
    P.test_p3_attention_brute_force,
    P.test_p3_softmax_rows_sum_to_one,
    P.test_p3_two_key_closed_form,
    P.test_p4_one_block_no_prefix_is_bidirectional,
    P.test_p4_block_size_one_is_causal,
    P.test_p4_multi_block_mask_is_causal_to_block_end,
    P.test_p4_gqa_equals_mha_with_shared_heads_and_mha_case,
    P.test_p5_lm_head_statistics,
    P.test_p6_unmask_against_enumeration,
    P.test_p6_threshold_is_strict,
    P.test_p2_block_and_subblock_of_one_is_textbook_greedy,
    lambda: P.test_p2_threshold_one_unmasks_one_token_per_step("dual"),
    lambda: P.test_p1_block_cache_equals_full_recompute(P.TINY, "dual"),
    P.test_p7_prefill_then_commit_equals_multi_block_prefill,
    P.test_p4_dualcache_whole_block_window_equals_exact_step_on_any_state,
    P.test_p4_dualcache_window_rows_are_exact_in_one_layer,
    P.test_p10_masked_positions_take_the_mask_embedding,
]

# the pin written for each mistake must catch it by itself
TARGETED = {
    "dualcache_window_keeps_snapshot_kv": [P.test_p4_dualcache_whole_block_window_equals_exact_step_on_any_state,
                                           P.test_p4_dualcache_window_rows_are_exact_in_one_layer],
    "masked_rows_embed_their_token_id": [P.test_p10_masked_positions_take_the_mask_embedding],
}


def test_pins_pass_unmutated():
    for pin in PINS:
        pin()


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(R, attr, fn)
    caught = []
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            caught.append(getattr(pin, "__name__", "pin"))
    assert caught, f"mutation {name} slipped through every pin"


@pytest.mark.parametrize("name", sorted(TARGETED))
def test_targeted_pin_catches_its_mutation(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(R, attr, fn)
    for pin in TARGETED[name]:
        with pytest.raises(AssertionError):
            pin()
