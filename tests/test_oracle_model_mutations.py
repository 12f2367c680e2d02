"""Plant plausible mistakes in the multi-layer oracle (on the CPU) and check
that the pins in test_oracle_model_pins.py catch each one.  Nothing here
touches the HIP path."""
import numpy as np
import pytest

import test_oracle_model_pins as P
from oracle import model as OM

_rope, _rmsnorm, _silu, _layer_rest, _forward_rows = OM.rope, OM.rmsnorm, OM.silu, OM.layer_rest, OM.forward_rows


def _rope_interleaved(x, pos, theta):
    """Pairs (x0, x1), (x2, x3), ... instead of (x_i, x_{i+d/2})."""
    x = np.asarray(x, dtype=np.float64)
    n, H, d = x.shape
    perm = np.concatenate([np.arange(0, d, 2), np.arange(1, d, 2)])
    y = _rope(x[..., perm], pos, theta)
    out = np.empty_like(y)
    out[..., perm] = y
    return out


def _rope_negative(x, pos, theta):
    return _rope(x, -np.asarray(pos, dtype=np.float64), theta)


def _rope_freq_d2(x, pos, theta):
    """Frequencies theta^(-i/d) instead of theta^(-2i/d)."""
    return _rope(x, pos, theta ** 0.5)


def _rmsnorm_sum(x, eps):
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def _rmsnorm_no_eps(x, eps):
    return _rmsnorm(x, 0.0)


def _silu_sigmoid(z):
    return 1.0 / (1.0 + np.exp(-np.asarray(z, dtype=np.float64)))


def _layer_rest_no_residual(model, layer, X, O):
    """Attention output replaces the residual stream instead of adding to it."""
    return _layer_rest(model, layer, np.zeros_like(X), O)


def _forward_rows_ignores_snapshot(model, seq, X, rows, D, snap_k=None, snap_v=None):
    """DualCache pass that attends only to the fresh window rows plus zeros."""
    if snap_k is not None:
        snap_k = [np.zeros_like(k) for k in snap_k]
        snap_v = [np.zeros_like(v) for v in snap_v]
    return _forward_rows(model, seq, X, rows, D, snap_k, snap_v)


def _forward_rows_window_keeps_snapshot(model, seq, X, rows, D, snap_k=None, snap_v=None):
    """DualCache pass whose window rows attend with the snapshot's K/V
    instead of their fresh ones."""
    if snap_k is None:
        return _forward_rows(model, seq, X, rows, D)
    rows = np.asarray(rows)
    pos = seq.L + rows
    Ks, Vs = [], []
    for li, layer in enumerate(model.layers):
        Q, K, V = OM.layer_qkv(model, layer, X, pos)
        Kc = np.concatenate([seq.cache_k[li], snap_k[li]], axis=0)
        Vc = np.concatenate([seq.cache_v[li], snap_v[li]], axis=0)
        O, _ = OM.attention(Q, Kc, Vc, OM.visible(pos, np.arange(seq.L + D), D), model.G)
        X = OM.layer_rest(model, layer, X, O)
        Ks.append(K)
        Vs.append(V)
    return OM._norm(model, X), Ks, Vs


def _embed_token_id_when_masked(model, tokens, masked):
    return model.E[np.asarray(tokens)].astype(np.float64)


MUTANTS = [
    ("forward_rows", _forward_rows_window_keeps_snapshot, P.test_dualcache_whole_block_window_equals_exact_step_on_any_state),
    ("embed", _embed_token_id_when_masked, P.test_masked_positions_take_the_mask_embedding),
    ("rope", _rope_interleaved, P.test_rope_hand_example_fixes_pairing_and_sign),
    ("rope", _rope_negative, P.test_rope_hand_example_fixes_pairing_and_sign),
    ("rope", _rope_freq_d2, P.test_rope_hand_example_fixes_pairing_and_sign),
    ("rmsnorm", _rmsnorm_sum, P.test_rmsnorm_closed_form_and_scale_invariance),
    ("rmsnorm", _rmsnorm_no_eps, P.test_rmsnorm_closed_form_and_scale_invariance),
    ("silu", _silu_sigmoid, P.test_silu_matches_logistic),
    ("layer_rest", _layer_rest_no_residual, P.test_reduces_to_one_layer_oracle),
    ("forward_rows", _forward_rows_ignores_snapshot, P.test_dualcache_pass_with_current_snapshot_equals_exact_pass),
]


@pytest.mark.parametrize("name,fn,pin", MUTANTS, ids=[f"{n}:{f.__name__}" for n, f, _ in MUTANTS])
def test_pin_catches_planted_mistake(monkeypatch, name, fn, pin):
    monkeypatch.setattr(OM, name, fn)
    with pytest.raises(AssertionError):
        pin()
