"""Plant plausible mistakes in the training-form oracle (on the CPU) and
check that the pins in test_oracle_train_pins.py catch each one.  Nothing
here touches the HIP path."""
import numpy as np
import pytest

import test_oracle_train_pins as P
from oracle import train as TR

_mask, _src, _sup, _nll, _fwd = TR.mask_2L, TR.source_row, TR.supervised, TR.token_nll, TR.forward_2L


def _mask_noisy_sees_own_clean_block(L, D):
    A = _mask(L, D)
    for p in range(L):
        b = p // D
        A[p, L + b * D:L + (b + 1) * D] = True
    return A


def _mask_clean_sees_noisy_block(L, D):
    A = _mask(L, D)
    for p in range(L, 2 * L):
        b = (p - L) // D
        A[p, b * D:(b + 1) * D] = True
    return A


def _mask_noisy_causal_in_block(L, D):
    A = _mask(L, D)
    for p in range(L):
        A[p, p + 1:(p // D + 1) * D] = False
    return A


def _src_always_noisy(i, L, D):
    return i - 1


def _src_no_shift(i, L, D):
    return i if i % D != 0 else L + i


def _supervised_unmasked(m):
    m = np.asarray(m, dtype=bool)
    idx = np.flatnonzero(~m)
    return idx[idx >= 1]


def _nll_wrong_sign(logits, target):
    return -_nll(logits, target)


def _nll_no_normaliser(logits, target):
    logits = np.atleast_2d(np.asarray(logits, dtype=np.float64))
    return -logits[np.arange(logits.shape[0]), np.asarray(target)]


def _forward_clean_half_noisy(model, x0, m, D, plant=None):
    """The clean half built from the noisy tokens."""
    from oracle import refine as R
    x0 = np.asarray(x0, dtype=np.int64)
    L = len(x0)
    X = np.concatenate([R.embed(model, x0, m), R.embed(model, x0, m)], axis=0)
    Q, K, V = R.project(model, X)
    O, _ = R.attention(Q, K, V, TR.mask_2L(L, D), model.G)
    return R.output(model, X, O), Q, K, V, O


ND = (96, 32)   # arguments of the parametrised pins
MUTANTS = [
    ("mask_2L", _mask_noisy_sees_own_clean_block, P.test_noisy_block_is_an_exact_step_over_the_clean_prefix, ND),
    ("mask_2L", _mask_noisy_sees_own_clean_block, P.test_mask_matches_the_hand_worked_example, ()),
    ("mask_2L", _mask_clean_sees_noisy_block, P.test_clean_half_is_the_block_causal_prefill, ND),
    ("mask_2L", _mask_noisy_causal_in_block, P.test_noisy_block_is_an_exact_step_over_the_clean_prefix, ND),
    ("source_row", _src_always_noisy, P.test_token_shift_rows_are_the_steps_source_rows, ND),
    ("source_row", _src_no_shift, P.test_token_shift_rows_are_the_steps_source_rows, ND),
    ("supervised", _supervised_unmasked, P.test_a_single_masked_position_is_the_only_supervised_one, ()),
    ("token_nll", _nll_wrong_sign, P.test_token_nll_matches_library_log_softmax, ()),
    ("token_nll", _nll_no_normaliser, P.test_zero_head_gives_log_vocab_per_token, ()),
    ("forward_2L", _forward_clean_half_noisy, P.test_clean_half_is_the_block_causal_prefill, ND),
]


@pytest.mark.parametrize("name,fn,pin,args", MUTANTS, ids=[f"{n}:{f.__name__}" for n, f, _, _ in MUTANTS])
def test_pin_catches_planted_mistake(monkeypatch, name, fn, pin, args):
    monkeypatch.setattr(TR, name, fn)
    with pytest.raises(AssertionError):
        pin(*args)
