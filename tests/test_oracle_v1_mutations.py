"""Plant plausible mistakes in the v1-style oracle (on the CPU) and check
that the pins in test_oracle_v1_pins.py catch each one."""
import numpy as np
import pytest

import test_oracle_v1_pins as P
from oracle import refine as R
from oracle import v1 as V1

_exact, _dual, _full = V1.exact_step, V1.dual_step, V1.full_forward


def _exact_prefix_only(model, seq, k, D, tau, refresh=True):
    res = _exact(model, seq, k, D, tau, refresh)
    lo = seq.P + k * D
    seq.cache_k, seq.cache_v = seq.cache_k[:lo], seq.cache_v[:lo]       # suffix dropped
    return res


def _exact_carry_off_by_one(model, seq, k, D, tau, refresh=True):
    res = _exact(model, seq, k, D, tau, refresh)
    H = _full(model, seq.tokens, seq.masked, seq.plant)[0]
    seq.carry = H[seq.P + k * D]
    return res


def _full_block_causal(model, tokens, masked, plant=None):
    X = R.embed(model, np.asarray(tokens), np.asarray(masked, dtype=bool))
    Q, K, V = R.project(model, X)
    pos = np.arange(X.shape[0])
    O, _ = R.attention(Q, K, V, R.visible(pos, pos, 32), model.G)
    return R.output(model, X, O), K, V


def _exact_cache_with_block(model, seq, k, D, tau, refresh=True):
    res = _exact(model, seq, k, D, tau, refresh)
    H, K, V = _full(model, seq.tokens, seq.masked, seq.plant)
    seq.cache_k, seq.cache_v = K, V                                      # block rows cached too
    return res


MUTANTS = [
    ("exact_step", _exact_prefix_only, P.test_dual_step_after_refresh_equals_the_exact_step, (1,)),
    ("exact_step", _exact_carry_off_by_one, P.test_dual_step_after_refresh_equals_the_exact_step, (0,)),
    ("exact_step", _exact_cache_with_block, P.test_dual_step_after_refresh_equals_the_exact_step, (1,)),
    ("full_forward", _full_block_causal, P.test_full_forward_matches_torch_sdpa, ()),
    ("full_forward", _full_block_causal, P.test_prompt_rows_see_the_generation_region, ()),
]


@pytest.mark.parametrize("name,fn,pin,args", MUTANTS, ids=[f"{n}:{f.__name__}" for n, f, _, _ in MUTANTS])
def test_pin_catches_planted_mistake(monkeypatch, name, fn, pin, args):
    monkeypatch.setattr(V1, name, fn)
    with pytest.raises(AssertionError):
        pin(*args)
