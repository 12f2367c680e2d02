"""Pins of the v1-style full-attention oracle (oracle/v1.py): the full
forward against torch's scaled-dot-product attention, the DualCache step
right after a refresh against the exact step (the cached prefix and suffix
plus the fresh block are the whole sequence), the full-attention property
that the prompt's rows see the generation region, and tau = 1 giving one
token per step."""
import copy

import numpy as np
import pytest
import torch

import bd_inputs as bi
from oracle import refine as R
from oracle import v1 as V1


def _model(seed=0, scale=1.0):
    cfg = bi.C1
    m = R.Model.from_weights(bi.make_weights(cfg, seed), cfg)
    m.Wlm = m.Wlm * scale
    return m, cfg


def _seq(rng, cfg, P=32, gen=96):
    return V1.new_sequence(rng.integers(0, cfg.V, P), gen)


def test_full_forward_matches_torch_sdpa():
    model, cfg = _model(1)
    rng = np.random.default_rng(2)
    seq = _seq(rng, cfg)
    seq.masked[40:50] = False
    seq.tokens[40:50] = rng.integers(0, cfg.V, 10)
    H, K, V = V1.full_forward(model, seq.tokens, seq.masked)
    X = R.embed(model, seq.tokens, seq.masked)
    T = X.shape[0]
    q = torch.from_numpy(X @ model.Wq.T).view(T, model.Hq, model.d).transpose(0, 1)
    k = torch.from_numpy(K).transpose(0, 1).repeat_interleave(model.G, dim=0)
    v = torch.from_numpy(V).transpose(0, 1).repeat_interleave(model.G, dim=0)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v).transpose(0, 1).reshape(T, -1).numpy()
    np.testing.assert_allclose(H, X + o @ model.Wo.T, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("k", [0, 1])
def test_dual_step_after_refresh_equals_the_exact_step(k):
    model, cfg = _model(3, scale=100.0)
    rng = np.random.default_rng(4)
    D = 32
    seq = _seq(rng, cfg)
    if k == 1:            # block 0 already decoded
        seq.tokens[32:64] = rng.integers(0, cfg.V, 32)
        seq.masked[32:64] = False
    seq.masked[32 + k * D + 5] = False
    before = (seq.tokens.copy(), seq.masked.copy())
    res_e = V1.exact_step(model, seq, k, D, 0.9)
    seq.tokens, seq.masked = before[0].copy(), before[1].copy()
    res_d = V1.dual_step(model, seq, k, D, 0.9)
    np.testing.assert_allclose(res_d.src, res_e.src, rtol=1e-12, atol=1e-12)
    assert res_d.picked == res_e.picked


def test_prompt_rows_see_the_generation_region():
    model, cfg = _model(5)
    rng = np.random.default_rng(6)
    seq = _seq(rng, cfg)
    H0 = V1.full_forward(model, seq.tokens, seq.masked)[0]
    seq.masked[80] = False
    seq.tokens[80] = 7
    H1 = V1.full_forward(model, seq.tokens, seq.masked)[0]
    assert np.abs(H1[:32] - H0[:32]).max() > 1e-9      # full attention: the prompt sees position 80


@pytest.mark.parametrize("mode", ["dual", "exact"])
def test_threshold_one_decodes_one_token_per_step(mode):
    model, cfg = _model(7)
    rng = np.random.default_rng(8)
    seq = _seq(rng, cfg, P=32, gen=64)
    counts = []
    steps = V1.decode(model, seq, 32, 1.0, mode, on_step=lambda k, kind, r: counts.append(len(r.picked)))
    assert steps == 64 and set(counts) == {1} and not seq.masked.any()
