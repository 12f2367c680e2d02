"""GPU parity of whole refinement steps and block loops (decoder + all calls)
against the fp64 oracle on the same seeded inputs.

Multi-step comparisons use teacher forcing: after every step the GPU state is
set to the oracle's unmask decisions, so exempt ties cannot make the two
sides drift apart."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import bd_inputs as bi
from gpu_util import (TOL, down, gpu_decoder, lm_stats_close, oracle_seqs, rows_close, say, unmask_close,
                      workload)
from oracle import refine as R

pytestmark = pytest.mark.gpu


def compare_step(cfg, dec, m, seqs, results, kind, s, S, before_masked, what, seq_ids=None):
    """One step of the GPU decoder against the oracle's results for the
    sequences ``seq_ids`` (default: all).  With candidate compaction the LM
    head writes only the masked candidates' window slots, so the statistics
    are compared there; otherwise at every window slot."""
    rtol = TOL[cfg.dtype]
    D = cfg.D
    ids = list(range(cfg.B)) if seq_ids is None else list(seq_ids)
    w = dec.last
    # output rows of this step
    H = down(dec.H)
    for b, r in zip(ids, results):
        rows_close(H[b, 1 + r.rows], r.H, rtol, f"{what} H seq {b}")
    # LM-head statistics of the window rows
    sel = np.ones((len(ids), S), bool)
    if dec.uses_compaction(S):
        sel = before_masked[:, s * S:(s + 1) * S].copy()
    src = np.stack([r.src for r in results])[sel]
    ref_logits = R.lm_logits(m.Wlm, src)
    stat = lambda k: down(w[k])[ids][sel] if k != "argmax" else w[k].cpu().numpy()[ids][sel]
    lm_stats_close(stat("argmax"), stat("conf"), stat("maxl"), stat("lse"), ref_logits, rtol, f"{what} lm")
    # unmask decisions
    ref_masked = np.stack([q.masked for q in seqs])
    n_cmp, n_tie = unmask_close(dec.masked_host()[ids], ref_masked, before_masked, [r.conf for r in results], s * S,
                                cfg.tau, rtol, f"{what} unmask", got_conf_win=down(w["conf"])[ids])
    return [len(r.picked) for r in results]


def force(dec, seqs):
    dec.set_tokens(np.stack([q.tokens for q in seqs]), np.stack([q.masked for q in seqs]))


# blocks of 64 positions: the most a sequence's 64-bit mask word holds
TINY_D64 = replace(bi.C1, name="c1-D64", D=64, S=16)


@pytest.mark.parametrize("cfg", [bi.C1, bi.C1_96, TINY_D64], ids=["tiny-64", "tiny-96", "tiny-D64"])
def test_tiny_prefill_and_commit_equal_oracle_cache(cfg):
    say(f"[step] prefill+commit {cfg.name}")
    w, pre, st, _, _ = workload(cfg, 0, all_masked=True)
    dec = gpu_decoder(cfg, w, pre, st)
    m, seqs = oracle_seqs(cfg, w, pre, st)
    for b, q in enumerate(seqs):
        L = q.L
        assert int(dec.kv_len[b]) == L
        rows_close(down(dec.cache_k)[b, :, :L].transpose(1, 0, 2).reshape(L, -1), q.cache_k.reshape(L, -1),
                   TOL[cfg.dtype], "cache k")
        rows_close(down(dec.cache_v)[b, :, :L].transpose(1, 0, 2).reshape(L, -1), q.cache_v.reshape(L, -1),
                   TOL[cfg.dtype], "cache v")
        rows_close(down(dec.H)[b, 0], q.carry, TOL[cfg.dtype], "carry")


# bf16 at unit LM-head scale, as the bf16 workloads (c1's scale sharpens fp32 logits)
TINY_D64_BF16 = replace(TINY_D64, name="c1-D64-bf16", dtype="bf16", S=64, lm_scale=1.0)


@pytest.mark.parametrize("cfg", [bi.C1, bi.C1_96, replace(bi.C1, S=4), replace(bi.C1_96, S=16), TINY_D64,
                                 replace(TINY_D64, S=64), TINY_D64_BF16],
                         ids=["tiny-64", "tiny-96", "tiny-64-S4", "tiny-96-S16", "tiny-D64-S16", "tiny-D64-S64",
                              "tiny-D64-S64-bf16"])
@pytest.mark.parametrize("mode", ["exact", "dual"])
def test_tiny_block_decode_teacher_forced(cfg, mode):
    say(f"[step] tiny block loop {cfg.name} {mode}")
    w, pre, st, _, _ = workload(cfg, 0, all_masked=True)
    dec = gpu_decoder(cfg, w, pre, st)
    m, seqs = oracle_seqs(cfg, w, pre, st)
    D, S, tau = cfg.D, cfg.S, cfg.tau
    n_steps, passes = 0, []
    for s in range(D // S):
        first = True
        while any(q.masked[s * S:(s + 1) * S].any() for q in seqs):
            kind = "E" if (first or mode == "exact") else "DC"
            before = np.stack([q.masked for q in seqs])
            res = [(R.e_step if kind == "E" else R.dc_step)(m, q, s, S, tau, D) for q in seqs]
            (dec.e_step if kind == "E" else dec.dc_step)(s, S, tau)
            passes += compare_step(cfg, dec, m, seqs, res, kind, s, S, before, f"{mode} step {n_steps} {kind}")
            force(dec, seqs)
            first = False
            n_steps += 1
    for q in seqs:
        R.commit(m, q, D)
    dec.commit()
    for b, q in enumerate(seqs):
        L = q.L
        assert int(dec.kv_len[b]) == L
        rows_close(down(dec.cache_k)[b, :, L - D:L].transpose(1, 0, 2).reshape(D, -1),
                   q.cache_k[L - D:].reshape(D, -1), TOL[cfg.dtype], "appended k")
        rows_close(down(dec.cache_v)[b, :, L - D:L].transpose(1, 0, 2).reshape(D, -1),
                   q.cache_v[L - D:].reshape(D, -1), TOL[cfg.dtype], "appended v")
        rows_close(down(dec.H)[b, 0], q.carry, TOL[cfg.dtype], "carry after commit")
    say(f"    {n_steps} steps, tokens per step {passes}")
    assert n_steps >= D // S and sum(passes) == cfg.B * D


@pytest.mark.parametrize("cfg,rate,compact", [(bi.C2, None, None), (bi.C3, 0.5, None), (bi.C3, 1.0, None),
                                              (bi.C3, 0.5, True)],
                         ids=["1.5B", "7B-r0.5", "7B-r1", "7B-r0.5-candidates"])
def test_refresh_then_dualcache_steps(cfg, rate, compact):
    """Window 1: exact refresh step, then two DualCache steps (the second after
    the first one's unmasking), against the oracle; with ``compact`` the LM
    head runs on the masked candidates only."""
    say(f"[step] {cfg.name} rate={rate} compact={compact}")
    w, pre, st, plant, carry_plant = workload(cfg, 0, window=1, plant_rate=rate)
    dec = gpu_decoder(cfg, w, pre, st, plant, carry_plant, compact=compact)
    assert dec.uses_compaction(cfg.S) == bool(compact)
    m, seqs = oracle_seqs(cfg, w, pre, st, plant, carry_plant)
    S, D, tau, s = cfg.S, cfg.D, cfg.tau, 1
    tokens_per_step = []
    n_cand0 = int(sum(q.masked[s * S:(s + 1) * S].sum() for q in seqs))
    for k, kind in enumerate(["E", "DC", "DC"]):
        if not any(q.masked[s * S:(s + 1) * S].any() for q in seqs):
            break
        before = np.stack([q.masked for q in seqs])
        res = [(R.e_step if kind == "E" else R.dc_step)(m, q, s, S, tau, D) for q in seqs]
        (dec.e_step if kind == "E" else dec.dc_step)(s, S, tau)
        tokens_per_step.append(sum(compare_step(cfg, dec, m, seqs, res, kind, s, S, before, f"{cfg.name} {kind}{k}")))
        force(dec, seqs)
    say(f"    tokens unmasked per step {tokens_per_step}")
    if rate == 1.0:                 # every candidate planted: all pass in the first step
        assert tokens_per_step[0] == n_cand0


def test_fixed_schedule_block_matches_oracle_loop():
    """Fixed 8 steps per window (1 exact + 7 DualCache, no host sync) on a
    fresh block gives the oracle's loop result: every step unmasks at least
    one token, so 8 steps finish a window of 8."""
    cfg = bi.C1
    say("[step] fixed schedule")
    w, pre, st, _, _ = workload(cfg, 1, all_masked=True)
    dec = gpu_decoder(cfg, w, pre, st)
    m, seqs = oracle_seqs(cfg, w, pre, st)
    R.decode_block(m, seqs, cfg.D, cfg.S, 1.0, mode="dual")
    dec.decode_block(cfg.S, 1.0, mode="dual", steps_per_window=cfg.S)
    torch.cuda.synchronize()
    got = dec.tokens.cpu().numpy()
    ref = np.stack([q.tokens for q in seqs])
    assert np.array_equal(got, ref)
    assert int(dec.mask_bits[0]) == 0 and int(dec.kv_len[0]) == seqs[0].L
