"""Oracle parity of refinement steps whose windows hold more than 64 rows.

When B * S > 64 the decoder lists the window's masked candidates
(bd_candidate_rows), runs the LM head on that list only
(bd_lmhead_confidence_rows: 256-row tiles above 64 listed rows) and applies
the threshold rule (bd_threshold_unmask).  Only masked positions are
predicted ("Fast-dLLM v2" notes, Key design 3: the masked tokens are refined,
those above the threshold unmasked), so statistics exist at the candidate
slots alone and are compared there.  Every case here runs against the fp64
oracle:

* a whole block, teacher forced, of 32 sequences x 8-row windows at a
  mid-size vocabulary (exact refresh + DualCache steps, planted passes in
  two windows, the fallback rule in the others);
* the 7B workload's exact variant (S = D = 32, 256 rows);
* the long-context workload (32 sequences x 16384 committed rows, 7B head):
  an exact step and a DualCache step, the oracle run on sampled sequences.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

import bd_inputs as bi
from gpu_util import TOL, gpu_decoder, oracle_seqs, say, workload
from oracle import refine as R
from test_gpu_step import compare_step

pytestmark = pytest.mark.gpu

# 32 sequences, 1.5B attention shape, vocabulary 20000, prefixes of 128-640
# rows; lm_scale 100 spreads the candidates' confidences (about 0.005-0.007,
# so the fallback picks differ by far more than the 2% tie band)
MID32 = replace(bi.C2, name="mid32", B=32, V=20000, len_lo_blocks=4, len_hi_blocks=20, cap=1024, lm_scale=100.0)


def _window_plants(cfg, w, windows, rate, seed=0):
    """Planted peaked logits for rate of the positions of each listed window
    (every position of a fresh block is masked)."""
    plant = np.zeros((cfg.B, cfg.D, cfg.hidden), np.float32)
    carry = np.zeros((cfg.B, cfg.hidden), np.float32)
    for s in windows:
        st = bi.BlockState(np.zeros((cfg.B, cfg.D), np.int32), np.ones((cfg.B, cfg.D), bool), s, cfg.S)
        p, c, _ = bi.make_plants(cfg, seed + 100 * s, w, st, rate)
        plant += p
        carry += c
    return plant, carry


def test_candidate_block_loop_matches_oracle():
    """A fresh block decoded window by window (exact refresh, then DualCache
    steps until the window is done), teacher forced, 256-row windows."""
    cfg = MID32
    say("[compaction] block loop, 32 sequences x 8-row windows, vocabulary 20000")
    w, pre, st, _, _ = workload(cfg, 0, all_masked=True)
    plant, carry = _window_plants(cfg, w, (1, 3), 0.5)
    dec = gpu_decoder(cfg, w, pre, st, plant, carry)
    assert dec.uses_compaction(cfg.S)
    m, seqs = oracle_seqs(cfg, w, pre, st, plant, carry)
    D, S, tau = cfg.D, cfg.S, cfg.tau
    n_steps, per_window = 0, []
    for s in range(D // S):
        first, toks = True, 0
        while any(q.masked[s * S:(s + 1) * S].any() for q in seqs):
            kind = "E" if first else "DC"
            before = np.stack([q.masked for q in seqs])
            res = [(R.e_step if first else R.dc_step)(m, q, s, S, tau, D) for q in seqs]
            (dec.e_step if first else dec.dc_step)(s, S, tau)
            toks += sum(compare_step(cfg, dec, m, seqs, res, kind, s, S, before, f"window {s} step {n_steps} {kind}"))
            dec.set_tokens(np.stack([q.tokens for q in seqs]), np.stack([q.masked for q in seqs]))
            first = False
            n_steps += 1
        per_window.append(toks)
    say(f"    {n_steps} steps, tokens per window {per_window}")
    # planted windows pass several tokens per step, the others decode one per step
    assert n_steps < 4 * S and sum(per_window) == cfg.B * D


def test_candidate_exact_window_7B():
    """The 7B workload's exact variant: one window of the whole block
    (S = D = 32), 8 sequences, so 256 rows and the 256-row LM-head tiles."""
    cfg = replace(bi.C3, S=32)
    say("[compaction] 7B exact window S=D=32")
    w, pre, st, plant, carry = workload(cfg, 0, window=0, S=32, plant_rate=0.5)
    dec = gpu_decoder(cfg, w, pre, st, plant, carry)
    assert dec.uses_compaction(cfg.S)
    m, seqs = oracle_seqs(cfg, w, pre, st, plant, carry)
    before = np.stack([q.masked for q in seqs])
    res = [R.e_step(m, q, 0, cfg.S, cfg.tau, cfg.D) for q in seqs]
    dec.e_step(0, cfg.S, cfg.tau)
    toks = compare_step(cfg, dec, m, seqs, res, "E", 0, cfg.S, before, "7B exact S=32")
    say(f"    tokens unmasked {toks}")


def test_candidate_steps_long_context_sampled():
    """The long-context workload (32 sequences x 16384 committed rows, 7B
    attention and head): exact refresh step and one DualCache step of window
    0 with half the candidates planted; the GPU runs the whole batch, the
    oracle the sampled sequences."""
    cfg = bi.C4
    sample = [0, 17, 31]
    say("[compaction] long context B=32 L=16384, sampled sequences " + str(sample))
    w, pre, st, plant, carry = workload(cfg, 0, window=0, all_masked=True, plant_rate=0.5)
    dec = gpu_decoder(cfg, w, pre, st, plant, carry)
    assert dec.uses_compaction(cfg.S)
    sub = replace(cfg, B=len(sample))
    pre_s = bi.Prefix("synthetic", kv_len=pre.kv_len[sample], cache_k=pre.cache_k[sample],
                      cache_v=pre.cache_v[sample], carry=pre.carry[sample])
    st_s = bi.BlockState(st.tokens[sample], st.masked[sample], st.window, st.S)
    del pre
    m, seqs = oracle_seqs(sub, w, pre_s, st_s, plant[sample], carry[sample])
    S, D, tau = cfg.S, cfg.D, cfg.tau
    for k, kind in enumerate(("E", "DC")):
        before = np.stack([q.masked for q in seqs])
        res = [(R.e_step if kind == "E" else R.dc_step)(m, q, 0, S, tau, D) for q in seqs]
        (dec.e_step if kind == "E" else dec.dc_step)(0, S, tau)
        toks = compare_step(sub, dec, m, seqs, res, kind, 0, S, before, f"long {kind}", seq_ids=sample)
        say(f"    {kind}: tokens unmasked on the sampled sequences {toks}")
        # teacher forcing on the sampled sequences; the others keep the GPU's decisions
        tokens = dec.tokens.cpu().numpy()
        masked = dec.masked_host()
        for i, b in enumerate(sample):
            tokens[b], masked[b] = seqs[i].tokens, seqs[i].masked
        dec.set_tokens(tokens, masked)
    torch.cuda.synchronize()
