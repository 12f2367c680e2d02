"""Per-sequence window progression (PerSequenceDecoder): every sequence opens
its next window as soon as it has decoded its own, so one batched step mixes
exact steps and DualCache steps.  Checked against the oracle's per-sequence
decode, teacher-forced (after every step the decoder takes the oracle's tokens
and mask bits): each sequence's LM-head statistics of its own window, its
unmask decisions, the committed cache and the carry; and the step count
against the most steps any one sequence takes."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import bd_inputs as bi
from gpu_util import DEV, TOL, down, lm_stats_close, rows_close, say, tdt, unmask_close, workload
from oracle import refine as R

pytestmark = pytest.mark.gpu

MID = replace(bi.C2, name="mid", B=4, V=20000, len_lo_blocks=4, len_hi_blocks=20, cap=1024)


def make_decoder(cfg, w, pre, st, plant):
    from block_diffusion_decoding_amd.decoder import Dims
    from block_diffusion_decoding_amd.persequence import PerSequenceDecoder
    dims = Dims(cfg.B, cfg.Hq, cfg.Hkv, cfg.d, cfg.hidden, cfg.V, cfg.D, cfg.cap)
    weights = {k: torch.from_numpy(getattr(w, k)) for k in ("E", "Wq", "Wk", "Wv", "Wo", "Wlm")}
    dec = PerSequenceDecoder(dims, weights, cfg.S, dtype=tdt(cfg.dtype), device=DEV)
    assert pre.kind != "prefill"
    dec.set_synthetic_prefix(pre.kv_len, pre.cache_k, pre.cache_v, pre.carry)
    dec.set_block(st.tokens, st.masked, plant)
    return dec


@pytest.mark.parametrize("graph", [False, True], ids=["eager", "graph"])
def test_per_sequence_progression_teacher_forced(graph):
    cfg = MID
    say(f"[per-sequence] {cfg.name} graph={graph}")
    # offsets planted so that every masked row passes the threshold, then kept
    # at a different rate per sequence: the sequences decode at different
    # speeds and their windows drift apart
    w, pre, st, plant, _ = workload(cfg, 0, all_masked=True, plant_rate=1.0)
    plant = np.array(plant, copy=True)
    keep = np.random.default_rng(3).random((cfg.B, cfg.D)) < np.array([0.9, 0.6, 0.3, 0.05])[:, None]
    plant[~keep] = 0.0
    dec = make_decoder(cfg, w, pre, st, plant)
    if graph:
        dec.capture_step(cfg.tau)
    m = R.Model.from_weights(w, cfg)
    seqs = R.seqs_from_inputs(m, cfg, pre, st, plant, None)
    D, S, tau, rtol = cfg.D, cfg.S, cfg.tau, TOL[cfg.dtype]
    dec.begin_block()
    n, mixed = 0, 0
    while dec.step(tau):
        kinds = dec.last_kinds
        mixed += len({k[1] for k in kinds if k is not None}) > 1
        got = np.stack([(dec.mask_bits_host()[b] >> np.arange(D, dtype=np.uint64)) & np.uint64(1)
                        for b in range(cfg.B)]).astype(bool)
        for b, q in enumerate(seqs):
            if kinds[b] is None:
                continue
            s_b, kind = kinds[b]
            before = q.masked.copy()
            res = (R.e_step if kind == "E" else R.dc_step)(m, q, s_b, S, tau, D)
            ref = R.lm_logits(m.Wlm, res.src)
            what = f"step {n} seq {b} window {s_b} {kind}"
            lm_stats_close(dec.argmax[b].cpu().numpy(), down(dec.conf[b]), down(dec.maxl[b]), down(dec.lse[b]),
                           ref, rtol, what)
            unmask_close(got[b:b + 1], q.masked[None], before[None], [res.conf], s_b * S, tau, rtol, what)
        dec.set_tokens(np.stack([q.tokens for q in seqs]), np.stack([q.masked for q in seqs]))
        n += 1
        assert n < 4 * D
    own = dec.own_steps.copy()
    for q in seqs:
        R.commit(m, q, D)
    dec.commit()
    for b, q in enumerate(seqs):
        L = q.L
        assert int(dec.kv_len[b]) == L
        rows_close(down(dec.cache_k)[b, :, L - D:L].transpose(1, 0, 2).reshape(D, -1),
                   q.cache_k[L - D:].reshape(D, -1), rtol, "appended k")
        rows_close(down(dec.H)[b, 0], q.carry, rtol, "carry after commit")
    say(f"    {n} batched steps, own steps per sequence {own.tolist()}, {mixed} mixed steps")
    assert n == own.max() and mixed > 0
