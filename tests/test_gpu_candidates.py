"""Candidate-row compaction: the LM head over only the masked positions of
the window (bd_candidate_rows + bd_lmhead_confidence_rows) against the LM
head over every window row, and whole decoders with and without it."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import bd_inputs as bi
from gpu_util import DEV, gpu_decoder, say, up, workload

pytestmark = pytest.mark.gpu


def ops():
    from block_diffusion_decoding_amd import ops as o
    return o


def ref_candidates(bits, win_lo, win_len, rows_per_seq):
    rows, pos = [], []
    for b, x in enumerate(bits):
        for r in range(win_len):
            if (int(x) >> (win_lo + r)) & 1:
                rows.append(b * rows_per_seq + win_lo + r)
                pos.append(b * win_len + r)
    return np.array(rows, np.int32), np.array(pos, np.int32)


@pytest.mark.parametrize("B,win_lo,win_len,density", [(37, 8, 8, 0.5), (100, 24, 8, 0.3), (3, 0, 32, 1.0),
                                                      (8, 16, 8, 0.0), (512, 0, 8, 0.7)])
def test_candidate_rows(B, win_lo, win_len, density):
    say(f"[candidates] B={B} window {win_lo}+{win_len} density {density}")
    rng = np.random.default_rng(B)
    masked = rng.random((B, 64)) < density
    bits = np.zeros(B, np.uint64)
    for j in range(64):
        bits |= masked[:, j].astype(np.uint64) << np.uint64(j)
    rps = win_lo + win_len + 1
    n = B * win_len
    row_idx = torch.full((n,), 7, dtype=torch.int32, device=DEV)
    out_pos = torch.full((n,), 7, dtype=torch.int32, device=DEV)
    count = torch.full((1,), -5, dtype=torch.int32, device=DEV)
    ops().bd_candidate_rows(up(bits.view(np.int64)), row_idx, out_pos, count, win_lo=win_lo, win_len=win_len,
                            rows_per_seq=rps)
    rr, rp = ref_candidates(bits, win_lo, win_len, rps)
    c = int(count.item())
    assert c == len(rr)
    got_r, got_p = row_idx.cpu().numpy(), out_pos.cpu().numpy()
    assert np.array_equal(got_r[:c], rr) and np.array_equal(got_p[:c], rp)
    assert (got_r[c:] == -1).all() and (got_p[c:] == -1).all()


@pytest.mark.parametrize("B,S,hidden,V", [(32, 8, 512, 5000), (8, 8, 512, 5000), (40, 8, 256, 3000)])
def test_lmhead_rows_match_full_rows(B, S, hidden, V):
    """Rows listed by bd_candidate_rows give, at their window slots, exactly
    the statistics of the full LM head (same kernels, same per-row order);
    the other slots are left alone."""
    say(f"[lmhead rows] B={B} S={S} hidden={hidden} V={V}")
    D, s = 32, 1
    rng = np.random.default_rng(B + V)
    w = bi.normal(5, "Wlm", (V, hidden), 0.02, "bf16")
    H = bi.normal(5, "h", (B * (1 + D), hidden), 0.6, "bf16")
    masked = rng.random((B, D)) < 0.55
    bits = np.zeros(B, np.uint64)
    for j in range(D):
        bits |= masked[:, j].astype(np.uint64) << np.uint64(j)
    T = torch.bfloat16
    Hd, Wd = up(H, T), up(w, T)
    idx = np.array([b * (1 + D) + s * S + r for b in range(B) for r in range(S)], np.int32)
    full = [torch.zeros(B * S, dtype=torch.int32, device=DEV)] + [torch.zeros(B * S, device=DEV) for _ in range(3)]
    ops().bd_lmhead_confidence(Hd, up(idx), Wd, full[0], full[1], max_logit=full[2], lse=full[3])
    rows = torch.zeros(B * S, dtype=torch.int32, device=DEV)
    pos = torch.zeros(B * S, dtype=torch.int32, device=DEV)
    cnt = torch.zeros(1, dtype=torch.int32, device=DEV)
    ops().bd_candidate_rows(up(bits.view(np.int64)), rows, pos, cnt, win_lo=s * S, win_len=S, rows_per_seq=1 + D)
    comp = [torch.full((B * S,), -7, dtype=torch.int32, device=DEV)] + \
           [torch.full((B * S,), -7.0, device=DEV) for _ in range(3)]
    ops().bd_lmhead_confidence_rows(Hd, rows, pos, cnt, Wd, comp[0], comp[1], max_logit=comp[2], lse=comp[3])
    torch.cuda.synchronize()
    cand = masked[:, s * S:(s + 1) * S].reshape(-1)
    assert int(cnt.item()) == int(cand.sum())
    for f, c in zip(full, comp):
        f, c = f.cpu().numpy(), c.cpu().numpy()
        assert np.array_equal(f[cand], c[cand])          # bit-identical at candidate slots
        assert (c[~cand] == -7).all()                      # other slots untouched
    # an empty list writes nothing
    cnt.zero_()
    ops().bd_lmhead_confidence_rows(Hd, rows, pos, cnt, Wd, comp[0], comp[1])
    torch.cuda.synchronize()
    assert (comp[0].cpu().numpy()[~cand] == -7).all()


def test_compacted_decoder_matches_full_decoder():
    """Two decoders on the same inputs, one computing the LM head on every
    window row and one on the masked candidates only: identical tokens, mask
    bits, hidden rows, in-block K/V and caches after every step and commit,
    and identical statistics at every candidate slot."""
    cfg = replace(bi.C2, name="mid16", B=16, V=20000, len_lo_blocks=4, len_hi_blocks=20, cap=1024)
    say("[candidates] decoders, 16 sequences x 8-row windows")
    w, pre, st, _, _ = workload(cfg, 0, all_masked=True, plant_rate=None)
    full = gpu_decoder(cfg, w, pre, st, compact=False)
    comp = gpu_decoder(cfg, w, pre, st, compact=True)
    S, tau = cfg.S, 0.3
    assert comp.uses_compaction(S) and not full.uses_compaction(S)
    rng = np.random.default_rng(1)
    plant = bi.normal(7, "plant", (cfg.B, cfg.D, cfg.hidden), 0.5, "bf16")
    plant[rng.random((cfg.B, cfg.D)) < 0.5] = 0.0
    for d in (full, comp):
        d.set_block(np.zeros((cfg.B, cfg.D), np.int32), np.ones((cfg.B, cfg.D), bool), plant)
    for s in range(cfg.D // S):
        for k in range(3):
            before = full.masked_host()[:, s * S:(s + 1) * S].reshape(-1)
            for d in (full, comp):
                (d.e_step if k == 0 else d.dc_step)(s, S, tau)
            torch.cuda.synchronize()
            for a, b in ((full.tokens, comp.tokens), (full.mask_bits, comp.mask_bits), (full.H, comp.H),
                         (full.blk_k, comp.blk_k), (full.blk_v, comp.blk_v)):
                assert torch.equal(a, b), f"window {s} step {k}"
            for key in ("argmax", "conf", "maxl", "lse"):
                fa, ca = full.last[key].cpu().numpy().reshape(-1), comp.last[key].cpu().numpy().reshape(-1)
                assert np.array_equal(fa[before], ca[before]), f"{key} window {s} step {k}"
    for d in (full, comp):
        d.set_tokens(d.tokens.cpu().numpy(), np.zeros((cfg.B, cfg.D), bool))
        d.commit()
    torch.cuda.synchronize()
    assert torch.equal(full.cache_k, comp.cache_k) and torch.equal(full.kv_len, comp.kv_len)
