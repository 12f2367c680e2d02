"""Helpers of the GPU parity tests: upload seeded inputs, build the decoder
and the oracle from the same draws, and the tolerance rules.

Tolerances (per element type): 1e-3 relative for fp32, 2e-2 for bf16.
* rows (attention outputs, hidden rows, logits): per row
  |d|_2 / |ref|_2 <= rtol and every element |d| <= rtol * (|ref| + RMS(row));
* max / lse: |d| <= rtol * max(1, RMS(logits row)); conf: |d| / conf <= rtol;
* argmax: exact unless the oracle's top-2 gap is within the row's tie band:
  rtol * max(|l1|, RMS(row)) at most, and, where the GPU's max logit is
  given, only max(4 |max logit error|, 2e-3 max(|l1|, RMS)): a swap needs the
  two logits' errors to add up to the gap, and the max logit's error measures
  them;
* unmask sets: exact except positions whose oracle confidence is within 1e-3
  of the threshold; a fallback pick is compared only when the best two
  candidate confidences differ by more than the tie band (rtol * conf at
  most; max(4 x the largest relative confidence error, 2e-3) of conf where
  the GPU's confidences are given), and a tied pick must still be a single
  candidate within the band.
"""
import sys

import numpy as np
import torch

import bd_inputs as bi
from oracle import refine as R

DEV = "cuda"
TOL = {"f32": 1e-3, "bf16": 2e-2}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def tdt(dtype: str):
    return torch.float32 if dtype == "f32" else torch.bfloat16


def up(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(DEV) if dtype is None else t.to(DEV, dtype)


def down(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def rows_close(got, ref, rtol, what=""):
    ref = np.asarray(ref, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64).reshape(ref.shape)
    g2 = got.reshape(-1, ref.shape[-1])
    r2 = ref.reshape(-1, ref.shape[-1])
    d = g2 - r2
    rn = np.linalg.norm(d, axis=1) / np.maximum(np.linalg.norm(r2, axis=1), 1e-30)
    rms = np.sqrt((r2 ** 2).mean(axis=1, keepdims=True))
    bad = np.abs(d) > rtol * (np.abs(r2) + rms)
    assert np.isfinite(g2).all(), f"{what}: non-finite output"
    assert rn.max() <= rtol and not bad.any(), \
        f"{what}: max row rel err {rn.max():.3g} (rtol {rtol}), {bad.sum()} elements out of tolerance"
    return float(rn.max())


def lm_stats_close(argmax, conf, mx, lse, ref_logits, rtol, what=""):
    """GPU (argmax, conf, max, lse) of each row against fp64 logits."""
    ref_logits = np.atleast_2d(ref_logits)
    am, rmx, rlse, rconf = R.confidence(ref_logits)
    rms = np.sqrt((ref_logits ** 2).mean(axis=1))
    tol = rtol * np.maximum(1.0, rms)
    if mx is not None:
        assert np.all(np.abs(mx - rmx) <= tol), f"{what}: max logit"
    if lse is not None:
        assert np.all(np.abs(lse - rlse) <= tol), f"{what}: lse"
    assert np.all(np.abs(conf - rconf) <= rtol * rconf), \
        f"{what}: conf max rel err {np.max(np.abs(conf - rconf) / rconf):.3g}"
    top2 = np.sort(ref_logits, axis=1)[:, -2:]
    gap = top2[:, 1] - top2[:, 0]
    scale = np.maximum(np.abs(top2[:, 1]), rms)
    band = rtol * scale
    if mx is not None:
        band = np.minimum(band, np.maximum(4.0 * np.abs(np.asarray(mx) - rmx), 2e-3 * scale))
    exempt = gap <= band
    ok = (argmax == am) | exempt
    assert ok.all(), f"{what}: argmax differs on rows {np.nonzero(~ok)[0][:10]}"
    # an exempt row must still pick a token whose logit ties the maximum within tolerance
    for m in np.nonzero(exempt & (argmax != am))[0]:
        assert 0 <= argmax[m] < ref_logits.shape[1]
        assert rmx[m] - ref_logits[m, argmax[m]] <= band[m]
    return int(exempt.sum())


def unmask_close(got_masked, ref_masked, before_masked, ref_conf_win, win_lo, tau, rtol, what="",
                 got_conf_win=None):
    """Compare unmask decisions of one window (bool arrays [B, D]).

    Returns (decisions compared, fallback ties).  On a fallback tie (no
    candidate passes and the best two oracle confidences lie within the tie
    band: rtol * conf, or, with the GPU's confidences got_conf_win, max(4 x
    their largest relative error over the candidates, 2e-3) * conf if
    smaller) the window must still unmask exactly one candidate, and that
    one must lie within the band of the best."""
    B, D = ref_masked.shape
    n_cmp = n_tie = 0
    for b in range(B):
        W = len(ref_conf_win[b])
        cand = [r for r in range(W) if before_masked[b, win_lo + r]]
        conf = np.asarray(ref_conf_win[b])
        near = {r for r in cand if abs(conf[r] - tau) <= 1e-3}
        passing = [r for r in cand if conf[r] > tau]
        rband = rtol
        if got_conf_win is not None and cand:
            gconf = np.asarray(got_conf_win[b], dtype=np.float64)
            err = max(abs(gconf[r] - conf[r]) / conf[r] for r in cand)
            rband = min(rtol, max(4.0 * err, 2e-3))
        fallback_tie = False
        if not passing and len(cand) >= 2:
            cs = sorted((conf[r] for r in cand), reverse=True)
            fallback_tie = cs[0] - cs[1] <= rband * cs[0]
        if fallback_tie:
            n_tie += 1
            if not near:
                best = max(conf[r] for r in cand)
                got = [r for r in cand if not got_masked[b, win_lo + r]]
                assert len(got) == 1, f"{what}: seq {b} fallback tie unmasked {len(got)} positions"
                assert best - conf[got[0]] <= rband * best, f"{what}: seq {b} fallback pick outside the tie band"
        for r in range(W):
            if r in near or fallback_tie:
                continue
            j = win_lo + r
            assert got_masked[b, j] == ref_masked[b, j], f"{what}: seq {b} position {j} unmask decision differs"
            n_cmp += r in cand
        # outside the window nothing changes
        outside = np.ones(D, bool)
        outside[win_lo:win_lo + W] = False
        assert np.array_equal(got_masked[b, outside], before_masked[b, outside])
    return n_cmp, n_tie


# --------------------------------------------------------------------------
def workload(cfg, seed=0, window=0, S=None, n_masked=None, all_masked=False, plant_rate=None):
    w = bi.make_weights(cfg, seed)
    pre = bi.make_prefix(cfg, seed)
    st = bi.make_block_state(cfg, seed, window, S=S, n_masked=n_masked, all_masked=all_masked)
    plant = carry_plant = None
    if plant_rate is not None:
        plant, carry_plant, _ = bi.make_plants(cfg, seed, w, st, plant_rate)
    return w, pre, st, plant, carry_plant


def gpu_decoder(cfg, w, pre, st, plant=None, carry_plant=None, compact=None):
    from block_diffusion_decoding_amd.decoder import BlockDecoder, Dims
    dims = Dims(cfg.B, cfg.Hq, cfg.Hkv, cfg.d, cfg.hidden, cfg.V, cfg.D, cfg.cap)
    weights = {k: torch.from_numpy(getattr(w, k)) for k in ("E", "Wq", "Wk", "Wv", "Wo", "Wlm")}
    dec = BlockDecoder(dims, weights, dtype=tdt(cfg.dtype), device=DEV, compact=compact)
    if pre.kind == "prefill":
        dec.prefill(pre.prompt)
        for blk in range(pre.committed.shape[1] // cfg.D):
            dec.set_block(pre.committed[:, blk * cfg.D:(blk + 1) * cfg.D], np.zeros((cfg.B, cfg.D), bool))
            dec.commit()
    else:
        dec.set_synthetic_prefix(pre.kv_len, pre.cache_k, pre.cache_v, pre.carry)
    dec.set_block(st.tokens, st.masked, plant, carry_offset=carry_plant)
    return dec


def oracle_seqs(cfg, w, pre, st, plant=None, carry_plant=None):
    m = R.Model.from_weights(w, cfg)
    return m, R.seqs_from_inputs(m, cfg, pre, st, plant, carry_plant)
