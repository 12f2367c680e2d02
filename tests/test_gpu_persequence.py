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
            unmask_close(got[b:b + 1], q.masked[None], before[None], [res.conf], s_b * S, tau, rtol, what,
                         got_conf_win=[down(dec.conf[b])])
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


# --------------------------------------------------------------------------
# the two calls of the per-sequence step, one by one
# --------------------------------------------------------------------------
def ops():
    from block_diffusion_decoding_amd import ops as o
    return o


@pytest.mark.parametrize("D,S", [(32, 8), (32, 4), (64, 16)])
@pytest.mark.parametrize("tau", [0.9, 0.3])
def test_threshold_unmask_windows_against_oracle_rule(D, S, tau):
    """Each sequence applies the threshold rule to its own window (the
    oracle's rule per sequence, decided in fp32 on both sides); a window at
    D (a sequence that has finished the block) changes nothing.  Tokens,
    mask bits, counts and compacted positions are compared bit for bit."""
    from gpu_util import up
    say(f"[per-sequence] unmask windows D={D} S={S} tau={tau}")
    B = 40
    rng = np.random.default_rng(D * 7 + S)
    conf = rng.choice(np.array([0.05, 0.3, 0.9, 0.95, 0.99], np.float32), size=(B, S)).astype(np.float32)
    conf[::6] = rng.random((len(conf[::6]), S)).astype(np.float32)
    conf[3] = 0.9                                    # exact threshold ties
    conf[4] = 0.25                                   # fallback ties: lowest position wins
    am = rng.integers(0, 150000, size=(B, S)).astype(np.int32)
    masked = rng.random((B, D)) < 0.5
    masked[5] = False                                # no candidates anywhere
    masked[6] = True
    tokens = np.where(masked, 0, rng.integers(0, 150000, size=(B, D))).astype(np.int32)
    win_lo = (rng.integers(0, D // S + 1, size=B) * S).astype(np.int32)
    win_lo[:4] = [D, 0, D - S, D]                    # finished sequences among them
    t_tok, t_bits = up(tokens), up(bi.mask_bits(masked).view(np.int64))
    n = torch.full((B,), -9, dtype=torch.int32, device=DEV)
    pos = torch.full((B, S), -9, dtype=torch.int32, device=DEV)
    ops().bd_threshold_unmask_windows(up(conf), up(am), t_tok, t_bits, up(win_lo), threshold=tau,
                                      n_unmasked=n, unmasked_pos=pos)
    got_t, got_m = t_tok.cpu().numpy(), bi.bits_to_mask(t_bits.cpu().numpy().view(np.uint64), D)
    got_n, got_p = n.cpu().numpy(), pos.cpu().numpy()
    for b in range(B):
        if win_lo[b] >= D:
            rt, rm, rn, rp = tokens[b:b + 1], masked[b:b + 1], [0], -np.ones((1, S), np.int64)
        else:
            rt, rm, rn, rp = R.batch_threshold_unmask(conf[b:b + 1], am[b:b + 1], tokens[b:b + 1], masked[b:b + 1],
                                                      int(win_lo[b]), np.float32(tau))
        what = f"sequence {b} window {win_lo[b]}"
        assert np.array_equal(got_t[b], rt[0]) and np.array_equal(got_m[b], rm[0]), what
        assert got_n[b] == rn[0] and np.array_equal(got_p[b], rp[0]), what


@pytest.mark.parametrize("n_rows,row_shape,dt,pair", [(32, (4, 128), torch.bfloat16, True),
                                                      (33, (1536,), torch.bfloat16, False),
                                                      (64, (4,), torch.float32, True),
                                                      (7, (2, 64), torch.float32, False)])
def test_copy_rows_random_masks(n_rows, row_shape, dt, pair):
    """dst[b, r] = src[b, r] exactly where bit r of row_mask[b] is set; every
    other row of dst is left as it was (one or two tensor pairs)."""
    say(f"[per-sequence] copy rows {n_rows} x {row_shape} {dt} pair={pair}")
    B = 19
    g = torch.Generator().manual_seed(n_rows)
    mk = lambda: torch.randn(B, n_rows, *row_shape, generator=g).to(DEV, dt)
    src0, dst0, src1, dst1 = mk(), mk(), mk(), mk()
    rng = np.random.default_rng(n_rows)
    keep = rng.random((B, n_rows)) < 0.4
    keep[0] = False
    keep[1] = True
    bits = np.zeros(B, np.uint64)
    for r in range(n_rows):
        bits |= keep[:, r].astype(np.uint64) << np.uint64(r)
    want0, want1 = dst0.clone(), dst1.clone()
    kt = torch.from_numpy(keep).to(DEV)
    want0[kt] = src0[kt]
    want1[kt] = src1[kt]
    mask = torch.from_numpy(bits.view(np.int64)).to(DEV)
    if pair:
        ops().bd_copy_rows(mask, src0, dst0, src1, dst1)
    else:
        ops().bd_copy_rows(mask, src0, dst0)
        want1 = dst1
    torch.cuda.synchronize()
    assert torch.equal(dst0, want0) and torch.equal(dst1, want1)


def test_graph_keeps_plant_and_workspaces_after_reset_and_growth():
    """A captured per-sequence step keeps reading its plant buffer after
    new_block() (no plant: the buffer is zeroed, not freed), and its
    workspaces stay alive after larger calls elsewhere replace the shared
    ones: replayed steps equal the steps of a decoder that never captured."""
    cfg = MID
    say("[per-sequence] graph after new_block and workspace growth")
    w, pre, st, plant, _ = workload(cfg, 1, all_masked=True, plant_rate=1.0)
    a = make_decoder(cfg, w, pre, st, None)
    b = make_decoder(cfg, w, pre, st, plant)
    b.capture_step(cfg.tau)
    held = {tag: t.data_ptr() for tag, t in b._held_ws.items()}
    assert set(held) == {"attn", "lm", "gemm"}
    # a larger call anywhere in the process replaces the shared workspace of its
    # tag (ops.workspace grows it); the graph's buffers must survive that
    o = ops()
    for tag, t in b._held_ws.items():
        grown = o.workspace(t.numel() + (1 << 20), b.device, tag)
        assert grown.data_ptr() != held[tag] and o.workspace(0, b.device, tag) is grown
    # and calls through the grown workspaces run
    Bg, cap = 8, 2048
    q = torch.zeros(Bg, 8, 12, 128, dtype=torch.bfloat16, device=DEV)
    kc = torch.zeros(Bg, 2, cap, 128, dtype=torch.bfloat16, device=DEV)
    kb = torch.zeros(Bg, 32, 2, 128, dtype=torch.bfloat16, device=DEV)
    lens = torch.full((Bg,), cap - 32, dtype=torch.int32, device=DEV)
    o.bd_block_attn(q, kc, kc, lens, kb, kb, torch.zeros_like(q), D=32, q_off=8)
    del q, kc, kb
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    for d in (a, b):
        d.new_block()
        d.begin_block()
    n = 0
    while True:
        ra, rb = a.step(cfg.tau), b.step(cfg.tau)
        assert ra == rb
        if not ra:
            break
        torch.cuda.synchronize()
        for x, y in ((a.tokens, b.tokens), (a.mask_bits, b.mask_bits), (a.Hcat, b.Hcat), (a.blk_k, b.blk_k)):
            assert torch.equal(x, y), f"step {n}"
        n += 1
        assert n < 4 * cfg.D
    say(f"    {n} steps replayed, bit-identical to eager")


# --------------------------------------------------------------------------
# queued mode: the schedule on the device
# --------------------------------------------------------------------------
def schedule_rule(B, D, S, bits, win, opening, ran):
    """The per-sequence schedule as bd.h states it, one sequence at a time."""
    nw = D // S
    full, wmask = (1 << D) - 1, (1 << S) - 1
    out = {k: np.zeros(B, np.int64) for k in ("win", "opening", "ran", "win_lo", "kinds")}
    out.update({k: np.zeros(B, np.uint64) for k in ("restore", "save", "save_h")})
    row_idx = np.zeros((B, S), np.int64)
    live = 0
    for b in range(B):
        w, op = int(win[b]), int(opening[b])
        if ran[b]:
            op = 0
        while w < nw and (int(bits[b]) >> (w * S)) & wmask == 0:
            w, op = w + 1, 1
        active = w < nw
        live |= active
        w0 = w * S if active else 0
        out["win"][b], out["opening"][b], out["ran"][b] = w, op, int(active)
        out["restore"][b] = (full & ~(wmask << w0)) if active and not op else 0
        out["save"][b] = full if active and op else 0
        out["save_h"][b] = (full << 1) if active and op else 0
        out["win_lo"][b] = w0 if active else D
        out["kinds"][b] = 2 * w + (0 if op else 1) if active else -1
        for j in range(S):
            q = w0 + j - 1
            if q < 0 or not active:
                row_idx[b, j] = (B + b) * (1 + D)
            else:
                row_idx[b, j] = (b if (op or q >= w0) else B + b) * (1 + D) + q + 1
    return out, row_idx, live


@pytest.mark.parametrize("B,D,S", [(40, 32, 8), (300, 32, 4), (9, 48, 16), (64, 63, 9), (5, 8, 8)])
def test_persequence_schedule_against_the_rule(B, D, S):
    """bd_persequence_schedule against the rule of its declaration, over three
    calls in a row (the state carried between them, bits cleared in between):
    state, copy masks, LM-head rows, windows, kinds and the live count, bit
    for bit."""
    from gpu_util import up
    from block_diffusion_decoding_amd import ops as o
    say(f"[per-sequence] schedule B={B} D={D} S={S}")
    rng = np.random.default_rng(B * 131 + D + S)
    nw = D // S
    masked = rng.random((B, D)) < rng.choice([0.0, 0.05, 0.3, 0.9], size=(B, 1))
    masked[:3] = [np.zeros(D, bool), np.ones(D, bool), np.arange(D) >= D - S]
    state = np.stack([rng.integers(0, nw + 1, B), rng.integers(0, 2, B), rng.integers(0, 2, B)]).astype(np.int32)
    t_state = up(state)
    t_bits = up(bi.mask_bits(masked).view(np.int64))
    masks = torch.zeros(3, B, dtype=torch.int64, device=DEV)
    rows_t = torch.full((B * S,), -7, dtype=torch.int32, device=DEV)
    lo = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    kinds = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    live = torch.zeros(1, dtype=torch.int32, device=DEV)
    ref_live = 0
    for call in range(3):
        bits = bi.mask_bits(masked)
        ref, ref_rows, any_active = schedule_rule(B, D, S, bits, *state)
        ref_live += int(any_active)
        o.bd_persequence_schedule(t_bits, t_state, masks[0], masks[1], masks[2], rows_t, lo, D=D, S=S, kinds=kinds,
                                  live=live)
        got_state = t_state.cpu().numpy()
        got_masks = masks.cpu().numpy().view(np.uint64)
        what = f"call {call}"
        assert np.array_equal(got_state[0], ref["win"]) and np.array_equal(got_state[1], ref["opening"]), what
        assert np.array_equal(got_state[2], ref["ran"]), what
        for i, k in enumerate(("restore", "save", "save_h")):
            assert np.array_equal(got_masks[i], ref[k]), (what, k)
        assert np.array_equal(rows_t.cpu().numpy().reshape(B, S), ref_rows), what
        assert np.array_equal(lo.cpu().numpy(), ref["win_lo"]) and np.array_equal(kinds.cpu().numpy(), ref["kinds"])
        assert int(live.item()) == ref_live, what
        state = got_state
        # the step decodes something in some of the active windows
        for b in range(B):
            if state[2][b]:
                w0 = int(state[0][b]) * S
                pos = np.flatnonzero(masked[b, w0:w0 + S])
                if len(pos) and rng.random() < 0.7:
                    masked[b, w0 + rng.choice(pos, size=rng.integers(1, len(pos) + 1), replace=False)] = False
        t_bits.copy_(up(bi.mask_bits(masked).view(np.int64)))


@pytest.mark.parametrize("S", [4, 8, 16])
def test_per_sequence_queued_equals_host_schedule(S):
    """The queued mode (schedule on the device, steps replayed back to back)
    against the host-scheduled captured steps on the same two blocks: tokens,
    mask bits, the committed cache and lengths, the carry and the number of
    batched steps, bit for bit (the host-scheduled path is the one checked
    against the oracle above), for windows of 4, 8 and 16 positions."""
    cfg = replace(MID, S=S)
    say(f"[per-sequence] queued vs host schedule, {cfg.name} S={S}")
    w, pre, st, plant, _ = workload(cfg, 0, all_masked=True, plant_rate=1.0)
    plant = np.array(plant, copy=True)
    keep = np.random.default_rng(5).random((cfg.B, cfg.D)) < np.array([0.9, 0.6, 0.3, 0.05])[:, None]
    plant[~keep] = 0.0
    plant2 = np.roll(plant, 1, axis=0)
    host = make_decoder(cfg, w, pre, st, plant)
    queued = make_decoder(cfg, w, pre, st, plant)
    host.capture_step(cfg.tau)
    queued.capture_step(cfg.tau, on_device=True)
    for blk, pl in enumerate((plant, plant2)):
        if blk:
            for dec in (host, queued):
                dec.set_block(st.tokens, st.masked, pl)
        n_host = host.decode_block(cfg.tau)
        n_queued = queued.decode_block_queued(cfg.tau)
        torch.cuda.synchronize()
        say(f"    block {blk}: {n_host} steps (host schedule), {n_queued} (device schedule)")
        assert n_host == n_queued
        for name in ("tokens", "mask_bits", "kv_len", "cache_k", "cache_v", "H"):
            assert torch.equal(getattr(host, name), getattr(queued, name)), (blk, name)
