"""Captured HIP graphs of the refinement steps against eager execution.

Two decoders get identical inputs; one runs eagerly, the other replays the
captured exact / DualCache / commit graphs.  Every replay is checked
bit-for-bit against the eager result (same kernels, same inputs), with the
eager decoder's own work and host synchronisations between the replays, over
several windows and two blocks."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import bd_inputs as bi
from gpu_util import gpu_decoder, say, workload

pytestmark = pytest.mark.gpu

MID = replace(bi.C2, name="mid", B=4, V=20000, len_lo_blocks=4, len_hi_blocks=20, cap=1024)


def state(dec):
    w = dec.last
    return [dec.tokens.clone(), dec.mask_bits.clone(), dec.H.clone(), dec.blk_k.clone(), dec.blk_v.clone(),
            w["conf"].clone(), w["argmax"].clone(), dec.cache_k.clone(), dec.kv_len.clone()]


def test_captured_steps_replay_like_eager():
    say("[graphs] mid-size decoder, captured vs eager")
    cfg = MID
    w, pre, st, plant, _ = workload(cfg, 0, all_masked=True, plant_rate=None)
    eager = gpu_decoder(cfg, w, pre, st)
    graph = gpu_decoder(cfg, w, pre, st)
    S, tau = cfg.S, 0.3          # low threshold: several tokens per step
    graph.capture(S, tau)
    rng = np.random.default_rng(0)
    n_cmp = 0
    for blk in range(2):
        plant = bi.normal(blk, "plant", (cfg.B, cfg.D, cfg.hidden), 0.5, "bf16")
        plant[rng.random((cfg.B, cfg.D)) < 0.5] = 0.0
        for d in (eager, graph):
            d.set_block(np.zeros((cfg.B, cfg.D), np.int32), np.ones((cfg.B, cfg.D), bool), plant)
        for s in range(cfg.D // S):
            for k in range(3):
                kind = "E" if k == 0 else "DC"
                (eager.e_step if kind == "E" else eager.dc_step)(s, S, tau)
                torch.cuda.synchronize()
                (graph.e_step if kind == "E" else graph.dc_step)(s, S, tau)
                torch.cuda.synchronize()
                for a, b in zip(state(eager), state(graph)):
                    assert torch.equal(a, b), f"block {blk} window {s} step {k} ({kind}) differs"
                # the host copy of the mask bits that each step refreshes
                want = eager.mask_bits.cpu().numpy().view(np.uint64)
                assert np.array_equal(eager.mask_bits_host(), want) and np.array_equal(graph.mask_bits_host(), want)
                n_cmp += 1
        eager.set_tokens(eager.tokens.cpu().numpy(), np.zeros((cfg.B, cfg.D), bool))
        graph.set_tokens(graph.tokens.cpu().numpy(), np.zeros((cfg.B, cfg.D), bool))
        eager.commit()
        graph.commit()
        torch.cuda.synchronize()
        for a, b in zip(state(eager), state(graph)):
            assert torch.equal(a, b), f"commit of block {blk} differs"
    assert n_cmp == 2 * (cfg.D // S) * 3


def test_captured_steps_follow_a_device_threshold_schedule():
    """Graphs captured with a threshold tensor replay with the values it holds
    at each replay: a schedule (here lowered every step, one value per
    sequence) gives the same results as eager steps with those thresholds."""
    say("[graphs] device threshold schedule")
    cfg = MID
    w, pre, st, _, _ = workload(cfg, 0, all_masked=True, plant_rate=None)
    eager = gpu_decoder(cfg, w, pre, st)
    graph = gpu_decoder(cfg, w, pre, st)
    S = cfg.S
    tau_dev = torch.full((cfg.B,), 0.9, dtype=torch.float32, device="cuda")
    graph.capture(S, tau_dev)
    plant = bi.normal(3, "plant", (cfg.B, cfg.D, cfg.hidden), 0.5, "bf16")
    for d in (eager, graph):
        d.set_block(np.zeros((cfg.B, cfg.D), np.int32), np.ones((cfg.B, cfg.D), bool), plant)
    step = 0
    for s in range(cfg.D // S):
        for k in range(3):
            kind = "E" if k == 0 else "DC"
            taus = np.float32(0.9 - 0.1 * step) + np.float32(0.05) * np.arange(cfg.B, dtype=np.float32)
            tau_e = torch.from_numpy(taus).cuda()
            (eager.e_step if kind == "E" else eager.dc_step)(s, S, tau_e, eager=True)
            torch.cuda.synchronize()
            tau_dev.copy_(torch.from_numpy(taus))
            (graph.e_step if kind == "E" else graph.dc_step)(s, S, tau_dev)
            torch.cuda.synchronize()
            for a, b in zip(state(eager), state(graph)):
                assert torch.equal(a, b), f"window {s} step {k} ({kind}) differs"
            step += 1
    assert len(graph.graphs) > 0


@pytest.mark.parametrize("compact,S", [(None, 8), (True, 8), (None, 16)])
def test_window_graphs_decode_like_single_steps(compact, S):
    """One captured graph per window (its exact step and slots(S) - 1
    DualCache step slots, then single DualCache steps while the window has
    masked positions) against single eager steps taken until the window is
    decoded: the same mask bits after every refinement step, the same tokens
    after every window, the same committed cache and carry after every block.
    Slots past the end of the window change no token and no bit.  compact:
    the LM head over the masked candidates only (row list, device count);
    None here: the LM head fused with the unmask.  S = 16: a window graph
    holds 8 of the window's up to 16 steps."""
    say(f"[graphs] window graphs vs single steps (compact={compact}, S={S})")
    cfg = replace(MID, S=S)
    w, pre, st, _, _ = workload(cfg, 0, all_masked=True, plant_rate=None)
    eager = gpu_decoder(cfg, w, pre, st, compact=compact)
    graph = gpu_decoder(cfg, w, pre, st, compact=compact)
    tau = 0.6 if S <= 8 else 1.0     # 1.0: one token per step, so a wide window outlasts its graph
    graph.capture(S, tau)
    slots = graph.slots(S)
    longest = 0
    rng = np.random.default_rng(5)
    wins = cfg.D // S
    n_steps = 0
    for blk in range(2):
        plant = bi.normal(10 + blk, "plant", (cfg.B, cfg.D, cfg.hidden), 0.5, "bf16")
        plant[rng.random((cfg.B, cfg.D)) < 0.5] = 0.0
        for d in (eager, graph):
            d.set_block(np.zeros((cfg.B, cfg.D), np.int32), np.ones((cfg.B, cfg.D), bool), plant)
        for s in range(wins):
            wmask = np.uint64(((1 << S) - 1) << (s * S))
            seen = []
            k = 0
            while k == 0 or (eager.mask_bits_host() & wmask).any():
                (eager.e_step if k == 0 else eager.dc_step)(s, S, tau)
                seen.append(eager.mask_bits_host())
                k += 1
            assert k <= S
            longest = max(longest, k)
            ring = graph.run_window(s, S, tau)
            assert ring.shape == (slots, cfg.B)
            for i in range(slots):
                want = seen[i] if i < k else seen[-1]
                assert np.array_equal(ring[i], want), f"block {blk} window {s} slot {i}"
            for i in range(slots, k):       # the rest of a wide window, one step at a time
                graph.dc_step(s, S, tau)
                assert np.array_equal(graph.mask_bits_host(), seen[i]), f"block {blk} window {s} step {i}"
            assert torch.equal(eager.tokens, graph.tokens) and torch.equal(eager.mask_bits, graph.mask_bits)
            assert np.array_equal(graph.mask_bits_host(), seen[-1])
            n_steps += k
        for d in (eager, graph):
            d.commit()
        torch.cuda.synchronize()
        assert torch.equal(eager.cache_k, graph.cache_k) and torch.equal(eager.cache_v, graph.cache_v)
        assert torch.equal(eager.kv_len, graph.kv_len) and torch.equal(eager.H[:, 0], graph.H[:, 0])
    assert n_steps > 2 * wins
    assert S <= slots or longest > slots


def test_window_graphs_follow_a_device_threshold_schedule():
    """Window graphs captured with a threshold tensor read the values it holds
    at each replay: per-sequence thresholds changed between windows give the
    same mask bits after every slot as eager single steps with those values."""
    say("[graphs] window graphs, device threshold schedule")
    cfg = MID
    w, pre, st, _, _ = workload(cfg, 0, all_masked=True, plant_rate=None)
    eager = gpu_decoder(cfg, w, pre, st)
    graph = gpu_decoder(cfg, w, pre, st)
    S = cfg.S
    tau_dev = torch.full((cfg.B,), 0.9, dtype=torch.float32, device="cuda")
    graph.capture(S, tau_dev)
    plant = bi.normal(4, "plant", (cfg.B, cfg.D, cfg.hidden), 0.5, "bf16")
    for d in (eager, graph):
        d.set_block(np.zeros((cfg.B, cfg.D), np.int32), np.ones((cfg.B, cfg.D), bool), plant)
    for s in range(cfg.D // S):
        taus = np.float32(0.3 + 0.2 * s) + np.float32(0.1) * np.arange(cfg.B, dtype=np.float32)
        tau_e = torch.from_numpy(taus).cuda()
        tau_dev.copy_(torch.from_numpy(taus))
        ring = graph.run_window(s, S, tau_dev)
        for i in range(graph.slots(S)):
            (eager.e_step if i == 0 else eager.dc_step)(s, S, tau_e, eager=True)
            assert np.array_equal(ring[i], eager.mask_bits_host()), f"window {s} slot {i}"
        assert torch.equal(eager.tokens, graph.tokens)


@pytest.mark.parametrize("compact,S,tau", [(None, 8, 0.6), (True, 8, 0.6), (None, 4, 1.0)])
def test_block_windows_back_to_back_decode_like_single_steps(compact, S, tau):
    """A block decoded as its window graphs launched back to back with one
    wait at the end (decode_block_windows) against the eager block loop that
    waits for the mask bits after every step: the same steps, tokens,
    committed cache and carry, over two blocks.  tau = 1.0: about one token
    per sequence and step, so the windows use most of their S slots."""
    say(f"[graphs] back-to-back window graphs vs eager block loop (compact={compact}, S={S}, tau={tau})")
    cfg = replace(MID, S=S)
    w, pre, st, _, _ = workload(cfg, 0, all_masked=True, plant_rate=None)
    eager = gpu_decoder(cfg, w, pre, st, compact=compact)
    graph = gpu_decoder(cfg, w, pre, st, compact=compact)
    graph.capture(S, tau)
    assert graph.windows_complete(S)
    rng = np.random.default_rng(8)
    for blk in range(2):
        plant = bi.normal(20 + blk, "plant", (cfg.B, cfg.D, cfg.hidden), 0.5, "bf16")
        plant[rng.random((cfg.B, cfg.D)) < 0.5] = 0.0
        for d in (eager, graph):
            d.set_block(np.zeros((cfg.B, cfg.D), np.int32), np.ones((cfg.B, cfg.D), bool), plant)
        tok_before = eager.tokens.clone()
        n_e = eager.decode_block(S, tau)
        n_g = graph.decode_block_windows(S, tau)
        torch.cuda.synchronize()
        assert n_e == n_g, f"block {blk}: {n_e} eager steps, {n_g} in the window graphs"
        assert cfg.D // S <= n_g <= cfg.D
        assert torch.equal(eager.tokens, graph.tokens) and not torch.equal(tok_before, graph.tokens)
        assert int(graph.mask_bits_host().max()) == 0
        assert torch.equal(eager.cache_k, graph.cache_k) and torch.equal(eager.cache_v, graph.cache_v)
        assert torch.equal(eager.kv_len, graph.kv_len) and torch.equal(eager.H[:, 0], graph.H[:, 0])
