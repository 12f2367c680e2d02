"""Per-sequence window progression on one GPU ("Fast-dLLM v2: Efficient
Block-Diffusion LLM" notes, Key designs 3-4: windows of S positions decoded
left to right, each opened by an exact step that refreshes the DualCache
snapshot).

In the lockstep decoder a window ends for the whole batch when its slowest
sequence has decoded it.  Here every sequence moves to its next window as soon
as it has decoded its own, so one batched step mixes sequences that open a
window (an exact step: all D rows recomputed, snapshot refreshed) with
sequences inside one (a DualCache step: their window rows fresh, the other
in-block rows from their snapshot).  The tokens are those of the lockstep
schedule (a sequence without candidates changes no state); the batch needs
fewer steps when the sequences decode at different rates.

One step, every arithmetic part a libbd call:
  * input rows, Q/K/V and output rows of all D block rows of every sequence
    (the exact step's work, for every sequence);
  * before the attention, a DualCache sequence's K/V rows outside its window
    are restored from its snapshot (bd_copy_rows), so its queries see the
    snapshot there, as in a DualCache step;
  * the LM head over each sequence's own window rows, the token shift read
    through the row list (a DualCache sequence's first window position reads
    its snapshot row, as in a DualCache step), then the threshold rule on each
    sequence's own window (bd_threshold_unmask_windows);
  * the sequences that opened a window save their K/V and output rows as
    their new snapshot (bd_copy_rows).
Row buffers: Hcat [2, B, 1 + D, hidden]: Hcat[0] holds this step's output rows,
Hcat[1] the snapshot rows (row 0 = carry).  The step is captured as one HIP
graph; the host writes the per-sequence windows, row lists and row masks
before each replay (step, decode_block).  Queued mode (decode_block_queued):
the same bookkeeping runs on the device (bd_persequence_schedule, first in
the captured step), so the steps are replayed back to back, one ahead of the
host, which only reads the mask bits to stop after the block is done; a step
queued after that finds every sequence finished and changes nothing that the
commit keeps (the commit recomputes the block's rows from its tokens).
"""
from __future__ import annotations

import numpy as np
import torch

from . import ops
from .decoder import BlockDecoder, Dims
from .ops import dense, rows


class PerSequenceDecoder(BlockDecoder):
    window_graphs = False

    def __init__(self, dims: Dims, weights: dict, S: int, dtype=torch.bfloat16, device="cuda"):
        super().__init__(dims, weights, dtype=dtype, device=device, compact=False)
        B, D, hid = dims.B, dims.D, dims.hidden
        assert D % S == 0 and D <= 63
        self.S = S
        dev = self.device
        self.Hcat = torch.zeros(2, B, 1 + D, hid, dtype=dtype, device=dev)
        self.Hcat[1].copy_(self.H)
        self.H = self.Hcat[1]                    # carry and snapshot rows: what the commit writes
        self.snap_k = torch.zeros_like(self.blk_k)
        self.snap_v = torch.zeros_like(self.blk_v)
        self.argmax = torch.zeros(B, S, dtype=torch.int32, device=dev)
        self.conf = torch.zeros(B, S, dtype=torch.float32, device=dev)
        self.maxl = torch.zeros(B, S, dtype=torch.float32, device=dev)
        self.lse = torch.zeros(B, S, dtype=torch.float32, device=dev)
        self.pos = torch.zeros(B, S, dtype=torch.int32, device=dev)
        # per-step host-written inputs, one buffer (one copy per step): restore /
        # save masks [3, B] (64-bit), then the row list [B * S] and windows [B] (int32)
        n64 = 3 * B + (B * S + B + 1) // 2
        self._inbuf = torch.zeros(n64, dtype=torch.int64, device=dev)
        self._stage = torch.zeros(n64, dtype=torch.int64, pin_memory=True)
        self.restore, self.save, self.save_h = self._inbuf[:B], self._inbuf[B:2 * B], self._inbuf[2 * B:3 * B]
        i32 = self._inbuf[3 * B:].view(torch.int32)
        self.row_idx, self.win_lo = i32[:B * S], i32[B * S:B * S + B]
        self._graph = None
        # device schedule (queued mode): win, opening, ran [3, B]; live-step count; kinds [B]
        self.ps_state = torch.zeros(3, B, dtype=torch.int32, device=dev)
        self.ps_live = torch.zeros(1, dtype=torch.int32, device=dev)
        self.ps_kinds = torch.zeros(B, dtype=torch.int32, device=dev)
        self._qgraph = None
        self.win = np.zeros(B, np.int64)         # current window per sequence (D // S = block done)
        self.opening = np.ones(B, bool)          # next step opens the window (exact step)
        self.own_steps = np.zeros(B, np.int64)

    def has_graphs(self) -> bool:
        return self._graph is not None or super().has_graphs()

    # ------------------------------------------------------------ host side
    def begin_block(self):
        self.win[:] = 0
        self.opening[:] = True
        self.own_steps[:] = 0

    def _inputs(self):
        """Row list, windows and masks of the next step from the host state."""
        B, D, S = self.dims.B, self.dims.D, self.S
        nw = D // S
        b = np.arange(B)[:, None]
        active = self.win < nw
        w0 = np.where(active, self.win * S, 0)
        q = w0[:, None] + np.arange(S)[None, :] - 1     # the token shift: position p reads row p - 1
        fresh = self.opening[:, None] | (q >= w0[:, None])
        # Hcat row of (buffer, sequence, row): buffer 0 = this step's rows, 1 = snapshot (row 0 = carry);
        # a DualCache sequence's first window position reads its snapshot row
        ridx = np.where(fresh, b * (1 + D) + q + 1, (B + b) * (1 + D) + q + 1)
        ridx = np.where((q < 0) | ~active[:, None], (B + b) * (1 + D), ridx)
        lo = np.where(active, w0, D)                     # a finished sequence: a window outside the block
        full = np.uint64((1 << D) - 1)
        win_bits = np.uint64((1 << S) - 1) << w0.astype(np.uint64)
        restore = np.where(active & ~self.opening, full & ~win_bits, np.uint64(0))
        save = np.where(active & self.opening, full, np.uint64(0))
        save_h = np.where(active & self.opening, np.uint64(((1 << (D + 1)) - 1) ^ 1), np.uint64(0))  # rows 1 .. D
        st = self._stage.numpy()
        st[:B] = restore.view(np.int64)
        st[B:2 * B] = save.view(np.int64)
        st[2 * B:3 * B] = save_h.view(np.int64)
        s32 = st[3 * B:].view(np.int32)
        s32[:B * S] = ridx.reshape(-1)
        s32[B * S:B * S + B] = lo
        self._inbuf.copy_(self._stage, non_blocking=True)

    # ---------------------------------------------------------------- step
    def _kernels(self, tau, on_device: bool = False):
        dm, W = self.dims, self.W
        B, D, S, hid = dm.B, dm.D, self.S, dm.hidden
        X = self.X
        if on_device:   # the windows, row list and masks from the device state
            ops.bd_persequence_schedule(self.mask_bits, self.ps_state, self.restore, self.save, self.save_h,
                                        self.row_idx, self.win_lo, D=D, S=S, kinds=self.ps_kinds, live=self.ps_live)
        ops.bd_embed_rows(W["E"], self.tokens, self.mask_bits, X, row_off=0, n_rows=D, plant=self.plant)
        kr = rows(D, D, 0)
        ops.bd_qkv_proj(X, dense(B * D), W["Wq"], self.q, dense(B * D), W["Wk"], W["Wv"], self.blk_k, kr,
                        self.blk_v, kr, M=B * D)
        ops.bd_copy_rows(self.restore, self.snap_k, self.blk_k, self.snap_v, self.blk_v)
        ops.bd_block_attn(self.q, self.cache_k, self.cache_v, self.kv_len, self.blk_k, self.blk_v, self.o,
                          D=D, q_off=0)
        ops.bd_linear(self.o, dense(B * D), W["Wo"], self.Hcat[0], rows(D, 1 + D, 1), M=B * D, res=X,
                      rr=dense(B * D))
        ops.bd_lmhead_confidence(self.Hcat.view(-1, hid), self.row_idx, W["Wlm"], self.argmax.view(-1),
                                 self.conf.view(-1), max_logit=self.maxl.view(-1), lse=self.lse.view(-1))
        ops.bd_threshold_unmask_windows(self.conf, self.argmax, self.tokens, self.mask_bits, self.win_lo,
                                        threshold=tau, n_unmasked=self.n_unmasked, unmasked_pos=self.pos)
        ops.bd_copy_rows(self.save, self.blk_k, self.snap_k, self.blk_v, self.snap_v)
        ops.bd_copy_rows(self.save_h, self.Hcat[0], self.Hcat[1])
        self.bits_host.copy_(self.mask_bits, non_blocking=True)

    def capture_step(self, tau: float, on_device: bool = False):
        """Capture the step as one HIP graph (every workspace sized first);
        on_device: the queued mode's step, which starts with the device
        schedule."""
        dm = self.dims
        B, D = dm.B, dm.D
        if self.plant is None:
            self.plant = torch.zeros(B, D, dm.hidden, dtype=self.dtype, device=self.device)
        self.hold_workspaces({
            "attn": ops.bd_block_attn_workspace_size(self.dtype, B, dm.Hq, dm.Hkv, dm.d, D, dm.cap, D),
            "lm": ops.bd_lmhead_workspace_size(self.dtype, B * self.S, dm.hidden, dm.V),
            "gemm": max(ops.bd_qkv_proj_workspace_size(self.dtype, B * D, dm.hidden, dm.Hq * dm.d, dm.Hkv * dm.d),
                        ops.bd_linear_workspace_size(self.dtype, B * D, dm.hidden, dm.Hq * dm.d),
                        ops.bd_linear_workspace_size(self.dtype, B, dm.hidden, dm.Hq * dm.d))})
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self._kernels(tau, on_device)
        if on_device:
            self._qgraph, self._qgraph_tau = g, tau
        else:
            self._graph, self._graph_tau_ps = g, tau
        torch.cuda.synchronize()

    def _advance(self, bits):
        """Move every sequence past the windows it has finished (from the
        current mask bits); a sequence entering a window opens it."""
        nw = self.dims.D // self.S
        for b in range(self.dims.B):
            while self.win[b] < nw and not (bits[b] & np.uint64(((1 << self.S) - 1) << (int(self.win[b]) * self.S))):
                self.win[b] += 1
                self.opening[b] = True

    def done(self) -> bool:
        self._advance(self.mask_bits_host())
        return bool((self.win >= self.dims.D // self.S).all())

    def step(self, tau: float) -> bool:
        """One batched step: every sequence with a masked position left in the
        block opens or continues its own window.  Returns False (and does
        nothing) when every sequence has finished the block.  last_kinds[b]
        is (window, "E" or "DC") of sequence b in this step, or None."""
        if self.done():
            return False
        nw = self.dims.D // self.S
        self.last_kinds = [(int(self.win[b]), "E" if self.opening[b] else "DC") if self.win[b] < nw else None
                           for b in range(self.dims.B)]
        self.own_steps += self.win < nw
        self._inputs()
        if self._graph is not None and tau == self._graph_tau_ps:
            self._graph.replay()
        else:
            self._kernels(tau)
        self._step_done()
        self.opening[self.win < nw] = False
        return True

    def decode_block(self, tau: float) -> int:
        """Decode the current block, every sequence on its own windows, then
        commit it; returns the number of batched steps."""
        self.begin_block()
        n = 0
        while self.step(tau):
            n += 1
        self.commit()
        return n

    def decode_block_queued(self, tau: float) -> int:
        """decode_block with the schedule on the device (needs
        capture_step(tau, on_device=True)): the captured step is replayed back
        to back, one step ahead of the host, which waits for the step before
        the one just queued and stops once the mask bits of the block are all
        clear.  Returns the batched steps in which some sequence took part
        (those of decode_block)."""
        assert self._qgraph is not None and tau == self._qgraph_tau, "capture_step(tau, on_device=True) first"
        D = self.dims.D
        self.begin_block()
        self.ps_state[0].zero_()
        self.ps_state[1].fill_(1)
        self.ps_state[2].zero_()
        self.ps_live.zero_()
        full = np.uint64((1 << D) - 1)
        bits = self.bits_host.numpy().view(np.uint64)
        prev = None
        # every step with a sequence in it decodes at least one of its masked
        # positions, so D steps finish the block; the host sees that one later
        for _ in range(D + 2):
            self._qgraph.replay()
            ev = torch.cuda.Event()
            ev.record()
            if prev is not None:
                prev.synchronize()
                if not (bits & full).any():   # bits of that step or a later one: the block is done
                    break
            prev = ev
        else:
            raise RuntimeError("per-sequence block did not finish within D + 2 steps")
        self._step_done()
        self.commit()
        return int(self.ps_live.item())
