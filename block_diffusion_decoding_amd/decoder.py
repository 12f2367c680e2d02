"""Block-diffusion refinement decoder on one GPU (one attention layer + LM head).

Every arithmetic step runs in libbd's HIP kernels through ``ops``; torch only
allocates device memory and supplies the stream.  Names follow the method
("Fast-dLLM v2: Efficient Block-Diffusion LLM" notes, Key designs 2-4):

* block of D positions, windows (sub-blocks) of S positions, threshold tau;
* exact step (E-step): every block row is recomputed; it also refreshes the
  DualCache snapshot (in-block K/V of all D rows and the output rows);
* DualCache step (DC-step): only the S window rows are recomputed; the other
  in-block K/V and output rows come from the snapshot;
* commit: forward pass over the finished clean block, its K/V appended to the
  block-level cache and its last output row kept as the carry.

Device buffers (per sequence b):
  cache_k/v [B, Hkv, cap, d]   block-level cache, kv_len [B] committed rows
  blk_k/v   [B, D, Hkv, d]     in-block K/V (fresh rows + snapshot rows)
  H         [B, 1 + D, hidden] row 0 = carry, row 1 + j = output row of block
                               position j (so position j is predicted from
                               row j: the token shift is row j - 1 of the block)
  tokens    [B, D] int32, mask_bits [B] (bit j = position j is [MASK])
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from . import ops
from .ops import dense, rows


@dataclass
class Dims:
    B: int
    Hq: int
    Hkv: int
    d: int
    hidden: int
    V: int
    D: int = 32
    cap: int = 0

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv


class BlockDecoder:
    """Owns the device state of a batch of sequences decoded block by block."""

    # capture() also records one graph per window (run_window): worth it when a
    # step slot past the end of a window (whose LM head does no work) costs
    # less than a host wait.  A window graph holds at most window_slots step
    # slots: a window of S positions needs at most S steps, but a slot past its
    # end still runs the step's other kernels (~75 us at the 7B shape, a host
    # wait ~37 us), so wide windows run their first steps as one graph and the
    # rest one by one.
    window_graphs = True
    window_slots = 8
    # X holds the block's input rows between steps (false where X is a
    # working buffer that every step refills)
    input_rows_kept = True

    def slots(self, S: int) -> int:
        """Step slots of a window graph for windows of S positions."""
        return min(S, self.window_slots)

    def __init__(self, dims: Dims, weights: dict, dtype=torch.bfloat16, device="cuda", compact=None):
        """``compact``: run the LM head only on the masked candidates of the
        window (bd_candidate_rows + bd_lmhead_confidence_rows); None = when a
        window has more than 64 rows (B*S > 64), where the LM head is
        MFMA-bound and skipped rows save time."""
        self.dims = dims
        self.compact = compact
        self.dtype = dtype
        self.device = torch.device(device)
        dev, dt = self.device, dtype
        B, D, Hq, Hkv, d, hid = dims.B, dims.D, dims.Hq, dims.Hkv, dims.d, dims.hidden
        self.W = {k: v.to(dev, dt).contiguous() for k, v in weights.items()}
        assert self.W["E"].shape == (dims.V + 1, hid)
        self.cache_k = torch.zeros(B, Hkv, dims.cap, d, dtype=dt, device=dev)
        self.cache_v = torch.zeros_like(self.cache_k)
        self.kv_len = torch.zeros(B, dtype=torch.int32, device=dev)
        self.kv_len_host = np.zeros(B, dtype=np.int32)
        self.blk_k = torch.zeros(B, D, Hkv, d, dtype=dt, device=dev)
        self.blk_v = torch.zeros_like(self.blk_k)
        self.H = torch.zeros(B, 1 + D, hid, dtype=dt, device=dev)
        self.X = torch.zeros(B, D, hid, dtype=dt, device=dev)
        self.q = torch.zeros(B, D, Hq, d, dtype=dt, device=dev)
        self.o = torch.zeros(B, D, Hq, d, dtype=dt, device=dev)
        self.tokens = torch.zeros(B, D, dtype=torch.int32, device=dev)
        self.mask_bits = torch.zeros(B, dtype=torch.int64, device=dev)
        # host copy of the mask bits, refreshed by every step (written by the
        # unmask itself, or by a copy behind it; pinned, so the host only
        # waits for the step's event)
        self.bits_host = torch.zeros(B, dtype=torch.int64, pin_memory=True)
        self._bits_ev = torch.cuda.Event()
        self._bits_fresh = False
        self.plant = None
        self.n_unmasked = torch.zeros(B, dtype=torch.int32, device=dev)
        self._win = {}
        self.last = None
        self.lm_timer = None    # object whose start() / stop() bracket every LM-head call when set
        self._capturing = False
        # captured HIP graphs: ("E" | "DC", s) one step, ("W", s, parity) a window's
        # slots, ("P", s, slot, parity) one slot, ("commit", 0) the commit
        self.graphs = {}
        self._held_ws = {}      # tag -> workspace the captured graphs point into
        self._guard = None      # (bits, mask, n): the step's projections and attention skip a finished window
        self._rings = {}        # S -> [2, D // S, slots(S), B] pinned: mask bits after each step slot of each window
        # whether X [B, D, hidden] holds the current input rows of the whole
        # block (kept so by the fused LM head + unmask, which rewrites the rows
        # of the positions it decodes: DualCache steps then embed nothing)
        self._rows_current = False

    # ------------------------------------------------------------------ state
    def set_synthetic_prefix(self, kv_len, cache_k, cache_v, carry):
        """Committed context given directly (random K/V rows and carry row)."""
        L = np.asarray(kv_len, dtype=np.int32)
        self.cache_k.copy_(torch.as_tensor(cache_k).to(self.device, self.dtype))
        self.cache_v.copy_(torch.as_tensor(cache_v).to(self.device, self.dtype))
        self.kv_len.copy_(torch.from_numpy(L).to(self.device))
        self.kv_len_host = L.copy()
        self.H[:, 0].copy_(torch.as_tensor(carry).to(self.device, self.dtype))

    def set_tokens(self, tokens, masked):
        """Token state of the current block: tokens [B, D], masked [B, D] bool."""
        D = self.dims.D
        t = np.asarray(tokens, dtype=np.int32)
        m = np.asarray(masked, dtype=bool)
        bits = np.zeros(self.dims.B, dtype=np.uint64)
        for j in range(D):
            bits |= m[:, j].astype(np.uint64) << np.uint64(j)
        # pinned copies queued on the stream: no wait for the queued steps
        # (the pinned blocks are not reused before their copies have run)
        self.tokens.copy_(torch.from_numpy(t).pin_memory(), non_blocking=True)
        self.mask_bits.copy_(torch.from_numpy(bits.view(np.int64)).pin_memory(), non_blocking=True)
        self._bits_fresh = False
        self._rows_current = False

    def set_block(self, tokens, masked, plant=None, carry_offset=None):
        """Current block: tokens [B, D], masked [B, D] bool, optional plant
        [B, D, hidden] (offset on the block's input rows) and carry offset."""
        self.set_tokens(tokens, masked)
        if plant is None:
            if self.has_graphs():
                self.plant.zero_()   # captured steps read the persistent plant buffer
            else:
                self.plant = None
        else:
            src = torch.as_tensor(plant).to(self.device, self.dtype)
            if self.plant is None:
                self.plant = src.contiguous().clone()
            else:
                self.plant.copy_(src)
        if carry_offset is not None:
            self.H[:, 0] += torch.as_tensor(carry_offset).to(self.device, self.dtype)
        self._rows_current = False

    def has_graphs(self) -> bool:
        """Whether captured graphs hold pointers into this decoder's buffers."""
        return bool(self.graphs)

    def hold_workspaces(self, needs: dict):
        """Size the shared workspaces for ``needs`` ({tag: bytes}) and keep
        references to them: captured graphs hold their raw pointers, and a
        later, larger call anywhere in the process replaces the shared
        workspace of that tag, which must not free the one the graphs use."""
        self._held_ws = {tag: ops.workspace(n, self.device, tag) for tag, n in needs.items()}

    def new_block(self):
        B, D = self.dims.B, self.dims.D
        self.set_block(np.zeros((B, D), np.int32), np.ones((B, D), bool))

    def mask_bits_host(self) -> np.ndarray:
        """Mask bits [B] (uint64) after the last step, without a blocking
        device-to-host copy when a step produced them."""
        if not self._bits_fresh:
            return self.mask_bits.cpu().numpy().view(np.uint64).copy()
        self._bits_ev.synchronize()
        return self.bits_host.numpy().view(np.uint64).copy()

    def masked_host(self) -> np.ndarray:
        bits = self.mask_bits_host()
        return np.stack([(bits >> np.uint64(j)) & np.uint64(1) for j in range(self.dims.D)], 1).astype(bool)

    # ------------------------------------------------------------ step parts
    def _window(self, s: int, S: int):
        """Per-window LM-head buffers; row_idx expresses the token shift."""
        key = (s, S)
        w = self._win.get(key)
        if w is None:
            B, D = self.dims.B, self.dims.D
            idx = np.array([b * (1 + D) + s * S + r for b in range(B) for r in range(S)], dtype=np.int32)
            w = dict(row_idx=torch.from_numpy(idx).to(self.device),
                     cand_rows=torch.zeros(B * S, dtype=torch.int32, device=self.device),
                     cand_pos=torch.zeros(B * S, dtype=torch.int32, device=self.device),
                     cand_count=torch.zeros(1, dtype=torch.int32, device=self.device),
                     argmax=torch.zeros(B, S, dtype=torch.int32, device=self.device),
                     conf=torch.zeros(B, S, dtype=torch.float32, device=self.device),
                     maxl=torch.zeros(B, S, dtype=torch.float32, device=self.device),
                     lse=torch.zeros(B, S, dtype=torch.float32, device=self.device),
                     pos=torch.zeros(B, S, dtype=torch.int32, device=self.device))
            self._win[key] = w
        return w

    def _forward_rows(self, lo: int, n: int, kept: bool = False):
        """Input rows, Q/K/V and attention of block rows [lo, lo + n).
        Returns (X, its row map, o).  All D rows: X is embedded whole; kept:
        the rows are read in place from X [B, D, hidden], which holds the
        block's current input rows; otherwise the window's rows are embedded
        into a packed [B, n, hidden] view."""
        dm, W = self.dims, self.W
        B, D = dm.B, dm.D
        q = self.q.view(-1)[: B * n * dm.Hq * dm.d].view(B, n, dm.Hq, dm.d)
        o = self.o.view(-1)[: B * n * dm.Hq * dm.d].view(B, n, dm.Hq, dm.d)
        if n == D or kept:
            X, xr = self.X, (dense(B * D) if n == D else rows(n, D, lo))
            if n == D:
                ops.bd_embed_rows(W["E"], self.tokens, self.mask_bits, X, row_off=0, n_rows=D, plant=self.plant)
        else:
            X, xr = self.X.view(-1)[: B * n * dm.hidden].view(B, n, dm.hidden), dense(B * n)
            ops.bd_embed_rows(W["E"], self.tokens, self.mask_bits, X, row_off=lo, n_rows=n, plant=self.plant)
        kr = rows(n, D, lo)
        ops.bd_qkv_proj(X, xr, W["Wq"], q, dense(B * n), W["Wk"], W["Wv"], self.blk_k, kr,
                        self.blk_v, kr, M=B * n, guard=self._guard)
        ops.bd_block_attn(q, self.cache_k, self.cache_v, self.kv_len, self.blk_k, self.blk_v, o,
                          D=D, q_off=lo, guard=self._guard)
        return X, xr, o

    def keeps_rows(self, S: int) -> bool:
        """Whether steps of S-position windows keep X current: the LM head
        runs fused with the unmask (bd_lmhead_unmask_next), which rewrites the
        rows of the positions it decodes."""
        return self.input_rows_kept and not self.uses_compaction(S) and self.dims.B * S <= 64

    def _make_rows_current(self):
        """Embed the whole block into X (after the token state changed from
        the host), so that DualCache steps can read their rows in place."""
        dm = self.dims
        ops.bd_embed_rows(self.W["E"], self.tokens, self.mask_bits, self.X, row_off=0, n_rows=dm.D,
                          plant=self.plant)
        self._rows_current = True

    def _lm_and_unmask(self, s: int, S: int, tau: float, bits_out=None):
        """LM head on the window's rows, then the threshold rule; the new mask
        bits also land in the pinned host tensor bits_out (default bits_host)."""
        bits_out = self.bits_host if bits_out is None else bits_out
        w = self._window(s, S)
        dm = self.dims
        if self.lm_timer is not None:
            self.lm_timer.start()
        fused = False
        if self.uses_compaction(S):
            # only the masked candidates: their conf/argmax land at their window
            # slots; the other slots are not candidates and the unmask ignores them
            ops.bd_candidate_rows(self.mask_bits, w["cand_rows"], w["cand_pos"], w["cand_count"], win_lo=s * S,
                                  win_len=S, rows_per_seq=1 + dm.D)
            ops.bd_lmhead_confidence_rows(self.H.view(-1, dm.hidden), w["cand_rows"], w["cand_pos"], w["cand_count"],
                                          self.W["Wlm"], w["argmax"], w["conf"], max_logit=w["maxl"], lse=w["lse"])
        elif dm.B * S <= 64:
            # one call: the LM head, then its final reduction fused with the
            # threshold rule, which also writes the new bits to host memory
            ops.bd_lmhead_unmask(self.H.view(-1, dm.hidden), w["row_idx"], self.W["Wlm"], w["argmax"], w["conf"],
                                 self.tokens, self.mask_bits, win_lo=s * S, threshold=tau, max_logit=w["maxl"],
                                 lse=w["lse"], n_unmasked=self.n_unmasked, unmasked_pos=w["pos"],
                                 mask_bits_host=bits_out,
                                 next_rows=(self.W["E"], self.plant, self.X) if self.input_rows_kept else None)
            fused = True
        else:
            ops.bd_lmhead_confidence(self.H.view(-1, dm.hidden), w["row_idx"], self.W["Wlm"], w["argmax"],
                                     w["conf"], max_logit=w["maxl"], lse=w["lse"])
        if self.lm_timer is not None:
            self.lm_timer.stop()
        if not fused:
            ops.bd_threshold_unmask(w["conf"], w["argmax"], self.tokens, self.mask_bits, win_lo=s * S,
                                    threshold=tau, n_unmasked=self.n_unmasked, unmasked_pos=w["pos"])
            bits_out.copy_(self.mask_bits, non_blocking=True)
        self.last = w

    def uses_compaction(self, S: int) -> bool:
        return self.compact if self.compact is not None else self.dims.B * S > 64

    def _step_done(self):
        self._bits_ev.record()
        self._bits_fresh = True

    def e_step(self, s: int, S: int, tau: float, eager: bool = False, bits_out=None):
        """Exact step for window s; refreshes the DualCache snapshot."""
        if eager or not self._replay("E", s, S, tau):
            dm = self.dims
            B, D = dm.B, dm.D
            X, xr, o = self._forward_rows(0, D)
            ops.bd_linear(o, dense(B * D), self.W["Wo"], self.H, rows(D, 1 + D, 1), M=B * D,
                          res=X, rr=xr, guard=self._guard)
            self._lm_and_unmask(s, S, tau, bits_out)
        if not self._capturing:
            self._rows_current = self.keeps_rows(S)
            self._step_done()

    def dc_step(self, s: int, S: int, tau: float, eager: bool = False, bits_out=None):
        """DualCache step for window s (snapshot rows outside the window)."""
        kept = self.keeps_rows(S)
        if kept and not self._capturing and not self._rows_current:
            self._make_rows_current()
        if eager or not self._replay("DC", s, S, tau):
            dm = self.dims
            B, D = dm.B, dm.D
            X, xr, o = self._forward_rows(s * S, S, kept=kept)
            ops.bd_linear(o, dense(B * S), self.W["Wo"], self.H, rows(S, 1 + D, 1 + s * S), M=B * S,
                          res=X, rr=xr, guard=self._guard)
            self._lm_and_unmask(s, S, tau, bits_out)
        if not self._capturing:
            self._rows_current = kept
            self._step_done()

    def _commit_kernels(self):
        dm = self.dims
        B, D = dm.B, dm.D
        X, _, o = self._forward_rows(0, D)
        ops.bd_linear(o, rows(1, D, D - 1), self.W["Wo"], self.H, rows(1, 1 + D, 0), M=B,
                      res=X, rr=rows(1, D, D - 1))
        ops.bd_kv_append(self.cache_k, self.cache_v, self.kv_len, self.blk_k, self.blk_v, n_rows=self.dims.D)

    def commit(self, check_capacity: bool = True):
        """Forward over the finished block, append its K/V, keep the carry.
        The capacity is checked on the host mirror of the lengths first."""
        D = self.dims.D
        if check_capacity and np.any(self.kv_len_host + D > self.dims.cap):
            raise ops.BdError("bd_kv_append", 3)
        if not self._replay("commit", 0, 0, 0.0):
            self._commit_kernels()
        self.kv_len_host = self.kv_len_host + D
        self._rows_current = False

    def prefill(self, prompt):
        """Block-aligned prompt [B, P] under the hybrid mask (multi-block
        attention); its K/V fill the cache and its last output row is the carry."""
        dm, W = self.dims, self.W
        B, D = dm.B, dm.D
        prompt = np.asarray(prompt, dtype=np.int32)
        P = prompt.shape[1]
        assert P % D == 0
        dev, dt = self.device, self.dtype
        toks = torch.from_numpy(prompt).to(dev)
        X = torch.empty(B, P, dm.hidden, dtype=dt, device=dev)
        q = torch.empty(B, P, dm.Hq, dm.d, dtype=dt, device=dev)
        o = torch.empty_like(q)
        pk = torch.empty(B, P, dm.Hkv, dm.d, dtype=dt, device=dev)
        pv = torch.empty_like(pk)
        zero_len = torch.zeros(B, dtype=torch.int32, device=dev)
        ops.bd_embed_rows(W["E"], toks, None, X, row_off=0, n_rows=P)
        ops.bd_qkv_proj(X, dense(B * P), W["Wq"], q, dense(B * P), W["Wk"], W["Wv"], pk, dense(B * P),
                        pv, dense(B * P), M=B * P)
        ops.bd_block_attn(q, self.cache_k, self.cache_v, zero_len, pk, pv, o, D=D, q_off=0)
        ops.bd_linear(o, rows(1, P, P - 1), W["Wo"], self.H, rows(1, 1 + D, 0), M=B,
                      res=X, rr=rows(1, P, P - 1))
        self.kv_len.zero_()
        self.kv_len_host = np.zeros(B, dtype=np.int32)
        ops.bd_kv_append(self.cache_k, self.cache_v, self.kv_len, pk, pv, n_rows=P, kv_len_host=self.kv_len_host)
        self.kv_len_host = self.kv_len_host + P

    # ---------------------------------------------------------------- graphs
    def capture(self, S: int, tau):
        """Capture the exact and DualCache step of every window and the commit
        as HIP graphs (through torch's graph API).  Every buffer and workspace
        the steps touch is sized first, so replays allocate nothing; a plant
        buffer always exists (zeros when nothing is planted).  tau: a float
        (fixed in the graphs) or a [B] fp32 device tensor whose values the
        replays read (a threshold schedule without re-capture)."""
        dm = self.dims
        B, D = dm.B, dm.D
        if self.plant is None:
            self.plant = torch.zeros(B, D, dm.hidden, dtype=self.dtype, device=self.device)
        self.hold_workspaces(self._workspace_needs(S))
        for s in range(D // S):
            self._window(s, S)
        torch.cuda.synchronize()
        self.graphs = {}
        self._capturing = True
        try:
            for s in range(D // S):
                for kind, fn in (("E", self.e_step), ("DC", self.dc_step)):
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g):
                        fn(s, S, tau, eager=True)
                    self.graphs[(kind, s)] = g
        finally:
            self._capturing = False
        # a window's first steps in one graph: its exact step and slots(S) - 1
        # DualCache steps (a window never needs more than S: every step decodes
        # at least one masked position of each sequence that has one), each step
        # writing its new mask bits to its own row of the pinned ring.  Steps
        # past the end of the window find no candidate and their LM head does
        # no work.
        # Two sets (ring parities) so that the windows of the next block can
        # be queued before the host has read this block's rings; with
        # windows_complete(S), also every slot as a graph of its own, for
        # runs that start or stop inside a window.
        ring = self._ring(S)
        self._capturing = True
        try:
            for par in range(2 if self.window_graphs else 0):
                for s in range(D // S):
                    # a slot past the end of its window skips its projections and
                    # attention (its LM head skips itself), so dead slots cost little
                    self._guard = (self.mask_bits, ((1 << S) - 1) << (s * S), B)
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g):
                        for i in range(self.slots(S)):
                            (self.e_step if i == 0 else self.dc_step)(s, S, tau, eager=True, bits_out=ring[par, s, i])
                    self.graphs[("W", s, par)] = g
                    for i in range(self.slots(S) if self.windows_complete(S) else 0):
                        g = torch.cuda.CUDAGraph()
                        with torch.cuda.graph(g):
                            (self.e_step if i == 0 else self.dc_step)(s, S, tau, eager=True, bits_out=ring[par, s, i])
                        self.graphs[("P", s, i, par)] = g
        finally:
            self._capturing = False
            self._guard = None
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self._commit_kernels()
        self.graphs[("commit", 0)] = g
        self._graph_S, self._graph_tau = S, tau
        torch.cuda.synchronize()

    def _workspace_needs(self, S: int) -> dict:
        """Workspace bytes per tag that the steps and the commit use."""
        dm = self.dims
        B, D, dt = dm.B, dm.D, self.dtype
        return {"attn": max(ops.bd_block_attn_workspace_size(dt, B, dm.Hq, dm.Hkv, dm.d, n, dm.cap, D)
                            for n in (S, D)),
                "lm": ops.bd_lmhead_workspace_size(dt, B * S, dm.hidden, dm.V),
                "gemm": max([ops.bd_qkv_proj_workspace_size(dt, M, dm.hidden, dm.Hq * dm.d, dm.Hkv * dm.d)
                             for M in (B * S, B * D)] +
                            [ops.bd_linear_workspace_size(dt, M, dm.hidden, dm.Hq * dm.d) for M in (B, B * S, B * D)])}

    def _replay_ok(self, S: int, tau) -> bool:
        """Whether the captured steps match (S, tau): a threshold tensor is read
        by the replayed kernels, so the same tensor (whatever values it holds
        now) matches the capture."""
        if self.lm_timer is not None:
            return False
        same_tau = (tau is self._graph_tau) if isinstance(tau, torch.Tensor) or \
            isinstance(self._graph_tau, torch.Tensor) else tau == self._graph_tau
        return S == self._graph_S and same_tau

    def _replay(self, kind: str, s: int, S: int, tau: float) -> bool:
        g = self.graphs.get((kind, s))
        if g is None or self.lm_timer is not None:
            return False
        if kind != "commit" and not self._replay_ok(S, tau):
            return False
        g.replay()
        if kind != "commit":
            self.last = self._window(s, S)
        return True

    def _ring(self, S: int):
        """Pinned [2, D // S, slots(S), B] mask-bit rings of the windows of S
        positions (kept for the decoder's lifetime: captured window graphs
        write into them), one ring per window and parity so that the windows
        of a block, and of the next block, can run back to back before the
        host reads any of them."""
        r = self._rings.get(S)
        if r is None:
            r = self._rings[S] = torch.zeros(2, self.dims.D // S, self.slots(S), self.dims.B, dtype=torch.int64,
                                             pin_memory=True)
        return r

    def windows_complete(self, S: int) -> bool:
        """Whether a window's slots always finish it: every step unmasks at
        least one masked position of the window in each sequence that has one
        (the fallback of the threshold rule), so S steps always do."""
        return self.slots(S) >= S

    def run_window(self, s: int, S: int, tau, wait: bool = True, parity: int = 0):
        """Window s from its exact step on: slots(S) step slots (one graph
        replay when captured), then one wait.  Returns the mask bits after
        every slot [slots(S), B] (uint64); slot i was a refinement step iff some
        sequence still had a masked position of the window before it.  When
        slots(S) < S the window may still have masked positions afterwards:
        its next steps are DualCache steps.  wait=False only queues the
        window and returns None: window_bits(s, S) reads its ring after a
        later wait (windows_complete(S) makes the next window's launch valid
        without looking).  parity: which of the two rings (and graph sets)."""
        g = self.graphs.get(("W", s, parity))
        ring = self._ring(S)
        if g is not None and self._replay_ok(S, tau):
            g.replay()
            self.last = self._window(s, S)
            self._rows_current = self.keeps_rows(S)
        else:
            self._guard = (self.mask_bits, ((1 << S) - 1) << (s * S), self.dims.B)
            try:
                for i in range(self.slots(S)):
                    (self.e_step if i == 0 else self.dc_step)(s, S, tau, eager=True, bits_out=ring[parity, s, i])
            finally:
                self._guard = None
        self._bits_fresh = False
        if not wait:
            return None
        self.wait()
        return self.window_bits(s, S, parity)

    def run_slots(self, s: int, S: int, tau, i0: int, i1: int, parity: int = 0):
        """Slots i0 .. i1-1 of window s (slot 0: its exact step; the others
        DualCache steps), queued without a wait; slot i writes its mask bits
        to row i of the window's ring (window_bits after a wait)."""
        ring = self._ring(S)
        ok = self._replay_ok(S, tau)
        for i in range(i0, i1):
            g = self.graphs.get(("P", s, i, parity))
            if g is not None and ok:
                if i > 0 and self.keeps_rows(S) and not self._rows_current:
                    self._make_rows_current()   # a DualCache slot reads its rows in place
                g.replay()
                self._rows_current = self.keeps_rows(S)
            else:
                self._guard = (self.mask_bits, ((1 << S) - 1) << (s * S), self.dims.B)
                try:
                    (self.e_step if i == 0 else self.dc_step)(s, S, tau, eager=True, bits_out=ring[parity, s, i])
                finally:
                    self._guard = None
        self.last = self._window(s, S)
        self._bits_fresh = False

    def wait(self):
        """Wait for the queued steps (their mask bits are then on the host).
        Queued windows and slots record no event of their own (an event
        record is a barrier with a cache release between two graphs); the
        wait records one after them."""
        self._bits_ev.record()
        self._bits_ev.synchronize()

    def fence(self) -> torch.cuda.Event:
        """An event recorded after the work queued so far: once it has
        completed, the rings written by that work can be read."""
        ev = torch.cuda.Event()
        ev.record()
        return ev

    def window_bits(self, s: int, S: int, parity: int = 0) -> np.ndarray:
        """Mask bits after every slot of window s's last run [slots(S), B]
        (uint64); valid once that run has finished (run_window or wait)."""
        return self._ring(S)[parity, s].numpy().view(np.uint64).copy()

    # ------------------------------------------------------------------ loop
    def decode_block_windows(self, S: int, tau) -> int:
        """Decode the current block as its captured window graphs launched
        back to back, then commit, with one wait at the end (needs capture(S,
        tau) and windows_complete(S)).  Returns the refinement steps taken:
        the slots before which some sequence had a masked position of the
        window."""
        assert self.windows_complete(S) and self._replay_ok(S, tau) and ("W", 0, 0) in self.graphs
        bits = self.mask_bits_host()
        n_win = self.dims.D // S
        for s in range(n_win):
            self.run_window(s, S, tau, wait=False)
        self.commit()
        self.wait()
        n = 0
        for s in range(n_win):
            ring = self.window_bits(s, S)
            wm = np.uint64(((1 << S) - 1) << (s * S))
            before = np.concatenate([bits[None], ring[:-1]])
            n += int(((before & wm) != 0).any(axis=1).sum())
            bits = ring[-1]
        return n

    def decode_block(self, S: int, tau: float, mode: str = "dual", steps_per_window: int | None = None,
                     on_step=None):
        """Decode the current block window by window (lockstep over the batch),
        then commit it.  With ``steps_per_window`` the number of steps per
        window is fixed (no host synchronisation); otherwise the window ends
        when no position of it is masked in any sequence."""
        D = self.dims.D
        n = 0
        for s in range(D // S):
            k = 0
            while True:
                if steps_per_window is not None:
                    if k >= steps_per_window:
                        break
                else:
                    bits = self.mask_bits_host()
                    wmask = np.uint64(((1 << S) - 1) << (s * S))
                    if not np.any(bits & wmask):
                        break
                kind = "E" if (k == 0 or mode == "exact") else "DC"
                (self.e_step if kind == "E" else self.dc_step)(s, S, tau)
                if on_step is not None:
                    on_step(n, s, kind)
                k += 1
                n += 1
        self.commit()
        return n
