"""Multi-layer block-diffusion decode on one GPU (a Qwen2.5-shaped decoder).

The decoding procedure is BlockDecoder's (exact refresh step at each window
start, DualCache steps, commit + append; "Fast-dLLM v2: Efficient
Block-Diffusion LLM" notes, Key designs 2-4); the forward pass runs a stack of
pre-norm layers (RMSNorm, rotary embedding of queries and keys at absolute
positions, grouped-query attention under the hybrid mask, SwiGLU MLP) and a
final RMSNorm before the LM head.  Every arithmetic step is a libbd call.

Device buffers, beyond BlockDecoder's (L layers):
  cache_k/v [L, B, Hkv, cap, d]  per-layer block-level caches (keys rotated)
  kv_len    [L, B] int32         committed rows (equal across layers; one row
                                 per layer so that one append call covers all
                                 layers and each layer's length moves once)
  blk_k/v   [L, B, D, Hkv, d]    per-layer in-block K/V (fresh + snapshot rows)
  H         [B, 1 + D, hidden]   final normalised rows: row 0 = carry, row
                                 1 + j = position j (the LM head input)
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from . import ops
from .decoder import BlockDecoder, Dims
from .ops import dense, rows


@dataclass
class ModelDims(Dims):
    n_layers: int = 1
    inter: int = 0
    eps: float = 1e-6
    theta: float = 1e6


class ModelDecoder(BlockDecoder):
    """Owns the device state of a batch decoded by the multi-layer model.

    weights: {"E": [V+1, hid], "Wlm": [V, hid], "layers": [{"Wq", "Wk", "Wv",
    "Wo", "Wg", "Wu", "Wd"}, ...]} (out x in); gate and up are stored as one
    [2*inter, hid] matrix so that one GEMM makes both."""

    # a step slot past the end of a window still runs every layer: no window graphs
    window_graphs = False
    # X is the residual stream of the step's rows, refilled by every step
    input_rows_kept = False
    # below this many rows the MLP's RMSNorm is folded into the gate/up
    # projection (its streaming kernel takes the sums of squares from the A
    # fragments it loads anyway: 32.9 us against 37.3 for norm + projection at
    # 128 rows of the 1.5B layer); with 256-row tiles the fold measured slower
    # (69.0 against 64.6 us at 512 rows), and there the output projection's
    # K-split reduction writes the norm for free
    fold_norm_below = 256

    def __init__(self, dims: ModelDims, weights: dict, dtype=torch.bfloat16, device="cuda", compact=None):
        top = {"E": weights["E"], "Wlm": weights["Wlm"]}
        # BlockDecoder's single-layer buffers are replaced below; give it the
        # first layer's attention weights so its constructor has what it reads
        l0 = weights["layers"][0]
        super().__init__(dims, {**top, "Wq": l0["Wq"], "Wk": l0["Wk"], "Wv": l0["Wv"], "Wo": l0["Wo"]},
                         dtype=dtype, device=device, compact=compact)
        dev, dt = self.device, dtype
        Lr, B, D, Hq, Hkv, d, hid, I = dims.n_layers, dims.B, dims.D, dims.Hq, dims.Hkv, dims.d, dims.hidden, dims.inter
        for k in ("Wq", "Wk", "Wv", "Wo"):
            del self.W[k]
        self.layers = []
        for lw in weights["layers"]:
            t = lambda a: torch.as_tensor(a).to(dev, dt).contiguous()
            self.layers.append({"Wq": t(lw["Wq"]), "Wk": t(lw["Wk"]), "Wv": t(lw["Wv"]), "Wo": t(lw["Wo"]),
                                "Wgu": torch.cat([t(lw["Wg"]), t(lw["Wu"])], 0).contiguous(), "Wd": t(lw["Wd"])})
        assert len(self.layers) == Lr
        self.cache_k = torch.zeros(Lr, B, Hkv, dims.cap, d, dtype=dt, device=dev)
        self.cache_v = torch.zeros_like(self.cache_k)
        self.kv_len = torch.zeros(Lr, B, dtype=torch.int32, device=dev)
        self.blk_k = torch.zeros(Lr, B, D, Hkv, d, dtype=dt, device=dev)
        self.blk_v = torch.zeros_like(self.blk_k)
        self.hbuf = torch.zeros(B * D, hid, dtype=dt, device=dev)
        self.act = torch.zeros(B * D, I, dtype=dt, device=dev)

    # ------------------------------------------------------------------ layers
    def _layers(self, X, h, q, o, a, M, n, lo, kr, attn_kv, layer_ids, final=None):
        """Layers ``layer_ids`` over M = B*n fresh rows X (block rows
        lo .. lo+n-1 of every sequence), the residual stream, updated in
        place.  attn_kv(l) gives layer l's (k_cache, v_cache, kv_len, k_blk,
        v_blk); the fresh K/V go to rows kr of k_blk/v_blk, rotated at
        positions kv_len[b] + lo + i.  h holds rmsnorm(X) for the next
        sublayer: the projections into the residual stream also normalise
        their result (bd_linear_residual_rmsnorm), except that below
        fold_norm_below rows the MLP's norm is folded into the gate/up
        projection instead (bd_gate_up_swiglu_rmsnorm: one launch fewer where
        the output projection has no reduction to carry the norm).  After the last layer that
        norm goes to ``final`` = (buffer, row map) when given (the final
        RMSNorm in front of the LM head), else it is not taken."""
        dm = self.dims
        ids = list(layer_ids)
        ops.bd_rmsnorm(X, dense(M), h, dense(M), M=M, eps=dm.eps)
        for idx, l in enumerate(ids):
            lw = self.layers[l]
            kc, vc, kvl, kb, vb = attn_kv(l)
            ops.bd_qkv_proj_rope(h, dense(M), lw["Wq"], q, dense(M), lw["Wk"], lw["Wv"], kb, kr, vb, kr, kvl, M=M,
                                 d=dm.d, n_rows=n, pos_off=lo, theta=dm.theta)
            ops.bd_block_attn(q, kc, vc, kvl, kb, vb, o, D=dm.D, q_off=lo)
            if M < self.fold_norm_below:
                # the pre-MLP RMSNorm rides on the gate/up projection's streaming kernel
                ops.bd_linear(o, dense(M), lw["Wo"], X, dense(M), M=M, res=X, rr=dense(M))
                ops.bd_gate_up_swiglu_rmsnorm(X, dense(M), lw["Wgu"], a, dense(M), M=M, eps=dm.eps)
            else:
                # many rows: the output projection's K-split reduction writes the norm
                ops.bd_linear_residual_rmsnorm(o, dense(M), lw["Wo"], X, dense(M), h, dense(M), M=M, eps=dm.eps)
                ops.bd_gate_up_swiglu(h, dense(M), lw["Wgu"], a, dense(M), M=M)
            if idx < len(ids) - 1:
                ops.bd_linear_residual_rmsnorm(a, dense(M), lw["Wd"], X, dense(M), h, dense(M), M=M, eps=dm.eps)
            elif final is not None:
                ops.bd_linear_residual_rmsnorm(a, dense(M), lw["Wd"], X, dense(M), final[0], final[1], M=M,
                                               eps=dm.eps)
            else:
                ops.bd_linear(a, dense(M), lw["Wd"], X, dense(M), M=M, res=X, rr=dense(M))

    def _forward_block_rows(self, lo: int, n: int, final=None):
        """Block rows [lo, lo + n) of every sequence through all layers;
        returns the residual stream X [B, n, hidden] after the last layer
        (with ``final`` = (buffer, row map) the final RMSNorm is written
        there on the way)."""
        dm = self.dims
        B, D = dm.B, dm.D
        M = B * n
        X = self.X.view(-1)[: M * dm.hidden].view(B, n, dm.hidden)
        q = self.q.view(-1)[: M * dm.Hq * dm.d].view(B, n, dm.Hq, dm.d)
        o = self.o.view(-1)[: M * dm.Hq * dm.d].view(B, n, dm.Hq, dm.d)
        ops.bd_embed_rows(self.W["E"], self.tokens, self.mask_bits, X, row_off=lo, n_rows=n)
        self._layers(X, self.hbuf, q, o, self.act, M, n, lo, rows(n, D, lo),
                     lambda l: (self.cache_k[l], self.cache_v[l], self.kv_len[l], self.blk_k[l], self.blk_v[l]),
                     range(dm.n_layers), final)
        return X

    # ------------------------------------------------------------------ steps
    def e_step(self, s: int, S: int, tau: float, eager: bool = False, bits_out=None):
        """Exact step for window s; refreshes every layer's DualCache snapshot."""
        if eager or not self._replay("E", s, S, tau):
            D = self.dims.D
            self._forward_block_rows(0, D, final=(self.H, rows(D, 1 + D, 1)))
            self._lm_and_unmask(s, S, tau, bits_out)
        if not self._capturing:
            self._step_done()

    def dc_step(self, s: int, S: int, tau: float, eager: bool = False, bits_out=None):
        """DualCache step for window s (every layer's snapshot rows outside the
        window; the row feeding the window's first position stays in H)."""
        if eager or not self._replay("DC", s, S, tau):
            D = self.dims.D
            self._forward_block_rows(s * S, S, final=(self.H, rows(S, 1 + D, 1 + s * S)))
            self._lm_and_unmask(s, S, tau, bits_out)
        if not self._capturing:
            self._step_done()

    def _commit_kernels(self):
        dm = self.dims
        B, D, Lr = dm.B, dm.D, dm.n_layers
        X = self._forward_block_rows(0, D)
        ops.bd_rmsnorm(X, rows(1, D, D - 1), self.H, rows(1, 1 + D, 0), M=B, eps=dm.eps)
        # one append for all layers: the per-layer caches, lengths and block
        # buffers are contiguous along the layer axis
        ops.bd_kv_append(self.cache_k.view(Lr * B, dm.Hkv, dm.cap, dm.d), self.cache_v.view(Lr * B, dm.Hkv, dm.cap, dm.d),
                         self.kv_len.view(Lr * B), self.blk_k.view(Lr * B, D, dm.Hkv, dm.d),
                         self.blk_v.view(Lr * B, D, dm.Hkv, dm.d), n_rows=D)

    def prefill(self, prompt):
        """Block-aligned prompts [B, P] through all layers under the
        block-causal mask; each layer's K/V fill its cache and the last row's
        final normalised state is the carry."""
        dm, W = self.dims, self.W
        B, D = dm.B, dm.D
        prompt = np.asarray(prompt, dtype=np.int32)
        P = prompt.shape[1]
        assert P % D == 0 and P <= dm.cap
        dev, dt = self.device, self.dtype
        M = B * P
        toks = torch.from_numpy(prompt).to(dev)
        X = torch.empty(B, P, dm.hidden, dtype=dt, device=dev)
        h = torch.empty(M, dm.hidden, dtype=dt, device=dev)
        q = torch.empty(B, P, dm.Hq, dm.d, dtype=dt, device=dev)
        o = torch.empty_like(q)
        a = torch.empty(M, dm.inter, dtype=dt, device=dev)
        pk = torch.empty(B, P, dm.Hkv, dm.d, dtype=dt, device=dev)
        pv = torch.empty_like(pk)
        self.kv_len.zero_()
        ops.bd_embed_rows(W["E"], toks, None, X, row_off=0, n_rows=P)
        # one K/V buffer serves every layer: layer l's rows are appended to
        # its cache (and its length moves to P) before layer l + 1 writes them
        for l in range(dm.n_layers):
            self._layers(X, h, q, o, a, M, P, 0, dense(M),
                         lambda l: (self.cache_k[l], self.cache_v[l], self.kv_len[l], pk, pv), (l,))
            ops.bd_kv_append(self.cache_k[l], self.cache_v[l], self.kv_len[l], pk, pv, n_rows=P)
        ops.bd_rmsnorm(X, rows(1, P, P - 1), self.H, rows(1, 1 + D, 0), M=B, eps=dm.eps)
        self.kv_len_host = np.full(B, P, dtype=np.int32)

    # ---------------------------------------------------------------- graphs
    def _workspace_needs(self, S: int) -> dict:
        dm = self.dims
        B, D, dt = dm.B, dm.D, self.dtype
        Ms = (B * S, B * D)
        gemm = [ops.bd_qkv_proj_rope_workspace_size(dt, M, dm.hidden, dm.Hq * dm.d, dm.Hkv * dm.d) for M in Ms]
        gemm += [ops.bd_linear_workspace_size(dt, M, N, K) for M in Ms
                 for N, K in ((dm.hidden, dm.Hq * dm.d), (dm.hidden, dm.inter))]
        return {"attn": max(ops.bd_block_attn_workspace_size(dt, B, dm.Hq, dm.Hkv, dm.d, n, dm.cap, D) for n in (S, D)),
                "lm": ops.bd_lmhead_workspace_size(dt, B * S, dm.hidden, dm.V),
                "gemm": max(gemm)}

    # ------------------------------------------------------------------- run
    def generate(self, prompt, n_blocks: int, S: int, tau: float, on_step=None) -> np.ndarray:
        """Prefill, then decode n_blocks blocks; returns the generated token ids
        [B, n_blocks * D] (host)."""
        self.prefill(prompt)
        out = []
        for _ in range(n_blocks):
            self.new_block()
            self.decode_block(S, tau, on_step=on_step)
            out.append(self.tokens.cpu().numpy().copy())
        return np.concatenate(out, axis=1)
