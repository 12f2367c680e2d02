"""v1-style decoding of a full-attention diffusion LM with the block-wise
approximate KV cache, on one GPU ("Fast-dLLM: Training-free Acceleration of
Diffusion LLM by Enabling KV Cache and Parallel Decoding" article, Core
techniques 1 and 2).

The sequence is [prompt | generation region]; every position attends to
every position.  The generation region starts masked and is decoded block
by block: the first step of a block is an exact forward pass over the whole
sequence (a refresh), whose K/V outside the block become the DualCache
(prefix rows, then suffix rows) and whose output row before the block is the
carry; the following steps recompute only the block's D rows, attending over
the cache and the fresh block.  Prediction for block position j: output row
j - 1 (the one-layer model's token shift).  Every arithmetic step is a libbd
call:

* the exact pass is bd_block_attn with one "block" spanning the whole
  sequence (n_blk = D_attn = T: every key visible) and no cache;
* a DualCache step is bd_block_attn over the cache (T - D rows) plus the D
  fresh rows, all visible.

Device buffers (B sequences of T = P + gen_len positions, P % D == 0):
  tok_full [B, T] int32, bits_full [B, T/D] 64-bit: tokens and [MASK] bits
      of the whole sequence in D-position entries (the embedding call's
      layout); the current block's state lives in tok_blk [B, D] / bits_blk
      [B] while it is refined and is written back before each exact pass
  X/H_full [B, T, hidden], q/o_full [B, T, Hq*d], k/v_full [B, T, Hkv*d]
  cache_k/v [B, Hkv, T - D, d], kv_len [B]: the DualCache
  Xb [B, D, hidden], qb/ob [B, D, Hq*d], kb/vb [B, D, Hkv*d]
  Hb [B, 1 + D, hidden]: row 0 = carry, row 1 + j = block position j
"""
from __future__ import annotations

import numpy as np
import torch

from . import ops
from .ops import dense, rows


class FullAttnDecoder:
    def __init__(self, weights: dict, B: int, P: int, gen_len: int, Hq: int, Hkv: int, d: int, D: int = 32,
                 dtype=torch.bfloat16, device="cuda"):
        assert P % D == 0 and gen_len % D == 0 and P >= D and D <= 64
        t = lambda a: torch.as_tensor(a).to(device, dtype).contiguous()
        self.W = {k: t(weights[k]) for k in ("E", "Wq", "Wk", "Wv", "Wo", "Wlm")}
        self.B, self.P, self.D, self.T = B, P, D, P + gen_len
        self.Hq, self.Hkv, self.d = Hq, Hkv, d
        self.V, self.hidden = self.W["Wlm"].shape
        dev, dt, T, hid = torch.device(device), dtype, self.T, self.hidden
        self.device, self.dtype = dev, dt
        z = lambda *s, dtype=dt: torch.zeros(*s, dtype=dtype, device=dev)
        self.tok_full = z(B, T, dtype=torch.int32)
        self.bits_full = z(B, T // D, dtype=torch.int64)
        self.X_full, self.H_full = z(B, T, hid), z(B, T, hid)
        self.q_full, self.o_full = z(B, T, Hq * d), z(B, T, Hq * d)
        self.k_full, self.v_full = z(B, T, Hkv * d), z(B, T, Hkv * d)
        self.cache_k, self.cache_v = z(B, Hkv, T - D, d), z(B, Hkv, T - D, d)
        self.kv_len = z(B, dtype=torch.int32)
        self.no_cache = z(B, dtype=torch.int32)
        self.tok_blk = z(B, D, dtype=torch.int32)
        self.bits_blk = z(B, dtype=torch.int64)
        self.Xb, self.Hb = z(B, D, hid), z(B, 1 + D, hid)
        self.qb, self.ob = z(B, D, Hq * d), z(B, D, Hq * d)
        self.kb, self.vb = z(B, D, Hkv * d), z(B, D, Hkv * d)
        self.argmax = z(B, D, dtype=torch.int32)
        self.conf = z(B, D, dtype=torch.float32)
        self.n_unmasked = z(B, dtype=torch.int32)
        self.unmasked_pos = z(B, D, dtype=torch.int32)
        self.lse = z(B, D, dtype=torch.float32)
        self.max_logit = z(B, D, dtype=torch.float32)
        # token-shift rows: the DualCache step reads Hb row j (row 0 = carry)
        self.rows_dual = torch.from_numpy((np.arange(B)[:, None] * (1 + D) + np.arange(D)[None, :])
                                          .astype(np.int32).reshape(-1)).to(dev)
        self.rows_exact = z(B * D, dtype=torch.int32)
        self.block = -1

    # ------------------------------------------------------------ state
    def set_prompts(self, prompts):
        """prompts [B, P]; the generation region becomes all [MASK]."""
        prompts = np.asarray(prompts, dtype=np.int32)
        B, P, D, T = self.B, self.P, self.D, self.T
        assert prompts.shape == (B, P)
        tok = np.zeros((B, T), np.int32)
        tok[:, :P] = prompts
        bits = np.zeros((B, T // D), np.uint64)
        bits[:, P // D:] = np.uint64((1 << D) - 1) if D < 64 else np.uint64(0xFFFFFFFFFFFFFFFF)
        self.tok_full.copy_(torch.from_numpy(tok))
        self.bits_full.copy_(torch.from_numpy(bits.view(np.int64)))
        self.block = -1

    def begin_block(self, k: int):
        """Block k becomes the current block (its state moves to tok_blk /
        bits_blk; the previous block's final state goes back to the full
        arrays)."""
        if self.block >= 0:
            self._sync_block()
        lo = self.P + k * self.D
        self.block = k
        self.tok_blk.copy_(self.tok_full[:, lo:lo + self.D])
        self.bits_blk.copy_(self.bits_full[:, lo // self.D])
        self.rows_exact.copy_(torch.from_numpy((np.arange(self.B)[:, None] * self.T + lo - 1 +
                                                np.arange(self.D)[None, :]).astype(np.int32).reshape(-1)))

    def _sync_block(self):
        if self.block < 0:          # no block begun since the prompts were set
            return
        lo = self.P + self.block * self.D
        self.tok_full[:, lo:lo + self.D].copy_(self.tok_blk)
        self.bits_full[:, lo // self.D].copy_(self.bits_blk)

    def mask_bits_host(self) -> np.ndarray:
        return self.bits_blk.cpu().numpy().view(np.uint64)

    def tokens_host(self) -> np.ndarray:
        self._sync_block()
        return self.tok_full.cpu().numpy()

    # ------------------------------------------------------------ steps
    def _decide(self, h_src, row_idx, tau):
        W = self.W
        ops.bd_lmhead_confidence(h_src, row_idx, W["Wlm"], self.argmax.view(-1), self.conf.view(-1),
                                 max_logit=self.max_logit.view(-1), lse=self.lse.view(-1))
        ops.bd_threshold_unmask(self.conf, self.argmax, self.tok_blk, self.bits_blk, win_lo=0, threshold=tau,
                                n_unmasked=self.n_unmasked, unmasked_pos=self.unmasked_pos)

    def exact_step(self, tau: float, refresh: bool = True):
        """Full forward pass over the whole sequence; with ``refresh`` its K/V
        outside the block refill the DualCache and its row before the block
        becomes the carry."""
        B, D, T, hid, W = self.B, self.D, self.T, self.hidden, self.W
        Hq, Hkv, d = self.Hq, self.Hkv, self.d
        lo = self.P + self.block * D
        hi = lo + D
        M = B * T
        self._sync_block()
        ops.bd_embed_rows(W["E"], self.tok_full.view(-1, D), self.bits_full.view(-1), self.X_full.view(-1, D, hid),
                          row_off=0, n_rows=D)
        ops.bd_qkv_proj(self.X_full, dense(M), W["Wq"], self.q_full, dense(M), W["Wk"], W["Wv"], self.k_full,
                        dense(M), self.v_full, dense(M), M=M)
        kf, vf = self.k_full.view(B, T, Hkv, d), self.v_full.view(B, T, Hkv, d)
        ops.bd_block_attn(self.q_full.view(B, T, Hq, d), None, None, self.no_cache, kf, vf,
                          self.o_full.view(B, T, Hq, d), D=T, q_off=0)
        ops.bd_linear(self.o_full, dense(M), W["Wo"], self.H_full, dense(M), M=M, res=self.X_full, rr=dense(M))
        if refresh:
            self.kv_len.zero_()
            ops.bd_kv_append(self.cache_k, self.cache_v, self.kv_len, kf, vf, n_rows=lo,
                             kv_len_host=np.zeros(B, np.int32))
            ops.bd_kv_append(self.cache_k, self.cache_v, self.kv_len, kf, vf, n_rows=T - hi, row_off=hi,
                             kv_len_host=np.full(B, lo, np.int32))
            self.Hb[:, 0].copy_(self.H_full[:, lo - 1])
        self._decide(self.H_full.view(-1, hid), self.rows_exact, tau)

    def dual_step(self, tau: float):
        """Only the block's D rows, over the DualCache and the fresh block."""
        B, D, hid, W = self.B, self.D, self.hidden, self.W
        Hq, Hkv, d = self.Hq, self.Hkv, self.d
        M = B * D
        ops.bd_embed_rows(W["E"], self.tok_blk, self.bits_blk, self.Xb, row_off=0, n_rows=D)
        ops.bd_qkv_proj(self.Xb, dense(M), W["Wq"], self.qb, dense(M), W["Wk"], W["Wv"], self.kb, dense(M),
                        self.vb, dense(M), M=M)
        ops.bd_block_attn(self.qb.view(B, D, Hq, d), self.cache_k, self.cache_v, self.kv_len,
                          self.kb.view(B, D, Hkv, d), self.vb.view(B, D, Hkv, d), self.ob.view(B, D, Hq, d),
                          D=D, q_off=0)
        ops.bd_linear(self.ob, dense(M), W["Wo"], self.Hb, rows(D, 1 + D, 1), M=M, res=self.Xb, rr=dense(M))
        self._decide(self.Hb.view(-1, hid), self.rows_dual, tau)

    # ------------------------------------------------------------ loop
    def generate(self, prompts, tau: float, mode: str = "dual", on_step=None) -> tuple:
        """Decode the whole generation region; returns (generated tokens
        [B, gen_len], number of steps)."""
        self.set_prompts(prompts)
        n_blocks = (self.T - self.P) // self.D
        steps = 0
        for k in range(n_blocks):
            self.begin_block(k)
            first = True
            while self.mask_bits_host().any():
                if first or mode == "exact":
                    self.exact_step(tau, refresh=True)
                    kind = "E"
                else:
                    self.dual_step(tau)
                    kind = "DC"
                if on_step is not None:
                    on_step(k, kind)
                first = False
                steps += 1
        return self.tokens_host()[:, self.P:], steps
