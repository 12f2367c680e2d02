"""Training form of block diffusion on one GPU: the forward pass and the loss
value of the one-layer model over the 2L layout ("Fast-dLLM v2: Efficient
Block-Diffusion LLM" notes, Key design 2).  Training itself (gradients,
optimiser, data) is not part of this package.

A batch of S samples x0 [S, L] with masks m [S, L]: every sample enters as
two views, masked by m and by its complement, so 2S sequences of 2L rows
[x_t | x_0] are embedded (x_t: masked positions take the [MASK] row),
projected, attended under the 2L hybrid mask (bd_train_attn), projected
back with the residual, and the masked positions' cross-entropies are taken
from the token-shift source rows: noisy row i - 1 inside a block, clean row
i - 1 at a block start (the row that is the carry at inference); position 0
is not supervised.  Every arithmetic step is a libbd call; the host only
lists the supervised positions (integer bookkeeping of the input masks).

Device buffers (M = 2S * 2L rows, view v of sample s is sequence 2s + v):
  X, H [M, hidden]           input rows, output rows
  q, o [M, Hq*d]; k, v [M, Hkv*d]
"""
from __future__ import annotations

import numpy as np
import torch

from . import ops
from .ops import dense


class TrainForward:
    """weights: {"E": [V+1, hid], "Wq", "Wk", "Wv", "Wo", "Wlm"} (out x in)."""

    def __init__(self, weights: dict, Hq: int, Hkv: int, d: int, D: int = 32, dtype=torch.bfloat16,
                 device="cuda"):
        t = lambda a: torch.as_tensor(a).to(device, dtype).contiguous()
        self.W = {k: t(weights[k]) for k in ("E", "Wq", "Wk", "Wv", "Wo", "Wlm")}
        self.Hq, self.Hkv, self.d, self.D = Hq, Hkv, d, D
        self.dtype, self.device = dtype, torch.device(device)
        self.V, self.hidden = self.W["Wlm"].shape
        self._bufs = {}

    def _buf(self, name, shape, dtype):
        b = self._bufs.get(name)
        if b is None or b.shape != torch.Size(shape) or b.dtype != dtype:
            b = torch.empty(shape, dtype=dtype, device=self.device)
            self._bufs[name] = b
        return b

    # ----------------------------------------------------------- host lists
    def plan(self, x0, m):
        """Per-view token and mask-bit arrays of the embedding call and the
        supervised positions: (tokens [2S*2L/D, D], mask_bits, row_idx,
        target, pos) where row m of row_idx/target is position pos[m] =
        (view sequence, i)."""
        x0 = np.asarray(x0, dtype=np.int32)
        m = np.asarray(m, dtype=bool)
        S, L = x0.shape
        D = self.D
        assert L % D == 0 and D <= 64
        nb = L // D
        views = np.stack([m, ~m], axis=1).reshape(2 * S, L)          # sequence 2s + v
        toks = np.repeat(x0, 2, axis=0)                              # [2S, L]
        tokens = np.stack([toks, toks], axis=1).reshape(2 * S * 2 * nb, D)   # (seq, half, block) entries
        bits = np.zeros((2 * S, 2, nb), dtype=np.uint64)
        wb = (views.reshape(2 * S, nb, D).astype(np.uint64) << np.arange(D, dtype=np.uint64)).sum(axis=2)
        bits[:, 0] = wb                                              # the clean half has no masked position
        seq, i = np.nonzero(views)
        keep = i >= 1
        seq, i = seq[keep], i[keep]
        src = np.where(i % D != 0, i - 1, L + i - 1)
        row_idx = (seq * 2 * L + src).astype(np.int32)
        target = toks[seq, i].astype(np.int32)
        return tokens, bits.reshape(-1).view(np.int64), row_idx, target, np.stack([seq, i], axis=1)

    # -------------------------------------------------------------- forward
    def forward(self, x0, m, plan=None):
        """Runs the forward pass and the loss; returns a dict of device
        tensors: loss_sum [1] fp32, nll [n] fp32 (per supervised position, in
        the order of ``pos``), lse [n], and the host arrays pos and count."""
        x0 = np.asarray(x0)
        S, L = x0.shape
        tokens, bits, row_idx, target, pos = self.plan(x0, m) if plan is None else plan
        dev, dt = self.device, self.dtype
        Hq, Hkv, d, D, hid = self.Hq, self.Hkv, self.d, self.D, self.hidden
        M = 2 * S * 2 * L
        n = len(row_idx)
        tok = self._buf("tokens", tokens.shape, torch.int32)
        tok.copy_(torch.from_numpy(tokens))
        mb = self._buf("bits", bits.shape, torch.int64)
        mb.copy_(torch.from_numpy(bits))
        ri = self._buf("row_idx", (n,), torch.int32)
        ri.copy_(torch.from_numpy(row_idx))
        tg = self._buf("target", (n,), torch.int32)
        tg.copy_(torch.from_numpy(target))
        X = self._buf("X", (M, hid), dt)
        q = self._buf("q", (M, Hq * d), dt)
        k = self._buf("k", (M, Hkv * d), dt)
        v = self._buf("v", (M, Hkv * d), dt)
        o = self._buf("o", (M, Hq * d), dt)
        H = self._buf("H", (M, hid), dt)
        am = self._buf("argmax", (n,), torch.int32)
        cf = self._buf("conf", (n,), torch.float32)
        lse = self._buf("lse", (n,), torch.float32)
        nll = self._buf("nll", (n,), torch.float32)
        loss = self._buf("loss", (1,), torch.float32)
        W = self.W
        ops.bd_embed_rows(W["E"], tok, mb, X.view(-1, D, hid), row_off=0, n_rows=D)
        ops.bd_qkv_proj(X, dense(M), W["Wq"], q, dense(M), W["Wk"], W["Wv"], k, dense(M), v, dense(M), M=M)
        ops.bd_train_attn(q.view(2 * S, 2 * L, Hq, d), k.view(2 * S, 2 * L, Hkv, d), v.view(2 * S, 2 * L, Hkv, d),
                          o.view(2 * S, 2 * L, Hq, d), L=L, D=D)
        ops.bd_linear(o, dense(M), W["Wo"], H, dense(M), M=M, res=X, rr=dense(M))
        ops.bd_lmhead_confidence(H, ri, W["Wlm"], am, cf, lse=lse)
        ops.bd_masked_nll(H, ri, W["Wlm"], tg, lse, nll, loss, M=n)
        return {"loss_sum": loss, "nll": nll, "lse": lse, "pos": pos, "count": n, "H": H, "o": o}
