"""Python binding of libbd: one function per C-ABI call, same names.

Argument marshalling only: tensors supply device pointers, the current torch
stream supplies the HIP stream, and every step runs in the library's HIP
kernels.  A non-OK status raises ``BdError``.  Shapes follow include/bd.h.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import BdRows

_DT = {torch.float32: _lib.BD_F32, torch.bfloat16: _lib.BD_BF16}


class BdError(RuntimeError):
    def __init__(self, name: str, status: int):
        lib = _lib.load()
        msg = lib.bd_status_string(status).decode()
        extra = f" (hipError {lib.bd_last_hip_error()})" if status == _lib.BD_EHIP else ""
        super().__init__(f"{name}: {msg}{extra}")
        self.status = status


def _check(name, status):
    if status != _lib.BD_OK:
        raise BdError(name, status)


def _p(t):
    """Device pointer of a tensor (or 0 for None); tensors must be contiguous."""
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("libbd tensors must be contiguous")
    return t.data_ptr()


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _dt(t):
    if t.dtype not in _DT:
        raise ValueError(f"unsupported dtype {t.dtype}")
    return _DT[t.dtype]


def rows(group: int, stride: int, offset: int = 0) -> BdRows:
    return BdRows(int(group), int(stride), int(offset))


def dense(n: int) -> BdRows:
    return BdRows(int(n), int(n), 0)


_workspaces: dict = {}


def workspace(nbytes: int, device, tag: str = "") -> torch.Tensor:
    """A cached zero-initialised workspace per (device, tag), grown on demand."""
    key = (str(device), tag)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


# ---------------------------------------------------------------------------
def bd_block_attn_workspace_size(dtype, B, Hq, Hkv, d, n_q, cap, n_blk) -> int:
    return int(_lib.load().bd_block_attn_workspace_size(_DT[dtype], B, Hq, Hkv, d, n_q, cap, n_blk))


def _guard(guard):
    """(bits [n] int64 tensor, mask, n) -> a BdGuard the call reads (None: no guard)."""
    if guard is None:
        return None
    bits, mask, n = guard
    return ctypes.byref(_lib.BdGuard(_p(bits), ctypes.c_uint64(int(mask) & (2 ** 64 - 1)), int(n)))


def bd_block_attn(q, k_cache, v_cache, kv_len, k_blk, v_blk, o, *, D, q_off=0, scale=None, lse=None,
                  ws=None, stream=None, guard=None):
    """q [B, n_q, Hq, d]; k/v_cache [B, Hkv, cap, d]; kv_len [B] int32; k/v_blk [B, n_blk, Hkv, d];
    o [B, n_q, Hq, d]; lse [B, Hq, n_q] fp32 or None.  guard: (bits, mask, n) or None
    (bd_block_attn_guarded: nothing is done when no bits[b] has a bit of mask set)."""
    lib = _lib.load()
    B, n_q, Hq, d = q.shape
    if k_cache is None:         # no cache rows: only the in-block keys
        Hkv, cap = k_blk.shape[2], 0
    else:
        _, Hkv, cap, _ = k_cache.shape
    n_blk = k_blk.shape[1]
    if scale is None:
        scale = d ** -0.5
    dt = _dt(q)
    need = lib.bd_block_attn_workspace_size(dt, B, Hq, Hkv, d, n_q, cap, n_blk)
    if ws is None:
        ws = workspace(need, q.device, "attn")
    args = (dt, B, Hq, Hkv, d, D, _p(q), n_q, q_off, _p(k_cache), _p(v_cache), _p(kv_len), cap,
            _p(k_blk), _p(v_blk), n_blk, float(scale), _p(o), _p(lse), _p(ws), ws.numel())
    if guard is None:
        _check("bd_block_attn", lib.bd_block_attn(*args, _stream(stream)))
    else:
        _check("bd_block_attn_guarded", lib.bd_block_attn_guarded(*args, _guard(guard), _stream(stream)))
    return o


def bd_block_attn_noalloc(q, k_cache, v_cache, kv_len, k_blk, v_blk, o, *, D, q_off=0, scale=None, lse=None,
                          stream=None):
    """bd_block_attn with its partials in the library's static device buffer
    (no workspace; nothing allocated); same tensors as bd_block_attn."""
    lib = _lib.load()
    B, n_q, Hq, d = q.shape
    if k_cache is None:
        Hkv, cap = k_blk.shape[2], 0
    else:
        _, Hkv, cap, _ = k_cache.shape
    if scale is None:
        scale = d ** -0.5
    st = lib.bd_block_attn_noalloc(_dt(q), B, Hq, Hkv, d, D, _p(q), n_q, q_off, _p(k_cache), _p(v_cache),
                                   _p(kv_len), cap, _p(k_blk), _p(v_blk), k_blk.shape[1], float(scale), _p(o),
                                   _p(lse), _stream(stream))
    _check("bd_block_attn_noalloc", st)
    return o


def bd_lmhead_workspace_size(dtype, M, hidden, V) -> int:
    return int(_lib.load().bd_lmhead_workspace_size(_DT[dtype], M, hidden, V))


def bd_lmhead_confidence(h_src, row_idx, w, argmax, conf, *, max_logit=None, lse=None, logits=None, M=None,
                         ws=None, stream=None):
    """h_src [n_src, hidden]; row_idx [M] int32 or None; w [V, hidden]; argmax [M] int32; conf [M] fp32."""
    lib = _lib.load()
    hidden = h_src.shape[-1]
    n_src = h_src.numel() // hidden
    V = w.shape[0]
    if M is None:
        M = row_idx.numel() if row_idx is not None else n_src
    dt = _dt(h_src)
    need = lib.bd_lmhead_workspace_size(dt, M, hidden, V)
    if ws is None:
        ws = workspace(need, h_src.device, "lm")
    st = lib.bd_lmhead_confidence(dt, M, hidden, V, _p(h_src), n_src, _p(row_idx), _p(w), _p(argmax), _p(conf),
                                  _p(max_logit), _p(lse), _p(logits), _p(ws), ws.numel(), _stream(stream))
    _check("bd_lmhead_confidence", st)


def bd_lmhead_confidence_rows(h_src, row_idx, out_pos, m_dev, w, argmax, conf, *, max_logit=None, lse=None,
                              logits=None, ws=None, stream=None):
    """Rows m < m_dev[0] of row_idx/out_pos (capacity M = row_idx.numel());
    results of row m land at out_pos[m] of argmax/conf (and max_logit/lse)."""
    lib = _lib.load()
    hidden = h_src.shape[-1]
    n_src = h_src.numel() // hidden
    V = w.shape[0]
    M = row_idx.numel()
    dt = _dt(h_src)
    need = lib.bd_lmhead_workspace_size(dt, M, hidden, V)
    if ws is None:
        ws = workspace(need, h_src.device, "lm")
    st = lib.bd_lmhead_confidence_rows(dt, M, hidden, V, _p(h_src), n_src, _p(row_idx), _p(out_pos), _p(m_dev),
                                       conf.numel(), _p(w), _p(argmax), _p(conf), _p(max_logit), _p(lse),
                                       _p(logits), _p(ws), ws.numel(), _stream(stream))
    _check("bd_lmhead_confidence_rows", st)


def bd_lmhead_unmask(h_src, row_idx, w, argmax, conf, tokens, mask_bits, *, win_lo, threshold, max_logit=None,
                     lse=None, n_unmasked=None, unmasked_pos=None, mask_bits_host=None, next_rows=None, ws=None,
                     stream=None):
    """LM head with fused confidence and the threshold unmask in one call:
    argmax/conf [B, win_len] (row b * win_len + r predicts position
    win_lo + r); tokens [B, D] int32, mask_bits [B] (64-bit) in/out;
    threshold a float or a [B] fp32 device tensor; mask_bits_host an
    optional pinned host tensor [B] (64-bit) that receives the new bits;
    next_rows = (E [V+1, hidden], plant [B, D, hidden] or None, x [B, D,
    hidden]): the rows of the positions decoded here are rewritten in x
    (bd_lmhead_unmask_next)."""
    lib = _lib.load()
    hidden = h_src.shape[-1]
    n_src = h_src.numel() // hidden
    V = w.shape[0]
    B, win_len = conf.shape
    D = tokens.shape[1]
    dt = _dt(h_src)
    if mask_bits_host is not None:
        assert mask_bits_host.device.type == "cpu" and mask_bits_host.is_pinned() and mask_bits_host.numel() == B
    tau_dev = None
    if isinstance(threshold, torch.Tensor):
        assert threshold.dtype == torch.float32 and threshold.numel() == B
        tau_dev, threshold = threshold, 0.0
    need = lib.bd_lmhead_workspace_size(dt, B * win_len, hidden, V)
    if ws is None:
        ws = workspace(need, h_src.device, "lm")
    if next_rows is None:
        st = lib.bd_lmhead_unmask(dt, B, D, win_lo, win_len, hidden, V, _p(h_src), n_src, _p(row_idx), _p(w),
                                  float(threshold), _p(tau_dev), _p(argmax), _p(conf), _p(max_logit), _p(lse),
                                  _p(tokens), _p(mask_bits), _p(n_unmasked), _p(unmasked_pos), _p(mask_bits_host),
                                  _p(ws), ws.numel(), _stream(stream))
        _check("bd_lmhead_unmask", st)
        return
    E, plant, x = next_rows
    assert E.dtype == x.dtype == w.dtype and E.shape == (V + 1, hidden) and x.shape == (B, D, hidden)
    assert plant is None or (plant.dtype == x.dtype and plant.shape == x.shape)
    nr = _lib.BdNextRows(_p(E), _p(plant), _p(x))
    st = lib.bd_lmhead_unmask_next(dt, B, D, win_lo, win_len, hidden, V, _p(h_src), n_src, _p(row_idx), _p(w),
                                   float(threshold), _p(tau_dev), _p(argmax), _p(conf), _p(max_logit), _p(lse),
                                   _p(tokens), _p(mask_bits), _p(n_unmasked), _p(unmasked_pos), _p(mask_bits_host),
                                   ctypes.byref(nr), _p(ws), ws.numel(), _stream(stream))
    _check("bd_lmhead_unmask_next", st)


def bd_candidate_rows(mask_bits, row_idx, out_pos, count, *, win_lo, win_len, rows_per_seq, stream=None):
    """mask_bits [B] (64-bit); row_idx/out_pos [B*win_len] int32; count [1] int32."""
    lib = _lib.load()
    B = mask_bits.numel()
    st = lib.bd_candidate_rows(B, win_lo, win_len, _p(mask_bits), rows_per_seq, _p(row_idx), _p(out_pos),
                               _p(count), _stream(stream))
    _check("bd_candidate_rows", st)


def bd_threshold_unmask(conf, argmax, tokens, mask_bits, *, win_lo, threshold, n_unmasked=None,
                        unmasked_pos=None, stream=None):
    """conf/argmax [B, win_len]; tokens [B, D] int32; mask_bits [B] (64-bit);
    threshold: a float, or a [B] fp32 device tensor read when the kernel runs."""
    lib = _lib.load()
    B, win_len = conf.shape
    D = tokens.shape[1]
    if isinstance(threshold, torch.Tensor):
        assert threshold.dtype == torch.float32 and threshold.numel() == B
        st = lib.bd_threshold_unmask_tau(B, D, win_lo, win_len, _p(conf), _p(argmax), _p(threshold), _p(tokens),
                                         _p(mask_bits), _p(n_unmasked), _p(unmasked_pos), _stream(stream))
        _check("bd_threshold_unmask_tau", st)
        return
    st = lib.bd_threshold_unmask(B, D, win_lo, win_len, _p(conf), _p(argmax), float(threshold), _p(tokens),
                                 _p(mask_bits), _p(n_unmasked), _p(unmasked_pos), _stream(stream))
    _check("bd_threshold_unmask", st)


def bd_threshold_unmask_windows(conf, argmax, tokens, mask_bits, win_lo, *, threshold, n_unmasked=None,
                                unmasked_pos=None, stream=None):
    """conf/argmax [B, win_len]; win_lo [B] int32 device: each sequence's window start."""
    lib = _lib.load()
    B, win_len = conf.shape
    D = tokens.shape[1]
    st = lib.bd_threshold_unmask_windows(B, D, win_len, _p(win_lo), _p(conf), _p(argmax), float(threshold),
                                         _p(tokens), _p(mask_bits), _p(n_unmasked), _p(unmasked_pos),
                                         _stream(stream))
    _check("bd_threshold_unmask_windows", st)


def bd_copy_rows(row_mask, src0, dst0, src1=None, dst1=None, *, stream=None):
    """src/dst [B, n_rows, ...] contiguous, same shape; row_mask [B] (64-bit) device."""
    lib = _lib.load()
    B, n_rows = src0.shape[0], src0.shape[1]
    row_bytes = src0[0, 0].numel() * src0.element_size()
    assert dst0.shape == src0.shape and (src1 is None or (src1.shape == src0.shape and dst1.shape == src0.shape))
    st = lib.bd_copy_rows(B, n_rows, row_bytes, _p(row_mask), _p(src0), _p(dst0), _p(src1), _p(dst1),
                          _stream(stream))
    _check("bd_copy_rows", st)


def bd_probe_weight_stream(w, x=None, *, work_groups, stream=None):
    """Measurement support: the streaming LM head's load pattern over w
    [rows, K] (and the 64 rows of x [64, K] when given), no arithmetic."""
    lib = _lib.load()
    rows, row_bytes = w.shape[0], w.shape[1] * w.element_size()
    if x is not None:
        assert x.shape[0] >= 64 and x.shape[1] * x.element_size() == row_bytes
    st = lib.bd_probe_weight_stream(_p(w), rows, row_bytes, _p(x), 0 if x is None else 4, int(work_groups),
                                    _stream(stream))
    _check("bd_probe_weight_stream", st)


def bd_persequence_schedule(mask_bits, state, restore, save, save_h, row_idx, win_lo, *, D, S, kinds=None,
                            live=None, stream=None):
    """mask_bits [B] (64-bit) device; state [3, B] int32 device (win, opening,
    ran); restore/save/save_h [B] 64-bit; row_idx [B * S] int32; win_lo [B]
    int32; kinds [B] int32 or None; live [1] int32 or None."""
    lib = _lib.load()
    B = mask_bits.shape[0]
    assert state.shape == (3, B) and state.dtype == torch.int32 and state.is_contiguous()
    assert row_idx.numel() == B * S and win_lo.numel() == B
    st = lib.bd_persequence_schedule(B, D, S, _p(mask_bits), _p(state[0]), _p(state[1]), _p(state[2]),
                                     _p(restore), _p(save), _p(save_h), _p(row_idx), _p(win_lo), _p(kinds),
                                     _p(live), _stream(stream))
    _check("bd_persequence_schedule", st)


def bd_kv_append(k_cache, v_cache, kv_len, k_blk, v_blk, *, n_rows, kv_len_host=None, row_off=0, stream=None):
    """k/v_cache [B, Hkv, cap, d]; kv_len [B] int32 (in/out); k/v_blk [B, n_blk, Hkv, d];
    appends rows row_off .. row_off + n_rows - 1 of each sequence's k/v_blk."""
    lib = _lib.load()
    B, Hkv, cap, d = k_cache.shape
    n_blk = k_blk.shape[1]
    assert 0 <= row_off and row_off + n_rows <= n_blk
    host = None
    if kv_len_host is not None:
        import numpy as np
        host = np.ascontiguousarray(kv_len_host, dtype=np.int32)
    off = row_off * Hkv * d * k_blk.element_size()
    kp, vp = _p(k_blk), _p(v_blk)
    st = lib.bd_kv_append(_dt(k_cache), B, Hkv, d, cap, _p(k_cache), _p(v_cache), _p(kv_len),
                          None if host is None else host.ctypes.data, kp + off, vp + off, n_blk,
                          n_rows, _stream(stream))
    _check("bd_kv_append", st)


def bd_embed_rows(E, tokens, mask_bits, x, *, row_off, n_rows, plant=None, stream=None):
    """E [V+1, hidden]; tokens [B, D] int32; mask_bits [B] or None; x [B, n_rows, hidden]."""
    lib = _lib.load()
    B, D = tokens.shape
    V = E.shape[0] - 1
    st = lib.bd_embed_rows(_dt(E), B, D, row_off, n_rows, E.shape[1], V, _p(E), _p(tokens), _p(mask_bits),
                           _p(plant), _p(x), _stream(stream))
    _check("bd_embed_rows", st)


def bd_linear_workspace_size(dtype, M, N, K) -> int:
    return int(_lib.load().bd_linear_workspace_size(_DT[dtype], M, N, K))


def bd_qkv_proj_workspace_size(dtype, M, K, Nq, Nkv) -> int:
    return int(_lib.load().bd_qkv_proj_workspace_size(_DT[dtype], M, K, Nq, Nkv))


def bd_linear(x, xr, w, y, yr, *, M, res=None, rr=None, ws=None, stream=None, guard=None):
    """y[yr(m)] = x[xr(m)] w^T (+ res[rr(m)]); w [N, K].  guard: as bd_block_attn."""
    lib = _lib.load()
    N, K = w.shape
    dt = _dt(w)
    if ws is None:
        ws = workspace(lib.bd_linear_workspace_size(dt, M, N, K), w.device, "gemm")
    args = (dt, M, N, K, _p(x), xr, _p(w), _p(res), rr if rr is not None else dense(1), _p(y), yr,
            _p(ws), ws.numel())
    if guard is None:
        _check("bd_linear", lib.bd_linear(*args, _stream(stream)))
    else:
        _check("bd_linear_guarded", lib.bd_linear_guarded(*args, _guard(guard), _stream(stream)))


def bd_linear_residual_rmsnorm(x, xr, w, y, yr, h, hr, *, M, eps, ws=None, stream=None):
    """y[yr(m)] += x[xr(m)] w^T, then h[hr(m)] = rmsnorm(y[yr(m)]) (unit gains)."""
    lib = _lib.load()
    N, K = w.shape
    dt = _dt(w)
    if ws is None:
        ws = workspace(lib.bd_linear_workspace_size(dt, M, N, K), w.device, "gemm")
    st = lib.bd_linear_residual_rmsnorm(dt, M, N, K, _p(x), xr, _p(w), _p(y), yr, float(eps), _p(h), hr, _p(ws),
                                        ws.numel(), _stream(stream))
    _check("bd_linear_residual_rmsnorm", st)


def bd_qkv_proj(x, xr, wq, q, qr, wk, wv, k, kr, v, vr, *, M, ws=None, stream=None, guard=None):
    """q[qr(m)] = x[xr(m)] wq^T, k[kr(m)] = x[xr(m)] wk^T, v[vr(m)] = x[xr(m)] wv^T.  guard: as
    bd_block_attn."""
    lib = _lib.load()
    Nq, K = wq.shape
    Nkv = wk.shape[0]
    dt = _dt(wq)
    if ws is None:
        ws = workspace(lib.bd_qkv_proj_workspace_size(dt, M, K, Nq, Nkv), wq.device, "gemm")
    args = (dt, M, K, _p(x), xr, _p(wq), Nq, _p(q), qr, _p(wk), _p(wv), Nkv, _p(k), kr, _p(v),
            vr, _p(ws), ws.numel())
    if guard is None:
        _check("bd_qkv_proj", lib.bd_qkv_proj(*args, _stream(stream)))
    else:
        _check("bd_qkv_proj_guarded", lib.bd_qkv_proj_guarded(*args, _guard(guard), _stream(stream)))


def bd_qkv_proj_rope_workspace_size(dtype, M, K, Nq, Nkv) -> int:
    return int(_lib.load().bd_qkv_proj_rope_workspace_size(_DT[dtype], M, K, Nq, Nkv))


def bd_qkv_proj_rope(x, xr, wq, q, qr, wk, wv, k, kr, v, vr, pos_base, *, M, d, n_rows, pos_off=0, theta,
                     ws=None, stream=None):
    """bd_qkv_proj, then q and k rotated at positions pos_base[m // n_rows] +
    pos_off + m % n_rows (heads of d elements)."""
    lib = _lib.load()
    Nq, K = wq.shape
    Nkv = wk.shape[0]
    dt = _dt(wq)
    if ws is None:
        ws = workspace(lib.bd_qkv_proj_rope_workspace_size(dt, M, K, Nq, Nkv), wq.device, "gemm")
    st = lib.bd_qkv_proj_rope(dt, M, K, _p(x), xr, _p(wq), Nq, _p(q), qr, _p(wk), _p(wv), Nkv, _p(k), kr, _p(v),
                              vr, int(d), _p(pos_base), int(n_rows), int(pos_off), float(theta), _p(ws), ws.numel(),
                              _stream(stream))
    _check("bd_qkv_proj_rope", st)


def bd_gate_up_swiglu(x, xr, w_gu, a, ar, *, M, stream=None):
    """a[ar(m)] = silu(x[xr(m)] Wg^T) * (x[xr(m)] Wu^T) with w_gu = [Wg; Wu]
    ([2*inter, K])."""
    inter2, K = w_gu.shape
    st = _lib.load().bd_gate_up_swiglu(_dt(w_gu), M, K, _p(x), xr, _p(w_gu), inter2 // 2, _p(a), ar,
                                       _stream(stream))
    _check("bd_gate_up_swiglu", st)


def bd_gate_up_swiglu_rmsnorm(x, xr, w_gu, a, ar, *, M, eps, stream=None):
    """bd_gate_up_swiglu on rmsnorm(x[xr(m)]) (unit gains), the norm folded
    into the projection's kernels."""
    inter2, K = w_gu.shape
    st = _lib.load().bd_gate_up_swiglu_rmsnorm(_dt(w_gu), M, K, _p(x), xr, float(eps), _p(w_gu), inter2 // 2, _p(a),
                                               ar, _stream(stream))
    _check("bd_gate_up_swiglu_rmsnorm", st)


def bd_rmsnorm(x, xr, y, yr, *, M, eps, stream=None):
    """y[yr(m)] = rmsnorm(x[xr(m)]) (unit gains); rows of x.shape[-1] elements."""
    st = _lib.load().bd_rmsnorm(_dt(x), M, x.shape[-1], _p(x), xr, float(eps), _p(y), yr, _stream(stream))
    _check("bd_rmsnorm", st)


def bd_rope(x, xr, pos_base, *, n_rows, H, d, pos_off=0, theta, stream=None):
    """Rotary embedding in place on rows xr(b*n_rows + i) of x at positions
    pos_base[b] + pos_off + i; B = pos_base.numel()."""
    st = _lib.load().bd_rope(_dt(x), pos_base.numel(), n_rows, H, d, _p(x), xr, _p(pos_base), int(pos_off),
                             float(theta), _stream(stream))
    _check("bd_rope", st)


def bd_swiglu(gu, gr, a, ar, *, M, inter, stream=None):
    """a[ar(m)] = silu(gate) * up of the row gu[gr(m)] = [gate | up]."""
    st = _lib.load().bd_swiglu(_dt(gu), M, inter, _p(gu), gr, _p(a), ar, _stream(stream))
    _check("bd_swiglu", st)



def bd_train_attn_workspace_size(dtype, S, L, D, Hq, Hkv, d) -> int:
    return int(_lib.load().bd_train_attn_workspace_size(_DT[dtype], S, L, D, Hq, Hkv, d))


def bd_train_attn(q, k, v, o, *, L, D, scale=None, ws=None, stream=None):
    """Attention of the 2L training layout: q [S, 2L, Hq, d], k/v [S, 2L, Hkv, d]
    (rows 0..L-1 noisy, L..2L-1 clean) -> o like q."""
    lib = _lib.load()
    S, L2, Hq, d = q.shape
    Hkv = k.shape[2]
    assert L2 == 2 * L
    dt = _dt(q)
    if ws is None:
        ws = workspace(lib.bd_train_attn_workspace_size(dt, S, L, D, Hq, Hkv, d), q.device, "train")
    sc = d ** -0.5 if scale is None else float(scale)
    st = lib.bd_train_attn(dt, S, L, D, Hq, Hkv, d, _p(q), _p(k), _p(v), sc, _p(o), _p(ws), ws.numel(),
                           _stream(stream))
    _check("bd_train_attn", st)


def bd_masked_nll(h_src, row_idx, w, target, lse, nll, loss_sum=None, *, M, stream=None):
    """nll[m] = lse[m] - h_src[row_idx[m]] . w[target[m]]; loss_sum[0] = sum."""
    V, hidden = w.shape
    n_src = h_src.numel() // hidden
    st = _lib.load().bd_masked_nll(_dt(w), M, hidden, V, _p(h_src), n_src, _p(row_idx), _p(w), _p(target),
                                   _p(lse), _p(nll), _p(loss_sum), _stream(stream))
    _check("bd_masked_nll", st)
