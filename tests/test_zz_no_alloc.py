"""bd_block_attn_noalloc (split-key partials in the library's static device
buffer) against bd_block_attn (caller workspace) through the C ABI: two calls
in a row on the same GPU, the second smaller, each bit-identical to the
workspace entry point, which the attention parity tests compare with the
oracle.  Also: a problem larger than the buffer is refused before launch."""
import ctypes

import numpy as np
import pytest
import torch

import bd_inputs as bi
from gpu_util import DEV, TOL, down, rows_close, say, up
from oracle import refine as R

pytestmark = pytest.mark.gpu


def _lib():
    from block_diffusion_decoding_amd import _lib as L
    return L


def _case(seed, B, n_q, q_off, lens, Hq=28, Hkv=4, d=128):
    lens = np.asarray(lens, np.int32)
    cap = int(lens.max() + 64)
    T = torch.bfloat16
    t = dict(q=up(bi.normal(seed, "q", (B, n_q, Hq, d), 0.02, "bf16"), T),
             kc=up(bi.normal(seed, "cache_k", (B, Hkv, cap, d), 0.02, "bf16"), T),
             vc=up(bi.normal(seed, "cache_v", (B, Hkv, cap, d), 0.02, "bf16"), T),
             kb=up(bi.normal(seed, "blk_k", (B, 32, Hkv, d), 0.02, "bf16"), T),
             vb=up(bi.normal(seed, "blk_v", (B, 32, Hkv, d), 0.02, "bf16"), T),
             lens=up(lens))
    return t, dict(B=B, Hq=Hq, Hkv=Hkv, d=d, n_q=n_q, q_off=q_off, cap=cap)


def _call(lib, fn, t, c, o, lse, ws=None):
    s = torch.cuda.current_stream().cuda_stream
    args = [1, c["B"], c["Hq"], c["Hkv"], c["d"], 32, t["q"].data_ptr(), c["n_q"], c["q_off"], t["kc"].data_ptr(),
            t["vc"].data_ptr(), t["lens"].data_ptr(), c["cap"], t["kb"].data_ptr(), t["vb"].data_ptr(), 32,
            c["d"] ** -0.5, o.data_ptr(), lse.data_ptr()]
    if ws is not None:
        args += [ws.data_ptr(), ws.numel()]
    return getattr(lib, fn)(*args, s)


def test_noalloc_equals_workspace_entry_point_twice_then_refuses_oversize():
    L = _lib()
    lib = L.load()
    cap_bytes = lib.bd_block_attn_noalloc_scratch_bytes()
    assert cap_bytes == 32 << 20
    # 1) the 7B workload's exact step (8 ragged sequences, 32 rows x 28 heads): ~29 MB of partials
    # 2) a smaller DualCache step (3 sequences, 8 rows) into the same buffer afterwards
    cases = [(5, 8, 32, 0, (np.random.default_rng(7).integers(32, 129, size=8) * 32)),
             (6, 3, 8, 16, [1000, 77, 4097])]
    for seed, B, n_q, q_off, lens in cases:
        t, c = _case(seed, B, n_q, q_off, lens)
        need = lib.bd_block_attn_workspace_size(1, B, c["Hq"], c["Hkv"], c["d"], n_q, c["cap"], 32)
        say(f"[noalloc] B={B} n_q={n_q} lens={list(lens)} partials {need} bytes")
        assert 0 < need <= cap_bytes
        o_ws = torch.zeros(B, n_q, c["Hq"], c["d"], dtype=torch.bfloat16, device=DEV)
        l_ws = torch.zeros(B, c["Hq"], n_q, dtype=torch.float32, device=DEV)
        o_na, l_na = torch.full_like(o_ws, 7.0), torch.full_like(l_ws, 7.0)
        ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
        assert _call(lib, "bd_block_attn", t, c, o_ws, l_ws, ws) == L.BD_OK
        assert _call(lib, "bd_block_attn_noalloc", t, c, o_na, l_na) == L.BD_OK
        torch.cuda.synchronize()
        assert torch.equal(o_na, o_ws) and torch.equal(l_na, l_ws)
        # and against the oracle on two sequences, at the parity tolerance
        bs = [0, B - 1]
        ro, _ = R.block_attn(down(t["q"])[bs], down(t["kc"])[bs], down(t["vc"])[bs], np.asarray(lens)[bs],
                             down(t["kb"])[bs], down(t["vb"])[bs], q_off, 32)
        rows_close(down(o_na)[bs], ro, TOL["bf16"], "noalloc vs oracle")
    # one sequence, an 8-block prefill over 4096 cached rows: needs more than the buffer; refused, nothing written
    t, c = _case(7, 1, 256, 0, [4096])
    need = lib.bd_block_attn_workspace_size(1, 1, 28, 4, 128, 256, c["cap"], 256)
    assert need > cap_bytes
    o = torch.full((1, 256, 28, 128), 3.0, dtype=torch.bfloat16, device=DEV)
    lse = torch.zeros(1, 28, 256, dtype=torch.float32, device=DEV)
    kb = torch.zeros(1, 256, 4, 128, dtype=torch.bfloat16, device=DEV)
    s = torch.cuda.current_stream().cuda_stream
    st = lib.bd_block_attn_noalloc(1, 1, 28, 4, 128, 32, t["q"].data_ptr(), 256, 0, t["kc"].data_ptr(),
                                   t["vc"].data_ptr(), t["lens"].data_ptr(), c["cap"], kb.data_ptr(), kb.data_ptr(),
                                   256, 128 ** -0.5, o.data_ptr(), lse.data_ptr(), s)
    torch.cuda.synchronize()
    assert st == L.BD_ESCRATCH
    assert bool((o == 3.0).all())
