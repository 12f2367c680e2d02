"""CPU checks of the C ABI: the library loads, exports every function that
include/bd.h declares, and rejects bad arguments on the host before any
launch (no GPU is touched by these tests)."""
import ctypes
import os
import re
import subprocess
import sys

import numpy as np
import pytest

from block_diffusion_decoding_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bd.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="libbd.so not built")


def declared_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(bd_[a-z0-9_]+)\s*\(", txt)))


def test_header_declares_the_four_calls_and_support():
    names = declared_functions()
    for n in ["bd_block_attn", "bd_lmhead_confidence", "bd_threshold_unmask", "bd_kv_append",
              "bd_embed_rows", "bd_linear", "bd_qkv_proj", "bd_block_attn_workspace_size",
              "bd_linear_workspace_size", "bd_qkv_proj_workspace_size",
              "bd_lmhead_workspace_size", "bd_status_string", "bd_last_hip_error", "bd_version",
              "bd_qkv_proj_rope", "bd_qkv_proj_rope_workspace_size", "bd_gate_up_swiglu", "bd_gate_up_swiglu_rmsnorm",
              "bd_train_attn", "bd_train_attn_workspace_size", "bd_masked_nll", "bd_threshold_unmask_tau",
              "bd_lmhead_unmask", "bd_threshold_unmask_windows", "bd_copy_rows", "bd_block_attn_noalloc",
              "bd_persequence_schedule", "bd_probe_weight_stream"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    names = declared_functions()
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    assert set(names) <= set(_lib.SIGNATURES), "binding lacks a signature"
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (bd_[a-z0-9_]+)$", out, flags=re.M))
    assert set(names) <= exported


def test_status_strings_and_version():
    lib = _lib.load()
    assert lib.bd_version().startswith(b"libbd")
    for s in range(6):
        assert lib.bd_status_string(s)
    assert lib.bd_last_hip_error() == 0


FAKE = 0x100000  # 16-byte aligned fake device address; never dereferenced


def attn(lib, **kw):
    a = dict(dt=1, B=1, Hq=4, Hkv=2, d=128, D=32, q=FAKE, n_q=8, q_off=8, kc=FAKE, vc=FAKE, kv_len=FAKE,
             cap=64, kb=FAKE, vb=FAKE, n_blk=32, scale=0.1, o=FAKE, lse=None, ws=FAKE, wsb=1 << 30, s=None)
    a.update(kw)
    return lib.bd_block_attn(a["dt"], a["B"], a["Hq"], a["Hkv"], a["d"], a["D"], a["q"], a["n_q"], a["q_off"],
                             a["kc"], a["vc"], a["kv_len"], a["cap"], a["kb"], a["vb"], a["n_blk"], a["scale"],
                             a["o"], a["lse"], a["ws"], a["wsb"], a["s"])


def test_attn_argument_errors():
    lib = _lib.load()
    E, U = _lib.BD_EINVAL, _lib.BD_EUNSUPPORTED
    assert attn(lib, B=0) == 0 and attn(lib, n_q=0) == 0          # empty work: no-op
    assert attn(lib, Hkv=3) == E                                     # Hq % Hkv
    assert attn(lib, q_off=30) == E                                  # q_off + n_q > n_blk
    assert attn(lib, n_blk=48) == E                                  # n_blk % D
    assert attn(lib, D=0) == E
    assert attn(lib, d=96) == U
    assert attn(lib, q=None) == E
    assert attn(lib, q=FAKE + 2) == E                                # misaligned
    assert attn(lib, dt=7) == E
    assert attn(lib, scale=float("nan")) == E
    need = lib.bd_block_attn_workspace_size(1, 32, 28, 4, 128, 8, 16416, 32)
    assert need > 0
    assert attn(lib, B=32, Hq=28, Hkv=4, n_q=8, cap=16416, wsb=need - 1) == E
    assert lib.bd_block_attn_workspace_size(0, 1, 4, 2, 64, 8, 64, 32) == 0   # fp32: no workspace


def test_lmhead_unmask_append_argument_errors():
    lib = _lib.load()
    E, U, C = _lib.BD_EINVAL, _lib.BD_EUNSUPPORTED, _lib.BD_ECAPACITY
    ws = lib.bd_lmhead_workspace_size(1, 64, 3584, 152064)
    assert ws >= 64 * 256 * 12          # one (max, argmax, sum) per row and streaming work-group (one per CU)
    assert lib.bd_lmhead_workspace_size(1, 8, 1536, 151936) >= 8 * 512 * 12  # narrower rows: two per CU
    assert lib.bd_lmhead_workspace_size(1, 1024, 3584, 152064) >= 1024 * 594 * 12  # per row and 256-column block
    lm = lambda **k: lib.bd_lmhead_confidence(k.get("dt", 1), k.get("M", 8), k.get("hidden", 1536), 151936,
                                              FAKE, k.get("n_src", 9), k.get("ri", FAKE), FAKE, FAKE, FAKE,
                                              None, None, None, FAKE, k.get("wsb", 1 << 30), None)
    assert lm(M=0) == 0
    assert lm(hidden=1000) == U
    assert lm(ri=None, n_src=4) == E
    assert lm(wsb=16) == E
    um = lambda **k: lib.bd_threshold_unmask(1, k.get("D", 32), k.get("lo", 8), k.get("wl", 8), FAKE, FAKE,
                                             k.get("t", 0.9), FAKE, FAKE, None, None, None)
    assert um(D=65) == E and um(lo=30) == E and um(wl=0) == E and um(t=float("nan")) == E
    h = np.array([16400, 16384], dtype=np.int32)
    ap = lambda host, n=32, cap=16416: lib.bd_kv_append(1, 2, 4, 128, cap, FAKE, FAKE, FAKE, host,
                                                        FAKE, FAKE, 32, n, None)
    assert ap(h.ctypes.data) == C
    assert ap(None, n=33) == E                                        # n_rows > n_blk
    assert ap(h.ctypes.data, n=0) == 0


def test_candidate_rows_argument_errors():
    lib = _lib.load()
    E = _lib.BD_EINVAL
    cr = lambda **k: lib.bd_candidate_rows(k.get("B", 4), k.get("lo", 8), k.get("wl", 8), k.get("bits", FAKE),
                                           k.get("rps", 33), FAKE, FAKE, FAKE, None)
    assert cr(B=0) == 0
    assert cr(B=-1) == E and cr(wl=0) == E and cr(wl=65) == E and cr(lo=60) == E
    assert cr(rps=15) == E                                            # row of position 15 would not exist
    assert cr(B=513) == E                                             # more than 4096 window entries
    assert cr(bits=None) == E
    lmr = lambda **k: lib.bd_lmhead_confidence_rows(1, 64, 512, 5000, FAKE, 100, k.get("ri", FAKE),
                                                    k.get("pos", FAKE), k.get("mdev", FAKE), 64, FAKE, FAKE, FAKE,
                                                    None, None, None, FAKE, 1 << 30, None)
    assert lmr(mdev=None) == E and lmr(pos=None) == E and lmr(ri=None) == E


def test_gemm_and_embed_argument_errors():
    lib = _lib.load()
    E, U = _lib.BD_EINVAL, _lib.BD_EUNSUPPORTED
    R = _lib.BdRows
    big = 1 << 30
    assert lib.bd_linear(1, 64, 3584, 3584, FAKE, R(64, 64, 0), FAKE, None, R(1, 1, 0), FAKE, R(0, 1, 0),
                         FAKE, big, None) == E                         # group 0
    assert lib.bd_linear(1, 64, 3584, 1000, FAKE, R(64, 64, 0), FAKE, None, R(1, 1, 0), FAKE, R(64, 64, 0),
                         FAKE, big, None) == U                         # K % 256
    assert lib.bd_linear(1, 0, 3584, 3584, FAKE, R(1, 1, 0), FAKE, None, R(1, 1, 0), FAKE, R(1, 1, 0),
                         None, 0, None) == 0
    # a short K with few columns: K split over the waves of a work-group, no workspace
    assert lib.bd_qkv_proj_workspace_size(1, 64, 1536, 1536, 256) == 0
    need = lib.bd_qkv_proj_workspace_size(1, 64, 8960, 1536, 256)
    assert need > 0                                                    # a long K with few columns splits K
    assert lib.bd_qkv_proj(1, 64, 8960, FAKE, R(64, 64, 0), FAKE, 1536, FAKE, R(64, 64, 0), FAKE, FAKE, 256,
                           FAKE, R(8, 32, 8), FAKE, R(8, 32, 8), FAKE, need - 16, None) == E
    # the split writes one fp32 partial sum per slice, row and 16-column tile column
    assert need % (64 * (1536 + 2 * 256) * 4) == 0
    assert lib.bd_linear_workspace_size(1, 128, 17920, 1536) == 0     # enough column tiles: no split
    assert lib.bd_linear_workspace_size(0, 64, 3584, 3584) == 0       # fp32: no workspace
    assert lib.bd_embed_rows(1, 1, 65, 0, 8, 64, 10, FAKE, FAKE, FAKE, None, FAKE, None) == E
    assert lib.bd_embed_rows(1, 1, 32, 30, 8, 64, 10, FAKE, FAKE, FAKE, None, FAKE, None) == E


def noalloc(lib, **kw):
    a = dict(dt=1, B=1, Hq=4, Hkv=2, d=128, D=32, q=FAKE, n_q=8, q_off=8, kc=FAKE, vc=FAKE, kv_len=FAKE,
             cap=64, kb=FAKE, vb=FAKE, n_blk=32, scale=0.1, o=FAKE, lse=None, s=None)
    a.update(kw)
    return lib.bd_block_attn_noalloc(a["dt"], a["B"], a["Hq"], a["Hkv"], a["d"], a["D"], a["q"], a["n_q"],
                                     a["q_off"], a["kc"], a["vc"], a["kv_len"], a["cap"], a["kb"], a["vb"],
                                     a["n_blk"], a["scale"], a["o"], a["lse"], a["s"])


def test_noalloc_attn_argument_errors_and_scratch_limit():
    """The static-scratch attention checks its arguments like bd_block_attn and
    refuses a problem whose partials exceed its buffer, all before any HIP
    call (so no device is needed here)."""
    lib = _lib.load()
    E, U = _lib.BD_EINVAL, _lib.BD_EUNSUPPORTED
    assert lib.bd_block_attn_noalloc_scratch_bytes() == 32 << 20
    assert noalloc(lib, B=0) == 0 and noalloc(lib, n_q=0) == 0
    assert noalloc(lib, Hkv=3) == E
    assert noalloc(lib, q_off=30) == E
    assert noalloc(lib, n_blk=48) == E
    assert noalloc(lib, d=96) == U
    assert noalloc(lib, q=None) == E
    assert noalloc(lib, o=FAKE + 4) == E
    assert noalloc(lib, scale=float("nan")) == E
    # one sequence, an 8-block prefill over 4160 cached rows: its partials do not fit in 32 MiB
    need = lib.bd_block_attn_workspace_size(1, 1, 28, 4, 128, 256, 4160, 256)
    assert need > lib.bd_block_attn_noalloc_scratch_bytes()
    assert noalloc(lib, B=1, Hq=28, Hkv=4, n_q=256, q_off=0, n_blk=256, cap=4160) == _lib.BD_ESCRATCH
    # every refinement step of the long-context workload fits (32 x 16384 rows, exact step)
    assert lib.bd_block_attn_workspace_size(1, 32, 28, 4, 128, 32, 16416, 32) <= \
        lib.bd_block_attn_noalloc_scratch_bytes()
    assert lib.bd_last_hip_error() == 0


def test_launch_without_gpu_reports_hip_error():
    """With no GPU present a valid call returns BD_EHIP instead of crashing
    (run in a child process so the HIP runtime state stays out of pytest)."""
    code = r"""
import ctypes, sys
sys.path.insert(0, %r)
import torch
if torch.cuda.device_count() != 0:
    print("visible-gpu"); sys.exit(0)
from block_diffusion_decoding_amd import _lib
lib = _lib.load()
st = lib.bd_threshold_unmask(1, 32, 0, 8, 0x100000, 0x100000, 0.9, 0x100000, 0x100000, None, None, None)
print(st, lib.bd_last_hip_error())
""" % ROOT
    env = dict(os.environ, HIP_VISIBLE_DEVICES="", ROCR_VISIBLE_DEVICES="", CUDA_VISIBLE_DEVICES="")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300, env=env)
    if r.returncode != 0:
        pytest.skip(f"child exited {r.returncode}: {r.stderr[-300:]}")
    if "visible-gpu" in r.stdout:
        pytest.skip("a GPU is visible; this check is for hosts without one")
    st, err = map(int, r.stdout.split()[-2:])
    assert st == _lib.BD_EHIP and err != 0


def test_layer_piece_argument_errors():
    """RMSNorm, rotary embedding and SwiGLU reject bad shapes before any
    launch; empty calls succeed."""
    lib = _lib.load()
    E = _lib.BD_EINVAL
    d1, bad = _lib.BdRows(1, 1, 0), _lib.BdRows(0, 1, 0)
    assert lib.bd_rmsnorm(1, 0, 1536, FAKE, d1, 1e-6, FAKE, d1, None) == 0
    assert lib.bd_rmsnorm(1, 4, 0, FAKE, d1, 1e-6, FAKE, d1, None) == E
    assert lib.bd_rmsnorm(1, 4, 1536, None, d1, 1e-6, FAKE, d1, None) == E
    assert lib.bd_rmsnorm(1, 4, 1536, FAKE, bad, 1e-6, FAKE, d1, None) == E
    assert lib.bd_rmsnorm(1, 4, 1536, FAKE, d1, -1.0, FAKE, d1, None) == E
    assert lib.bd_rmsnorm(7, 4, 1536, FAKE, d1, 1e-6, FAKE, d1, None) == E
    assert lib.bd_rope(1, 2, 0, 12, 128, FAKE, d1, FAKE, 0, 1e6, None) == 0
    assert lib.bd_rope(1, 2, 8, 12, 127, FAKE, d1, FAKE, 0, 1e6, None) == E
    assert lib.bd_rope(1, 2, 8, 12, 128, FAKE, d1, None, 0, 1e6, None) == E
    assert lib.bd_rope(1, 2, 8, 12, 128, FAKE, d1, FAKE, -1, 1e6, None) == E
    assert lib.bd_rope(1, 2, 8, 12, 128, FAKE, d1, FAKE, 0, 1.0, None) == E
    assert lib.bd_swiglu(1, 0, 8960, FAKE, d1, FAKE, d1, None) == 0
    assert lib.bd_swiglu(1, 3, 0, FAKE, d1, FAKE, d1, None) == E
    assert lib.bd_swiglu(1, 3, 8960, FAKE, d1, None, d1, None) == E
    assert lib.bd_swiglu(1, 3, 8960, FAKE, bad, FAKE, d1, None) == E


def test_fused_layer_call_argument_errors():
    """The fused projections check their shapes before any launch."""
    lib = _lib.load()
    E = _lib.BD_EINVAL
    d1 = _lib.BdRows(1, 1, 0)
    big = 1 << 30
    rope = lambda **k: lib.bd_qkv_proj_rope(1, k.get("M", 128), 1536, FAKE, d1, FAKE, k.get("Nq", 1536), FAKE, d1,
                                            FAKE, FAKE, 256, FAKE, d1, FAKE, d1, k.get("d", 128),
                                            k.get("pos", FAKE), k.get("n", 8), k.get("off", 0), k.get("theta", 1e6),
                                            FAKE, big, None)
    assert rope(d=100) == E          # d % 8
    assert rope(Nq=1500) == E        # Nq % d
    assert rope(M=100) == E          # M % n_rows
    assert rope(pos=None) == E and rope(off=-1) == E and rope(theta=0.5) == E and rope(n=0) == E
    # 128 rows x 128 tiles: K split over the waves, the rotation in a pass of its own
    assert lib.bd_qkv_proj_rope_workspace_size(1, 128, 1536, 1536, 256) == 0
    # 256 rows x 3584 + 1024 columns: K split over work-groups, the rotation in the reduction
    assert lib.bd_qkv_proj_rope_workspace_size(1, 256, 8960, 3584, 512) > 0
    assert lib.bd_gate_up_swiglu(1, 128, 1000, FAKE, d1, FAKE, 8960, FAKE, d1, None) == _lib.BD_EUNSUPPORTED
    assert lib.bd_gate_up_swiglu(1, 128, 1536, FAKE, d1, None, 8960, FAKE, d1, None) == E
    assert lib.bd_gate_up_swiglu(1, 0, 1536, FAKE, d1, FAKE, 8960, FAKE, d1, None) == 0
    gn = lambda **k: lib.bd_gate_up_swiglu_rmsnorm(1, k.get("M", 128), k.get("K", 1536), FAKE, d1, k.get("eps", 1e-6),
                                                   k.get("w", FAKE), 8960, FAKE, d1, None)
    assert gn(eps=-1.0) == E and gn(eps=float("nan")) == E and gn(w=None) == E
    assert gn(K=1000) == _lib.BD_EUNSUPPORTED and gn(M=0) == 0


def test_training_form_argument_errors():
    """The 2L attention and the cross-entropy terms check their shapes
    before any launch."""
    lib = _lib.load()
    E, U = _lib.BD_EINVAL, _lib.BD_EUNSUPPORTED
    need = lib.bd_train_attn_workspace_size(1, 8, 2048, 32, 12, 2, 128)
    # two bf16 clean caches of 8 x 2 x 2048 x 128 plus 1024 entry lengths
    assert need >= 2 * 8 * 2 * 2048 * 128 * 2 + 1024 * 4
    assert lib.bd_train_attn_workspace_size(1, 8, 2000, 32, 12, 2, 128) == 0        # L % D
    ta = lambda **k: lib.bd_train_attn(1, k.get("S", 8), k.get("L", 2048), k.get("D", 32), k.get("Hq", 12), 2,
                                       k.get("d", 128), FAKE, FAKE, FAKE, 0.088, FAKE, k.get("ws", FAKE),
                                       k.get("wsb", need), None)
    assert ta(L=2000) == E and ta(Hq=13) == E and ta(d=96) == U and ta(ws=None) == E and ta(wsb=need - 16) == E
    assert ta(S=0) == 0
    nl = lambda **k: lib.bd_masked_nll(1, k.get("M", 10), k.get("hid", 1536), 151936, FAKE, 100, FAKE, FAKE,
                                       k.get("tg", FAKE), FAKE, FAKE, None, None)
    assert nl(hid=1530) == U and nl(tg=None) == E and nl(M=0) == 0


def test_device_threshold_unmask_argument_errors():
    lib = _lib.load()
    E = _lib.BD_EINVAL
    call = lambda **k: lib.bd_threshold_unmask_tau(k.get("B", 4), k.get("D", 32), k.get("lo", 8), 8, FAKE, FAKE,
                                                   k.get("tau", FAKE), FAKE, FAKE, None, None, None)
    assert call(tau=None) == E and call(D=65) == E and call(lo=30) == E and call(B=-1) == E
    assert call(B=0) == 0


def test_lmhead_unmask_argument_errors():
    lib = _lib.load()
    E = _lib.BD_EINVAL
    need = lib.bd_lmhead_workspace_size(1, 64, 3584, 152064)
    call = lambda **k: lib.bd_lmhead_unmask(1, k.get("B", 8), k.get("D", 32), k.get("lo", 8), k.get("win", 8), 3584,
                                            152064, FAKE, 300, FAKE, FAKE, k.get("tau", 0.9), k.get("tdev", None),
                                            FAKE, FAKE, None, None, k.get("tok", FAKE), k.get("bits", FAKE), None,
                                            None, None, FAKE, k.get("wsb", need), None)
    assert call(B=9) == E                       # more than 64 rows
    assert call(win=16, B=4, lo=24) == E        # window past D
    assert call(D=65) == E and call(tok=None) == E and call(bits=None) == E
    assert call(tau=float("nan")) == E          # a NaN fixed threshold
    assert call(wsb=need - 16) == E
    assert call(B=0) == 0


def test_per_sequence_window_calls_argument_errors():
    lib = _lib.load()
    E = _lib.BD_EINVAL
    un = lambda **k: lib.bd_threshold_unmask_windows(k.get("B", 4), k.get("D", 32), k.get("win", 8),
                                                     k.get("lo", FAKE), FAKE, FAKE, k.get("tau", 0.9), FAKE, FAKE,
                                                     None, None, None)
    assert un(lo=None) == E and un(D=65) == E and un(win=33) == E and un(tau=float("nan")) == E
    assert un(B=0) == 0
    cp = lambda **k: lib.bd_copy_rows(k.get("B", 4), k.get("n", 33), k.get("rb", 3072), k.get("mask", FAKE),
                                      FAKE, FAKE, k.get("s1", None), k.get("d1", None), None)
    assert cp(n=65) == E and cp(rb=3000) == E and cp(mask=None) == E and cp(s1=FAKE) == E
    assert cp(s1=FAKE + 8, d1=FAKE) == E          # misaligned
    assert cp(B=0) == 0 and cp(n=0) == 0
    sc = lambda **k: lib.bd_persequence_schedule(k.get("B", 4), k.get("D", 32), k.get("S", 8), k.get("bits", FAKE),
                                                 FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, k.get("rows", FAKE), FAKE,
                                                 None, None, None)
    assert sc(B=-1) == E and sc(S=0) == E and sc(D=64, S=8) == E and sc(D=32, S=12) == E and sc(D=4, S=8) == E
    assert sc(bits=None) == E and sc(rows=None) == E
    assert sc(B=0) == 0


def test_probe_argument_errors():
    lib = _lib.load()
    E = _lib.BD_EINVAL
    pr = lambda **k: lib.bd_probe_weight_stream(k.get("w", FAKE), k.get("rows", 1024), k.get("rb", 7168),
                                                k.get("x", None), k.get("xt", 0), k.get("wg", 64), None)
    assert pr(w=None) == E and pr(rows=1000) == E and pr(rb=7000) == E and pr(xt=4) == E and pr(xt=2, x=FAKE) == E
    assert pr(wg=0) == E and pr(wg=65) == E and pr(w=FAKE + 8) == E and pr(xt=4, x=FAKE + 8) == E


def test_guard_argument_errors():
    """A guard's words must be given, 8-byte aligned and 1..4096 of them;
    errors come back before any launch (no GPU touched)."""
    lib = _lib.load()
    E = _lib.BD_EINVAL
    R = _lib.BdRows
    big = 1 << 30
    G = _lib.BdGuard
    for g in (G(None, 1, 4), G(FAKE + 4, 1, 4), G(FAKE, 1, 0), G(FAKE, 1, 4097)):
        ref = ctypes.byref(g)
        assert lib.bd_linear_guarded(1, 64, 3584, 3584, FAKE, R(64, 64, 0), FAKE, None, R(1, 1, 0), FAKE,
                                     R(64, 64, 0), FAKE, big, ref, None) == E
        assert lib.bd_qkv_proj_guarded(1, 64, 3584, FAKE, R(64, 64, 0), FAKE, 3584, FAKE, R(64, 64, 0), FAKE, FAKE,
                                       512, FAKE, R(64, 64, 0), FAKE, R(64, 64, 0), FAKE, big, ref, None) == E
        assert lib.bd_block_attn_guarded(1, 2, 28, 4, 128, 32, FAKE, 8, 8, FAKE, FAKE, FAKE, 64, FAKE, FAKE, 32,
                                         0.1, FAKE, None, FAKE, big, ref, None) == E
    # a valid guard on an empty problem is fine (nothing to launch)
    ok = ctypes.byref(G(FAKE, 1, 4))
    assert lib.bd_linear_guarded(1, 0, 3584, 3584, FAKE, R(1, 1, 0), FAKE, None, R(1, 1, 0), FAKE, R(1, 1, 0),
                                 None, 0, ok, None) == 0
    assert lib.bd_last_hip_error() == 0
