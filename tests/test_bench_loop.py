"""Host logic of bench.py's decode loop, on the CPU with a stand-in decoder
whose steps unmask positions deterministically from the mask bits alone:
pipelined runs (whole windows queued ahead of the host over at most two
blocks with two ring parities, the oldest read back while later ones run;
slots of one window with one wait at the ends) book exactly the steps,
tokens, commits and per-block schedules of the same loop taken one step at
a time, and book them from rings no later block has overwritten.  Also: the
committed traffic records belong to the current kernel sources."""
import json
import os
from types import SimpleNamespace

import numpy as np
import pytest

import bench


class FakeDecoder:
    """Mask-bit state of B sequences; a step of window s unmasks, in every
    sequence with masked positions there, 1 to 3 of the lowest ones (a count
    fixed by the block, window, sequence and bits), so that any order of
    launching the same steps gives the same bits."""

    def __init__(self, B, D, S):
        self.B, self.D, self.S = B, D, S
        self.bits = np.zeros(B, np.uint64)
        self.blk = -1
        self.rings = np.zeros((2, D // S, S, B), np.uint64)
        self.inflight = []                          # blocks of the runs queued and not yet read back
        self.max_inflight = 0
        self.commits = 0
        self.log = []

    def slots(self, S):
        return S

    def windows_complete(self, S):
        return True

    def set_block(self, tokens, masked, plant=None):
        self.blk += 1
        self.bits = np.full(self.B, (1 << self.D) - 1, np.uint64)

    def _step(self, s):
        self.log.append(("step", self.blk, s))
        wm = ((1 << self.S) - 1) << (s * self.S)
        for b in range(self.B):
            m = int(self.bits[b]) & wm
            if m:
                k = 1 + (self.blk * 7 + s * 3 + b + bin(m).count("1")) % 3
                for _ in range(k):
                    if m:
                        low = m & -m
                        m ^= low
                        self.bits[b] = np.uint64(int(self.bits[b]) & ~low)

    def e_step(self, s, S, tau):
        self._step(s)

    def dc_step(self, s, S, tau):
        self._step(s)

    def mask_bits_host(self):
        return self.bits.copy()

    def commit(self):
        self.commits += 1
        self.log.append(("commit", self.blk))

    def run_window(self, s, S, tau, wait=True, parity=0):
        for i in range(S):
            self._step(s)
            self.rings[parity, s, i] = self.bits
        if wait:
            return self.rings[parity, s].copy()
        self._queued()
        return None

    def fence(self):
        return SimpleNamespace(synchronize=lambda: None)

    def run_slots(self, s, S, tau, i0, i1, parity=0):
        for i in range(i0, i1):
            self._step(s)
            self.rings[parity, s, i] = self.bits
        self._queued()

    def wait(self):
        pass

    def window_bits(self, s, S, parity=0):
        # one read per queued run (the loop books runs in order); a ring row
        # overwritten by a later block before its run was booked would make
        # the booking differ from the one-step-at-a-time loop
        self.inflight.pop(0)
        return self.rings[parity, s].copy()

    def _queued(self):
        self.inflight.append(self.blk)
        self.max_inflight = max(self.max_inflight, len(self.inflight))
        # a block's windows write the ring parity of the block two back
        assert len(set(self.inflight)) <= 2, "more than two blocks in flight"


def _state(loop):
    return (loop.steps, loop.tokens, loop.commits, list(loop.done_blocks), loop.blk, loop.s, loop.first,
            loop.bits.tolist(), loop.own.tolist(), loop.block_steps)


@pytest.mark.parametrize("B,S", [(8, 8), (3, 4), (5, 16)])
def test_pipelined_runs_book_like_single_steps(B, S):
    cfg = SimpleNamespace(B=B, D=32, S=S, tau=0.9)
    a = bench.Loop(FakeDecoder(B, 32, S), cfg, [None])
    b = bench.Loop(FakeDecoder(B, 32, S), cfg, [None])
    for n in [10, 60, 7, 1, 33, 64, 5, 120, 3, 400]:
        a.run(n, windows=True)            # pipelined runs
        b.run(n, windows=False)           # one step and one wait at a time
        assert _state(a) == _state(b), n
        assert a.dec.commits == b.dec.commits == a.commits
        assert a.dec.inflight == []       # every queued window read back before run() returns
        # the same real steps on the device, in order (queued runs add only
        # slots past the end of a window)
        assert b.dec.log == _real_steps(a.dec.log, b.dec.log)
    assert a.commits >= 3
    # runs really were queued ahead of the read-backs (up to two blocks)
    assert a.dec.max_inflight > 1


def _real_steps(log_a, log_b):
    """log_a without the dead slots: the entries of log_b, matched in order."""
    out, j = [], 0
    for e in log_a:
        if j < len(log_b) and e == log_b[j]:
            out.append(e)
            j += 1
    assert j == len(log_b)
    return out


def test_pipelined_runs_keep_at_most_two_blocks_in_flight():
    """A window is queued only while no window of the block two back is
    unread (its ring parity): with a large budget the GPU is never more than
    two blocks ahead of the host's read-backs."""
    cfg = SimpleNamespace(B=2, D=32, S=8, tau=0.9)
    dec = FakeDecoder(2, 32, 8)
    loop = bench.Loop(dec, cfg, [None])
    loop.run(200, windows=True)
    assert loop.steps == 200 and dec.inflight == []
    assert dec.max_inflight > 4


def test_pipelined_whole_blocks_book_like_single_steps():
    """stop_blk: whole blocks, pipelined, until a given block starts."""
    cfg = SimpleNamespace(B=3, D=32, S=8, tau=0.9)
    a = bench.Loop(FakeDecoder(3, 32, 8), cfg, [None])
    b = bench.Loop(FakeDecoder(3, 32, 8), cfg, [None])
    for blk in (1, 4, 5):
        a.pipelined(0, stop_blk=blk)
        while b.blk < blk:
            b.step()
        assert a.blk == blk and a.dec.inflight == []
        assert _state(a) == _state(b), blk


def test_traffic_records_match_the_kernel_sources():
    """Every committed HBM traffic record under profiles/ was measured on the
    current sources of its kernels (bench.py reports it only then): a kernel
    change without a new counter run fails here rather than silently turning
    the reported traffic into null."""
    import bench
    for kind, spec in bench.TRAFFIC.items():
        rec = json.load(open(os.path.join(bench.ROOT, "profiles", spec["file"])))
        assert rec["kernel_source_hash"] == bench.kernel_source_hash(kind), \
            f"{spec['file']}: retake the FETCH_SIZE/WRITE_SIZE passes of bench.py --section {spec['section']}"
        assert rec["bytes_per_launch"] > 0
