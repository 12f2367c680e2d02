"""Benchmark of the block-diffusion refinement step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--rate 0.5]

Headline workload (7B shape): Qwen2.5-7B-shaped attention layer (28 query /
4 KV heads of dim 128, hidden 3584) + LM head 3584 x 152064, bf16, batch 8
with committed prefixes drawn uniformly from 1024..4096 tokens (block
aligned), block 32, sub-block 8, threshold 0.9, planted peaked logits for a
fraction `rate` of the masked rows.  The timed loop is a real lockstep block
decode: every window starts with an exact step (which refreshes the DualCache
snapshot), DualCache steps follow until no position of the window is masked
in any sequence, and a finished block is committed (forward over the clean
block + cache append) before the next one starts.  W untimed steps, then
exactly K timed refinement steps; value = K / time (steps/s), and decoded
tokens / time is reported beside it.

Also measured in the same run (reported under "extra"):
* attention alone at the long-context shape (batch 32, 16384 committed tokens,
  28/4 heads) in DualCache (8 rows) and exact (32 rows) form, against 8 TB/s;
* the LM head alone at batch 1 (1.5B shape, 8 rows) against 8 TB/s and at 1024
  rows (7B shape) against the dense bf16 MFMA peak (2.5 PFLOP/s);
* a fixed-schedule long-context block (32 sequences x 16384 prefix: 4 windows
  x 8 steps + commit), decoded tokens/s.

roofline: the dominant kernel of the headline step is the LM head (its
weights are ~92% of the step's bytes); its launches are timed with HIP events
on the launch stream, over a second timed pass of the same loop with eager
launches (the headline pass replays each step as a captured HIP graph).
cpu_baseline: the fp64 oracle (oracle/), timed on this host on a bounded
sample of the same workload (DualCache steps of the same 8 sequences).
"""
import os

try:
    _CORES = len(os.sched_getaffinity(0))
except AttributeError:  # pragma: no cover
    _CORES = os.cpu_count() or 1
for _v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
    os.environ[_v] = str(_CORES)

import argparse
import collections
import hashlib
import json
import sys
import time

from dataclasses import replace
from typing import NamedTuple

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import bd_inputs as bi  # noqa: E402

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
METRIC = "block-refine steps/s & decoded tokens/s at 7B shape; % of HBM/MFMA peak"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


CALIB_BYTES = 1 << 30  # plain device copy that calibrates the HBM byte counters

# Measured HBM traffic records (profiles/*.json), one per counted launch: the
# launch's main kernel (its template instance, as rocprofv3 names it) and the
# kernel that follows it in the same call, the section of this script whose
# profiling run counts them, and the sources the kernels are built from (a
# stored reading is used only while they are unchanged).
TRAFFIC = {
    "lm": {"file": "lmhead_7B_M64_traffic.json", "section": "lm",
           "sources": ("lmhead.hip", "stream_gemm.h", "bd_device.h", "bd_launch.h"),
           "main": "lm_stream_kernel<4, 4>", "then": "lm_merge_unmask_kernel",
           "launch": "bd_lmhead_unmask: lm_stream_kernel<4, 4> (256 work-groups, one per CU, weight tiles with "
                     "the non-temporal hint) + lm_merge_unmask_kernel (8 work-groups x 512), 64 rows x 152064 x "
                     "3584 (8 sequences x window of 8)"},
    "attn_dualcache": {"file": "attention_long_context_dualcache_traffic.json", "section": "attn",
                       "sources": ("attn.hip", "bd_device.h", "bd_launch.h"),
                       "main": "attn_bf16_kernel<128, 32, 1,", "then": "attn_merge_kernel",
                       "launch": "bd_block_attn DualCache step: attn_bf16_kernel<128, 32, 1, 8, 2> (committed "
                                 "K/V with the non-temporal hint) + attn_merge_kernel<128, 2>, 32 sequences x 16384 "
                                 "cached rows, 8 fresh rows x 28 query heads, 4 KV heads, d 128"},
    "attn_exact": {"file": "attention_long_context_exact_traffic.json", "section": "attn",
                   "sources": ("attn.hip", "bd_device.h", "bd_launch.h"),
                   "main": "attn_bf16_kernel<128, 32, 2,", "then": "attn_merge_kernel",
                   "launch": "bd_block_attn exact step: attn_bf16_kernel<128, 32, 2, 8, 2> (committed K/V with "
                             "the non-temporal hint) + attn_merge_kernel<128, 2>, 32 sequences x 16384 cached rows, "
                             "32 fresh rows x 28 query heads, 4 KV heads, d 128"},
}


def kernel_source_hash(kind: str = "lm") -> str:
    """Hash of the sources a counted launch's kernels are built from."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_diffusion_decoding_amd", "csrc")
    for f in TRAFFIC[kind]["sources"]:
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def traffic_from(kind, fetch_csv, write_csv):
    """Turn two rocprofv3 --pmc counter files (FETCH_SIZE, then WRITE_SIZE,
    both over `bench.py --section <section of kind>`) into the HBM bytes per
    launch of the counted call: every dispatch of its main kernel plus the
    dispatch of its second kernel that follows it.  Each counter is scaled by
    what it reads for the plain device copy of CALIB_BYTES the section makes
    first (the copy reads and writes exactly CALIB_BYTES)."""
    import csv
    spec = TRAFFIC[kind]

    def rows(path, counter):
        rs = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        key = "Dispatch_Id" if rs and "Dispatch_Id" in rs[0] else "Correlation_Id"
        return sorted(rs, key=lambda r: int(r[key])), key

    out = {"kernel_source_hash": kernel_source_hash(kind), "calibration_bytes": CALIB_BYTES, "launch": spec["launch"]}
    total = 0.0
    for path, counter in ((fetch_csv, "FETCH_SIZE"), (write_csv, "WRITE_SIZE")):
        rs, key = rows(path, counter)
        main, then = [], []
        for i, r in enumerate(rs):
            if spec["main"] in r["Kernel_Name"]:
                nxt = next((x for x in rs[i + 1:] if spec["then"] in x["Kernel_Name"]), None)
                if nxt is not None:
                    main.append(float(r["Counter_Value"]))
                    then.append(float(nxt["Counter_Value"]))
        cp = [float(r["Counter_Value"]) for r in rs
              if "copyBuffer" in r["Kernel_Name"] or "copy_kernel" in r["Kernel_Name"]]
        if not main or not cp:
            raise SystemExit(f"{path}: no {counter} reading for {spec['main']} + {spec['then']} or the calibration copy")
        kib = float(np.median(main)) + float(np.median(then))
        scale = CALIB_BYTES / (max(cp) * 1024.0)
        out[counter] = {"kib_per_launch": kib, "main_kib": float(np.median(main)),
                        "then_kib": float(np.median(then)), "dispatches": len(main), "copy_kib": max(cp),
                        "scale": scale, "bytes_per_launch": kib * 1024.0 * scale}
        total += kib * 1024.0 * scale
    out["bytes_per_launch"] = total
    path = os.path.join(ROOT, "profiles", spec["file"])
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def make_decoder(cfg, w, pre):
    from block_diffusion_decoding_amd.decoder import BlockDecoder, Dims
    dims = Dims(cfg.B, cfg.Hq, cfg.Hkv, cfg.d, cfg.hidden, cfg.V, cfg.D, cfg.cap)
    weights = {k: torch.from_numpy(getattr(w, k)) for k in ("E", "Wq", "Wk", "Wv", "Wo", "Wlm")}
    dec = BlockDecoder(dims, weights, dtype=torch.bfloat16, device="cuda")
    dec.set_synthetic_prefix(pre.kv_len, pre.cache_k, pre.cache_v, pre.carry)
    return dec


def block_plants(cfg, w, rate, seed, n_blocks):
    """Planted offsets for fresh blocks: a seeded fraction `rate` of all D
    positions j >= 1 get an offset on input row j - 1 (position 0 is never
    planted, so the carry row stays as the model computed it)."""
    out = []
    for k in range(n_blocks):
        st = bi.BlockState(np.zeros((cfg.B, cfg.D), np.int32), np.ones((cfg.B, cfg.D), bool), 0, cfg.D)
        st.masked[:, 0] = False
        plant, _, _ = bi.make_plants(cfg, seed + 1000 + k, w, st, rate)
        out.append(torch.from_numpy(plant).to("cuda", torch.bfloat16))
    return out


class LaunchTimer:
    """HIP events around launches on the current stream.  Before each start
    event a short spin kernel is queued, so the host has queued the timed
    launch before the GPU reaches the event: the interval holds GPU time only
    (without it, a GPU that has caught up with the host would wait inside the
    interval for the launch to be submitted)."""

    SPIN_CYCLES = 200000

    def __init__(self):
        self.events = []

    def start(self):
        torch.cuda._sleep(self.SPIN_CYCLES)
        ev = torch.cuda.Event(enable_timing=True)
        ev.record()
        self.events.append([ev, None])

    def stop(self):
        ev = torch.cuda.Event(enable_timing=True)
        ev.record()
        self.events[-1][1] = ev

    def seconds(self) -> np.ndarray:
        return np.array([a.elapsed_time(b) for a, b in self.events]) * 1e-3


class Loop:
    """Lockstep block decode, one refinement step per call of step(), or
    many steps per call of run()."""

    def __init__(self, dec, cfg, plants):
        self.dec, self.cfg, self.plants = dec, cfg, plants
        self.blk = -1
        self.s = 0
        self.first = True
        self.slot = 0                    # next slot of the current window (run's queued path)
        self.steps = self.tokens = self.commits = 0
        self.bits = None
        self.wmask = [np.uint64(((1 << cfg.S) - 1) << (w * cfg.S)) for w in range(cfg.D // cfg.S)]
        self.full = np.full(cfg.B, (1 << cfg.D) - 1, dtype=np.uint64)
        # steps each sequence needed on its own (it had a masked position of the
        # window before the step), per block: the schedule a per-sequence
        # window progression would follow (identical tokens, pinned in the oracle)
        self.own = np.zeros(cfg.B, np.int64)
        self.block_steps = 0
        self.done_blocks = []            # (lockstep steps, max over sequences of own steps)
        self._new_block()

    def _new_block(self):
        cfg = self.cfg
        self.blk += 1
        self.dec.set_block(np.zeros((cfg.B, cfg.D), np.int32), np.ones((cfg.B, cfg.D), bool),
                           self.plants[self.blk % len(self.plants)])
        self.s, self.first, self.slot = 0, True, 0
        self.bits = self.full.copy()

    def step(self):
        cfg, dec = self.cfg, self.dec
        S = cfg.S
        if self.first:
            dec.e_step(self.s, S, cfg.tau)
        else:
            dec.dc_step(self.s, S, cfg.tau)
        self.first = False
        self.steps += 1
        self.block_steps += 1
        self.own += (self.bits & self.wmask[self.s]) != 0
        bits = dec.mask_bits_host()      # 8 bytes per sequence, refreshed by the step itself
        self.tokens += int(np.bitwise_count(self.bits ^ bits).sum())
        self.bits = bits
        self.slot += 1
        if not (bits & self.wmask[self.s]).any():
            self._next_window()

    def _next_window(self):
        self.s += 1
        self.first = True
        self.slot = 0
        if self.s == self.cfg.D // self.cfg.S:
            self.dec.commit()
            self._block_done()

    def _book_block(self):
        """Book a committed block."""
        self.commits += 1
        self.done_blocks.append((self.block_steps, int(self.own.max())))
        self.own[:] = 0
        self.block_steps = 0

    def _block_done(self):
        """Book a committed block and set up the next one."""
        self._book_block()
        self._new_block()

    def _account(self, ring, s, before) -> int:
        """Book slots of window s (mask bits after each slot, [n, B], and the
        bits before the first); returns the refinement steps among them (the
        slots before which a masked position of the window was left)."""
        wm = self.wmask[s]
        prev = np.concatenate([before[None], ring[:-1]])
        had = (prev & wm) != 0                       # [n, B]
        steps = int(had.any(axis=1).sum())
        self.own += had.sum(axis=0)
        self.block_steps += steps
        self.tokens += int(np.bitwise_count(before ^ ring[-1]).sum())
        self.steps += steps
        return steps

    def window(self) -> int:
        """The current window's first steps (from its exact step on) as one
        captured graph of slots(S) step slots and one wait; returns the
        refinement steps they took."""
        assert self.first
        ring = self.dec.run_window(self.s, self.cfg.S, self.cfg.tau)
        steps = self._account(ring, self.s, self.bits)
        self.bits = ring[-1]
        self.first = False
        self.slot = len(ring)
        if not (self.bits & self.wmask[self.s]).any():
            self._next_window()
        return steps

    def pipelined(self, n: int, stop_blk=None):
        """Exactly n refinement steps, queued ahead of the host.  A cursor
        walks the step slots in order (S per window; a window's S slots
        always finish it, so the cursor moves on without looking at the
        bits) and queues as many slots as the worst case allows: slots in
        flight (each may be a step) never exceed the steps still to take.
        Whole windows from their first slot go as one graph, other runs as
        per-slot graphs.  The host waits only for the oldest run in flight
        when the budget is used up (or the ring parity of the cursor's block
        is still unread: at most two blocks in flight) and books it; runs
        that turn out to hold slots past the end of their window free that
        much budget.  Requires windows_complete(S).  With stop_blk (from a
        block start): whole blocks until block stop_blk starts, n ignored."""
        cfg, dec = self.cfg, self.dec
        S, nw = cfg.S, cfg.D // cfg.S
        if stop_blk is not None:
            assert self.slot == 0 and self.s == 0
            n = 1 << 62
        left = n                          # steps not yet booked
        worst = 0                         # slots in flight (each may be a step)
        pend = collections.deque()        # runs in flight: (event, block, window, first slot, end slot)
        cur = self.bits                   # mask bits after the last booked slot
        while left > 0:
            if stop_blk is not None and self.blk >= stop_blk and not pend:
                break
            room = left - worst
            if (room > 0 and (not pend or pend[0][1] >= self.blk - 1)
                    and (stop_blk is None or self.blk < stop_blk)):
                k = min(room, S - self.slot)
                if self.slot == 0 and k == S:
                    dec.run_window(self.s, S, cfg.tau, wait=False, parity=self.blk % 2)
                else:
                    dec.run_slots(self.s, S, cfg.tau, self.slot, self.slot + k, parity=self.blk % 2)
                pend.append((dec.fence(), self.blk, self.s, self.slot, self.slot + k))
                worst += k
                self.slot += k
                if self.slot == S:
                    self.s, self.slot = self.s + 1, 0
                    if self.s == nw:
                        dec.commit()
                        self._new_block()  # queued copies; the block is booked when read back
                continue
            ev, blk, s, i0, i1 = pend.popleft()
            ev.synchronize()
            ring = dec.window_bits(s, S, blk % 2)[i0:i1]
            before = self.full if (s == 0 and i0 == 0) else cur
            left -= self._account(ring, s, before)
            worst -= i1 - i0
            cur = ring[-1]
            if i1 == S:
                if (cur & self.wmask[s]).any():
                    raise RuntimeError(f"window {s} still has masked positions after its {S} slots")
                if s == nw - 1:
                    self._book_block()
            if not pend:
                self.bits = self.full.copy() if (self.s == 0 and self.slot == 0) else cur
                if self.slot > 0 and not (cur & self.wmask[self.s]).any():
                    self._next_window()   # the cursor's window ended early: skip its other slots
        self.first = self.slot == 0

    def run(self, n: int, windows: bool):
        """Exactly n refinement steps.  With window graphs: whole windows
        queued ahead of the host (pipelined) when a window's slots always
        finish it, else window graphs while at least a graph's slots remain;
        single steps otherwise."""
        left = n
        S = self.cfg.S
        slots = self.dec.slots(S)
        if windows and self.dec.windows_complete(S):
            self.pipelined(n)
            return
        while left > 0:
            if windows and self.first and left >= slots:
                left -= self.window()
            else:
                self.step()
                left -= 1


def graph_costs(dec, cfg, plant, reps=10) -> dict:
    """GPU time of the captured graphs the loop replays, each from a fresh
    block (every position masked, so every slot of window 0 is a refinement
    step): a whole window (its exact step and DualCache slots as one graph),
    the exact step alone, a DualCache step alone, and the commit.  HIP events
    around each replay, medians.  A window against its slots gives a step's
    cost inside one graph; a graph launched on its own adds its launch."""
    S = cfg.S
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    zeros, ones = np.zeros((cfg.B, cfg.D), np.int32), np.ones((cfg.B, cfg.D), bool)

    def fresh():
        dec.set_block(zeros, ones, plant)
        torch.cuda.synchronize()

    def med(fn, n=reps, prep=fresh):
        ts = []
        for i in range(n + 2):
            prep()
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            if i >= 2:
                ts.append(e0.elapsed_time(e1) * 1e3)
        return round(float(np.median(ts)), 1)

    def after_exact():  # a DualCache step follows its window's exact step (which leaves the rows current)
        fresh()
        dec.e_step(0, S, cfg.tau)
        torch.cuda.synchronize()

    win = med(lambda: dec.run_window(0, S, cfg.tau, wait=False))
    fresh()
    bits = dec.run_window(0, S, cfg.tau, wait=True)
    before = np.concatenate([np.full((1, cfg.B), (1 << cfg.D) - 1, np.uint64), bits[:-1]])
    live = int(((before & np.uint64((1 << S) - 1)) != 0).any(axis=1).sum())
    out = {"window_graph_us": win, "window_slots": int(len(bits)), "window_live_slots": live,
           "us_per_slot_in_window": round(win / len(bits), 1),
           "exact_step_graph_us": med(lambda: dec.e_step(0, S, cfg.tau)),
           "dualcache_step_graph_us": med(lambda: dec.dc_step(0, S, cfg.tau), prep=after_exact)}
    n_commit = 3
    if np.all(dec.kv_len_host + cfg.D * (n_commit + 2) <= cfg.cap):
        out["commit_graph_us"] = med(dec.commit, n_commit, prep=torch.cuda.synchronize)
    out["what"] = ("medians of HIP-event intervals around replays of the captured graphs, each from a fresh "
                   "block: window 0 as one graph, its exact step alone, a DualCache step alone, the commit")
    return out


class Timing(NamedTuple):
    median: float
    mean: float
    p10: float
    p90: float

    def record(self) -> dict:
        """Microsecond fields of a single-call record."""
        return {"us": self.mean * 1e6, "us_median": self.median * 1e6, "us_p10": self.p10 * 1e6,
                "us_p90": self.p90 * 1e6}


def time_call(fn, reps, warm=3, warm_s=0.1, before=None) -> Timing:
    """Median, mean, 10th and 90th percentile (seconds) of `reps` calls, each
    bracketed by HIP events on the current stream, after at least `warm` calls
    and `warm_s` seconds of the same call (the clocks take ~20 ms of sustained
    load to settle after the host-side input generation left the GPU idle).
    before(): queued ahead of every timed call, outside its interval."""
    t_end = time.perf_counter() + warm_s
    n = 0
    while n < warm or time.perf_counter() < t_end:
        fn()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in evs:
        if before is not None:
            before()
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) for a, b in evs]) * 1e-3
    return Timing(float(np.median(t)), float(np.mean(t)), float(np.percentile(t, 10)), float(np.percentile(t, 90)))


def extras_e2e(graphs=True, n_blocks=None):
    """End-to-end decode of the random-init 1.5B-shaped model: B prompts of
    prompt_len ids, prefill, then n_blocks blocks of D generated in windows of
    S with threshold tau (steps replayed as captured HIP graphs).  The weights
    are N(0, 0.02) drawn on the GPU from a seeded generator (no oracle runs at
    this size)."""
    from block_diffusion_decoding_amd.model import ModelDecoder, ModelDims
    cfg = bi.C5
    nb = cfg.n_blocks if n_blocks is None else n_blocks
    log(f"[bench] end-to-end 1.5B-shape decode: {cfg.n_layers} layers, B {cfg.B}, prompt {cfg.prompt_len}, "
        f"{nb} blocks")
    dev, dt = "cuda", torch.bfloat16
    g = torch.Generator(device=dev)
    g.manual_seed(5)

    def rnd(*shape):
        return (torch.randn(*shape, generator=g, device=dev, dtype=torch.float32) * cfg.std).to(dt)

    hq, hkv, hid, I = cfg.Hq * cfg.d, cfg.Hkv * cfg.d, cfg.hidden, cfg.inter
    weights = {"E": rnd(cfg.V + 1, hid), "Wlm": rnd(cfg.V, hid),
               "layers": [{"Wq": rnd(hq, hid), "Wk": rnd(hkv, hid), "Wv": rnd(hkv, hid), "Wo": rnd(hid, hq),
                           "Wg": rnd(I, hid), "Wu": rnd(I, hid), "Wd": rnd(hid, I)} for _ in range(cfg.n_layers)]}
    dims = ModelDims(cfg.B, cfg.Hq, cfg.Hkv, cfg.d, hid, cfg.V, cfg.D, cfg.prompt_len + nb * cfg.D,
                     n_layers=cfg.n_layers, inter=I, eps=cfg.eps, theta=cfg.theta)
    dec = ModelDecoder(dims, weights, dtype=dt, device=dev)
    del weights
    prompts = bi.make_prompts(cfg, 0)
    layer_bytes = sum(t.numel() * 2 for lw in dec.layers for t in lw.values())
    lm_bytes = dec.W["Wlm"].numel() * 2
    n_weight_bytes = layer_bytes + 2 * lm_bytes   # layers, LM head and embedding table
    # warm-up: a prefill and one block (also sizes every workspace), then capture
    dec.prefill(prompts)
    dec.new_block()
    dec.decode_block(cfg.S, cfg.tau)
    if graphs:
        dec.capture(cfg.S, cfg.tau)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    dec.prefill(prompts)
    torch.cuda.synchronize()
    t_pre = time.perf_counter() - t0
    steps = []
    t1 = time.perf_counter()
    for _ in range(nb):
        dec.new_block()
        steps.append(dec.decode_block(cfg.S, cfg.tau))
    torch.cuda.synchronize()
    t_dec = time.perf_counter() - t1
    tokens = cfg.B * nb * cfg.D
    n_steps = int(sum(steps))
    log(f"[bench] e2e: prefill {t_pre * 1e3:.1f} ms, decode {t_dec * 1e3:.1f} ms for {tokens} tokens "
        f"({n_steps} refinement steps + {nb} commits): {tokens / t_dec:.0f} tokens/s decoding, "
        f"{tokens / (t_pre + t_dec):.0f} tokens/s with the prefill")
    out = {"e2e_1.5B": {"shape": f"{cfg.n_layers} layers, hidden {hid}, {cfg.Hq}q/{cfg.Hkv}kv heads d{cfg.d}, "
                                 f"MLP {I}, vocab {cfg.V}; B {cfg.B}, prompt {cfg.prompt_len}, {nb} blocks of "
                                 f"{cfg.D} (sub-block {cfg.S}), tau {cfg.tau}",
                        "prefill_ms": t_pre * 1e3, "decode_ms": t_dec * 1e3, "tokens": tokens,
                        "refinement_steps": n_steps, "commits": nb,
                        "decode_tokens_per_s": tokens / t_dec, "tokens_per_s_with_prefill": tokens / (t_pre + t_dec),
                        "ms_per_step": t_dec / (n_steps + nb) * 1e3, "weight_bytes_per_forward": n_weight_bytes,
                        # a refinement step streams every layer's weights and the LM head once, a
                        # commit the layers' weights: those bytes per second of the decode against
                        # the 8 TB/s spec
                        "weight_GB_per_s": (n_steps * (layer_bytes + lm_bytes) + nb * layer_bytes) / t_dec / 1e9,
                        "frac_hbm_weights": (n_steps * (layer_bytes + lm_bytes) + nb * layer_bytes) / t_dec / 1e9
                        / HBM_PEAK_GBS,
                        "graphs": graphs}}
    del dec
    torch.cuda.empty_cache()
    return out


def train_attn_flops(cfg) -> float:
    """Algorithmic FLOPs of one 2L-layout attention call: every visible
    (query, key) pair costs a d-long dot product for the score and one for
    the output (2 flops per multiply-add each).  Per view sequence and query
    head, block b's D noisy and D clean rows each see (b + 1) * D keys."""
    nb = cfg.L // cfg.D
    pairs = 2 * sum(cfg.D * (b + 1) * cfg.D for b in range(nb))
    return 4.0 * cfg.d * pairs * cfg.Hq * 2 * cfg.S


def extras_train(reps):
    """Training form (forward pass and loss value) of the 1.5B-shaped layer:
    S samples of L tokens in both complementary views, i.e. 2S sequences of
    2L rows; the 2L attention alone and the whole forward + loss."""
    from block_diffusion_decoding_amd import ops
    from block_diffusion_decoding_amd.train import TrainForward
    cfg = bi.T3
    log(f"[bench] training form: {cfg.S} samples x L {cfg.L} in 2 views, {cfg.Hq}q/{cfg.Hkv}kv heads d{cfg.d}, "
        f"hidden {cfg.hidden}, vocab {cfg.V}")
    dev, dt = "cuda", torch.bfloat16
    g = torch.Generator(device=dev)
    g.manual_seed(7)

    def rnd(*shape):
        return (torch.randn(*shape, generator=g, device=dev, dtype=torch.float32) * cfg.std).to(dt)

    hq, hkv, hid = cfg.Hq * cfg.d, cfg.Hkv * cfg.d, cfg.hidden
    W = {"E": rnd(cfg.V + 1, hid), "Wq": rnd(hq, hid), "Wk": rnd(hkv, hid), "Wv": rnd(hkv, hid),
         "Wo": rnd(hid, hq), "Wlm": rnd(cfg.V, hid)}
    tf = TrainForward(W, cfg.Hq, cfg.Hkv, cfg.d, cfg.D, dtype=dt, device=dev)
    del W
    x0, m = bi.make_train_batch(cfg, 0)
    plan = tf.plan(x0, m)
    res = tf.forward(x0, m, plan)
    t_fwd = time_call(lambda: tf.forward(x0, m, plan), max(3, reps // 4)).median
    n = res["count"]
    S2, L2 = 2 * cfg.S, 2 * cfg.L
    q = tf._bufs["q"].view(S2, L2, cfg.Hq, cfg.d)
    k = tf._bufs["k"].view(S2, L2, cfg.Hkv, cfg.d)
    v = tf._bufs["v"].view(S2, L2, cfg.Hkv, cfg.d)
    o = tf._bufs["o"].view(S2, L2, cfg.Hq, cfg.d)
    t_att, t_att_mean = time_call(lambda: ops.bd_train_attn(q, k, v, o, L=cfg.L, D=cfg.D), reps)[:2]
    fl = train_attn_flops(cfg)
    loss = float(res["loss_sum"].cpu()[0])
    log(f"[bench] training form: forward + loss {t_fwd * 1e3:.2f} ms for {n} supervised tokens "
        f"({n / t_fwd:.0f} tokens/s), mean loss {loss / n:.4f}; 2L attention {t_att * 1e6:.1f} us = "
        f"{fl / t_att / 1e15:.3f} PFLOP/s ({fl / t_att / 2.5e15 * 100:.1f}% of the bf16 MFMA peak)")
    out = {"train_1.5B_layer": {
        "shape": f"{cfg.S} samples x L {cfg.L} (D {cfg.D}), 2 complementary views = {S2} sequences of {L2} rows; "
                 f"{cfg.Hq}q/{cfg.Hkv}kv heads d{cfg.d}, hidden {hid}, vocab {cfg.V}",
        "forward_and_loss_ms": t_fwd * 1e3, "supervised_tokens": n, "supervised_tokens_per_s": n / t_fwd,
        "mean_loss": loss / n,
        "attention_us_median": t_att * 1e6, "attention_us_mean": t_att_mean * 1e6, "attention_flops": fl,
        "attention_pflops": fl / t_att / 1e15, "attention_frac_of_bf16_mfma_peak": fl / t_att / 2.5e15}}
    del tf
    torch.cuda.empty_cache()
    return out


def extras_subblock(w3, graphs, steps=40, warmup=10):
    """The headline loop (7B shape, planted pass rate 0.5) at sub-block sizes
    4, 8, 16 and 32 (= the block: every step recomputes all D rows): the pages
    call the best sub-block size task-dependent."""
    out = {}
    pre = None
    for S in (4, 8, 16, 32):
        cfg = replace(bi.C3, S=S)
        if pre is None:
            pre = bi.make_prefix(cfg, 0)
        dec = make_decoder(cfg, w3, pre)
        plants = block_plants(cfg, w3, 0.5, 0, 8)
        if graphs:
            dec.capture(cfg.S, cfg.tau)
        loop = Loop(dec, cfg, plants)
        loop.run(warmup, graphs)
        torch.cuda.synchronize()
        s0, t0_tok = loop.steps, loop.tokens
        t0 = time.perf_counter()
        loop.run(steps, graphs)
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        n, tok = loop.steps - s0, loop.tokens - t0_tok
        log(f"[bench] sub-block {S}: {n / el:.1f} steps/s, {tok / el:.0f} tokens/s ({tok / n:.2f} tokens per step)")
        out[f"S{S}"] = {"steps_per_s": n / el, "tokens_per_s": tok / el, "tokens_per_step": tok / n}
        del dec, plants, loop
        torch.cuda.empty_cache()
    return {"subblock_sweep_7B": out}


def extras_proj(reps):
    """The projections of the refinement steps one call at a time, each after
    1 GiB of other reads has passed through the caches (as in a step, where
    the LM head's weight stream comes between two uses of a projection's
    weights): the 7B QKV and output projections at the 7B DualCache (64
    rows) and exact (256 rows) steps, and the 1.5B layer's four projections at
    the 28-layer decode's DualCache (128 rows) and exact (512 rows) steps.
    Beside each, the vendor GEMM (torch.matmul, hipBLASLt) of the same
    product without the epilogue, timed the same way: the reference rate of
    this part at these shapes."""
    from block_diffusion_decoding_amd import ops
    from block_diffusion_decoding_amd.ops import dense
    T = torch.bfloat16
    flush_src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    flush_dst = torch.empty(1 << 29, dtype=torch.uint8, device="cuda")

    def cold(fn):
        def run():
            flush_dst.copy_(flush_src[: 1 << 29])
            flush_dst.copy_(flush_src[1 << 29:])
            torch.cuda._sleep(20000)
        return time_call(fn, reps, warm_s=0.02, before=run)

    def rnd(*shape, s=1.0):
        return (torch.randn(*shape, device="cuda") * s).to(T)
    def vendor(xm, w):  # the same product as a plain vendor GEMM (torch.matmul -> hipBLASLt), no epilogue
        yv = torch.empty(xm.shape[0], w.shape[0], dtype=T, device="cuda")
        wt = w.t()
        return cold(lambda: torch.matmul(xm, wt, out=yv)).record()["us"]

    out = {}
    for M, K, Nq, Nkv, inter, tag in ((64, 3584, 3584, 512, None, "7B_M64"), (256, 3584, 3584, 512, None, "7B_M256"),
                                      (128, 1536, 1536, 256, 8960, "1.5B_M128"), (512, 1536, 1536, 256, 8960,
                                                                                  "1.5B_M512")):
        x, wq, wk, wv = rnd(M, K), rnd(Nq, K, s=.02), rnd(Nkv, K, s=.02), rnd(Nkv, K, s=.02)
        q, k, v = rnd(M, Nq), rnd(M, Nkv), rnd(M, Nkv)
        t = cold(lambda: ops.bd_qkv_proj(x, dense(M), wq, q, dense(M), wk, wv, k, dense(M), v, dense(M), M=M))
        by = (Nq + 2 * Nkv) * K * 2
        out[f"qkv_{tag}"] = {**t.record(), "weight_bytes": by, "GB/s": by / t.mean / 1e9,
                             "vendor_us": vendor(x, torch.cat([wq, wk, wv]))}
        wo, y = rnd(K, Nq, s=.02), rnd(M, K)
        t = cold(lambda: ops.bd_linear(q, dense(M), wo, y, dense(M), M=M, res=x, rr=dense(M)))
        by = K * Nq * 2
        out[f"o_{tag}"] = {**t.record(), "weight_bytes": by, "GB/s": by / t.mean / 1e9, "vendor_us": vendor(q, wo)}
        if inter:
            wgu, a = rnd(2 * inter, K, s=.02), rnd(M, inter)
            t = cold(lambda: ops.bd_gate_up_swiglu(x, dense(M), wgu, a, dense(M), M=M))
            by = 2 * inter * K * 2
            out[f"gate_up_{tag}"] = {**t.record(), "weight_bytes": by, "GB/s": by / t.mean / 1e9,
                                     "vendor_us": vendor(x, wgu)}
            wd = rnd(K, inter, s=.02)
            t = cold(lambda: ops.bd_linear(a, dense(M), wd, y, dense(M), M=M, res=y, rr=dense(M)))
            by = K * inter * 2
            out[f"down_{tag}"] = {**t.record(), "weight_bytes": by, "GB/s": by / t.mean / 1e9,
                                  "vendor_us": vendor(a, wd)}
    log("[bench] projections (cold caches; vendor GEMM of the same product): " +
        ", ".join(f"{k} {v['us']:.1f} us ({v['vendor_us']:.1f})" for k, v in out.items()))
    del flush_src, flush_dst
    torch.cuda.empty_cache()
    return {"projections": out}


def timed_loop(dec, cfg, plants, graphs, steps, warmup):
    """Steps/s and tokens/s of the lockstep loop over `plants` after `warmup`
    steps (window graphs replayed when `graphs`)."""
    loop = Loop(dec, cfg, plants)
    loop.run(warmup, graphs)
    torch.cuda.synchronize()
    s0, t0_tok, c0 = loop.steps, loop.tokens, loop.commits
    t0 = time.perf_counter()
    loop.run(steps, graphs)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    n, tok = loop.steps - s0, loop.tokens - t0_tok
    return {"steps": n, "steps_per_s": n / el, "tokens_per_s": tok / el, "tokens_per_step": tok / n,
            "ms_per_step": el / n * 1e3, "commits": loop.commits - c0}


def step_floor_bytes(cfg, kv_len) -> int:
    """Bytes a DualCache step must read once: LM head and projection weights
    and the batch's committed plus in-block K/V."""
    attn = int(sum((int(L) + cfg.D) * 2 * cfg.Hkv * cfg.d * 2 for L in kv_len))
    proj = (cfg.Hq * cfg.d + 2 * cfg.Hkv * cfg.d) * cfg.hidden * 2 + cfg.hidden * cfg.Hq * cfg.d * 2
    return cfg.V * cfg.hidden * 2 + proj + attn


def extras_rates(w3, graphs, rates=(0.0, 0.25, 0.5, 0.75, 1.0), steps=40, warmup=10):
    """The headline loop at planted pass rates 0 .. 1 of the masked rows: the
    threshold rule trades steps for tokens ("Fast-dLLM v2" notes, key findings
    on the threshold); at rate 0 every step unmasks only the fallback token."""
    cfg = bi.C3
    pre = bi.make_prefix(cfg, 0)
    dec = make_decoder(cfg, w3, pre)
    if graphs:
        dec.capture(cfg.S, cfg.tau)
    out = {}
    for r in rates:
        plants = block_plants(cfg, w3, r, 0, 8)
        rec = timed_loop(dec, cfg, plants, graphs, steps, warmup)
        dec.set_synthetic_prefix(pre.kv_len, pre.cache_k, pre.cache_v, pre.carry)   # same context for every rate
        log(f"[bench] pass rate {r}: {rec['steps_per_s']:.1f} steps/s, {rec['tokens_per_s']:.0f} tokens/s "
            f"({rec['tokens_per_step']:.2f} tokens per step)")
        out[f"r{r}"] = rec
        del plants
    del dec
    torch.cuda.empty_cache()
    return {"pass_rate_sweep_7B": out}


def extras_step_small(graphs, steps=60, warmup=10):
    """Whole refinement steps at the 1.5B shape (batch 1, one attention layer
    and the 1536 x 151936 LM head, prefix 2048, planted pass rate 0.5)."""
    cfg = bi.C2
    w2 = bi.make_weights(cfg, 0)
    pre = bi.make_prefix(cfg, 0)
    dec = make_decoder(cfg, w2, pre)
    if graphs:
        dec.capture(cfg.S, cfg.tau)
    rec = timed_loop(dec, cfg, block_plants(cfg, w2, 0.5, 0, 8), graphs, steps, warmup)
    fb = step_floor_bytes(cfg, pre.kv_len)
    rec.update({"bytes_per_dualcache_step": fb, "floor_us_at_peak": fb / (HBM_PEAK_GBS * 1e9) * 1e6,
                "frac_of_floor": fb / (HBM_PEAK_GBS * 1e9) / (rec["ms_per_step"] * 1e-3)})
    log(f"[bench] 1.5B-shape step loop: {rec['steps_per_s']:.1f} steps/s, {rec['tokens_per_s']:.0f} tokens/s, "
        f"{rec['ms_per_step'] * 1e3:.1f} us/step")
    del dec
    torch.cuda.empty_cache()
    return {"step_1.5B": rec}


def oracle_one_thread(n_steps=3):
    """The fp64 oracle on one host thread: DualCache steps (window 1) of the
    tiny fp32 workload and of the 1.5B-shape workload."""
    from threadpoolctl import threadpool_limits
    from oracle import refine as R
    out = {}
    for cfg in (bi.C1, bi.C2):
        w = bi.make_weights(cfg, 0)
        pre = bi.make_prefix(cfg, 0)
        st = bi.make_block_state(cfg, 0, 1)
        plant, carry_plant, _ = bi.make_plants(cfg, 0, w, st, 0.5)
        with threadpool_limits(limits=1):
            m = R.Model.from_weights(w, cfg)
            seqs = R.seqs_from_inputs(m, cfg, pre, st, plant, carry_plant)
            for q in seqs:
                R.e_step(m, q, 1, cfg.S, cfg.tau, cfg.D)
            times = []
            for _ in range(n_steps if cfg is bi.C2 else 10 * n_steps):
                for q, b in zip(seqs, range(cfg.B)):
                    q.tokens = st.tokens[b].astype(np.int64).copy()
                    q.masked = st.masked[b].copy()
                t0 = time.perf_counter()
                for q in seqs:
                    R.dc_step(m, q, 1, cfg.S, cfg.tau, cfg.D)
                times.append(time.perf_counter() - t0)
        sec = float(np.median(times))
        out[cfg.name] = {"steps_per_s": 1.0 / sec, "s_per_step_median": sec, "threads": 1, "steps": len(times)}
        log(f"[bench] oracle, one thread, {cfg.name}: {sec * 1e3:.1f} ms per DualCache step")
    return {"oracle_one_thread": out}


def extras_persequence(w3, n_blocks=4):
    """The headline workload (7B shape, planted pass rate 0.5) decoded block by
    block with per-sequence window progression (one captured mixed step per
    batched step; queued: the schedule on the device and the steps replayed
    back to back; host: the host schedules every step) against the lockstep
    loop (window graphs), same blocks."""
    from block_diffusion_decoding_amd.decoder import Dims
    from block_diffusion_decoding_amd.persequence import PerSequenceDecoder
    cfg = bi.C3
    pre = bi.make_prefix(cfg, 0)
    plants = block_plants(cfg, w3, 0.5, 0, n_blocks + 1)
    dims = Dims(cfg.B, cfg.Hq, cfg.Hkv, cfg.d, cfg.hidden, cfg.V, cfg.D, cfg.cap)
    weights = {k: torch.from_numpy(getattr(w3, k)) for k in ("E", "Wq", "Wk", "Wv", "Wo", "Wlm")}
    out = {}
    # per-sequence progression
    dec = PerSequenceDecoder(dims, weights, cfg.S, dtype=torch.bfloat16, device="cuda")
    dec.set_synthetic_prefix(pre.kv_len, pre.cache_k, pre.cache_v, pre.carry)
    dec.set_block(np.zeros((cfg.B, cfg.D), np.int32), np.ones((cfg.B, cfg.D), bool), plants[0])
    dec.capture_step(cfg.tau)
    dec.capture_step(cfg.tau, on_device=True)
    ctx = (dec.kv_len.clone(), dec.cache_k.clone(), dec.cache_v.clone(), dec.H[:, 0].clone())

    def run_ps(queued):
        dec.kv_len.copy_(ctx[0])
        dec.kv_len_host = ctx[0].cpu().numpy()
        dec.cache_k.copy_(ctx[1])
        dec.cache_v.copy_(ctx[2])
        dec.H[:, 0].copy_(ctx[3])
        decode = dec.decode_block_queued if queued else dec.decode_block
        dec.set_block(np.zeros((cfg.B, cfg.D), np.int32), np.ones((cfg.B, cfg.D), bool), plants[0])
        decode(cfg.tau)                           # warm-up block
        torch.cuda.synchronize()
        n = 0
        t0 = time.perf_counter()
        for k in range(n_blocks):
            dec.set_block(np.zeros((cfg.B, cfg.D), np.int32), np.ones((cfg.B, cfg.D), bool), plants[1 + k])
            n += decode(cfg.tau)
        torch.cuda.synchronize()
        return n, time.perf_counter() - t0
    steps_h, t_h = run_ps(False)
    steps, t_ps = run_ps(True)
    del dec, ctx
    torch.cuda.empty_cache()
    # lockstep (window graphs), the same blocks from the same context
    dec = make_decoder(cfg, w3, pre)
    dec.capture(cfg.S, cfg.tau)
    loop = Loop(dec, cfg, plants)

    def advance_to(blk):
        if dec.windows_complete(cfg.S):
            loop.pipelined(0, stop_blk=blk)
        while loop.blk < blk:
            if loop.first:
                loop.window()
            else:
                loop.step()
    advance_to(1)                                 # warm-up block
    torch.cuda.synchronize()
    s0 = loop.steps
    t0 = time.perf_counter()
    advance_to(1 + n_blocks)
    torch.cuda.synchronize()
    t_ls = time.perf_counter() - t0
    tokens = n_blocks * cfg.B * cfg.D
    out["per_sequence_7B"] = {"blocks": n_blocks, "tokens": tokens,
                              "per_sequence": {"steps": steps, "ms": t_ps * 1e3, "tokens_per_s": tokens / t_ps,
                                               "ms_per_step": t_ps / steps * 1e3, "schedule": "device, queued"},
                              "per_sequence_host_schedule": {"steps": steps_h, "ms": t_h * 1e3,
                                                             "tokens_per_s": tokens / t_h,
                                                             "ms_per_step": t_h / steps_h * 1e3},
                              "lockstep": {"steps": loop.steps - s0, "ms": t_ls * 1e3, "tokens_per_s": tokens / t_ls,
                                           "ms_per_step": t_ls / (loop.steps - s0) * 1e3}}
    log(f"[bench] per-sequence progression: {steps} steps, {tokens / t_ps:.0f} tokens/s queued "
        f"({tokens / t_h:.0f} with the host scheduling every step); lockstep "
        f"{loop.steps - s0} steps, {tokens / t_ls:.0f} tokens/s ({n_blocks} blocks)")
    del dec, loop
    torch.cuda.empty_cache()
    return out


def extras_v1():
    """v1-style decoding of a full-attention model (one 1.5B-shaped layer +
    the 1.5B head) with the block-wise DualCache, against the same decode
    with an exact full forward pass every step: 4 prompts of 256 ids, 256
    generated tokens in blocks of 32, tau 0.9, eager launches (the prefix and
    suffix lengths change every block)."""
    from block_diffusion_decoding_amd.v1 import FullAttnDecoder
    cfg = bi.T3
    B, P, gen = 4, 256, 256
    log(f"[bench] v1 full-attention decode: B {B}, prompt {P}, {gen} new tokens, {cfg.Hq}q/{cfg.Hkv}kv d{cfg.d}, "
        f"hidden {cfg.hidden}, vocab {cfg.V}")
    dev, dt = "cuda", torch.bfloat16
    g = torch.Generator(device=dev)
    g.manual_seed(9)

    def rnd(*shape):
        return (torch.randn(*shape, generator=g, device=dev, dtype=torch.float32) * cfg.std).to(dt)

    hq, hkv, hid = cfg.Hq * cfg.d, cfg.Hkv * cfg.d, cfg.hidden
    W = {"E": rnd(cfg.V + 1, hid), "Wq": rnd(hq, hid), "Wk": rnd(hkv, hid), "Wv": rnd(hkv, hid),
         "Wo": rnd(hid, hq), "Wlm": rnd(cfg.V, hid)}
    dec = FullAttnDecoder(W, B, P, gen, cfg.Hq, cfg.Hkv, cfg.d, cfg.D, dtype=dt, device=dev)
    del W
    prompts = bi.make_train_batch(replace(cfg, S=B, L=P), 9)[0]
    out = {}
    for mode in ("dual", "exact"):
        dec.generate(prompts[:, :P], 0.9, mode)          # warm-up pass
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        _, steps = dec.generate(prompts[:, :P], 0.9, mode)
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        log(f"[bench] v1 {mode}: {steps} steps in {el * 1e3:.1f} ms, {B * gen / el:.0f} tokens/s")
        out[mode] = {"steps": steps, "ms": el * 1e3, "tokens_per_s": B * gen / el}
    out["dual_speedup"] = out["exact"]["ms"] / out["dual"]["ms"]
    del dec
    torch.cuda.empty_cache()
    return {"v1_full_attention_1.5B_layer": out}


def extras(w3, reps, parts=("attn", "long", "lm", "proj", "e2e", "train", "subblock", "rates", "small", "persequence",
                            "v1"),
           graphs=True,
           e2e_blocks=None):
    """Attention and LM head alone at the long-context / batched shapes, the
    long-context block loop and the end-to-end multi-layer decode."""
    from block_diffusion_decoding_amd import ops
    out = {}
    T = torch.bfloat16
    c4 = bi.C4
    if "attn" in parts:
        out.update(extras_attn(c4, reps))
    if "long" in parts:
        out.update(extras_long(c4, w3, graphs))
    if "lm" in parts:
        out.update(extras_lm(w3, reps))
    if "proj" in parts:
        out.update(extras_proj(reps))
    if "e2e" in parts:
        out.update(extras_e2e(graphs, e2e_blocks))
    if "train" in parts:
        out.update(extras_train(reps))
    if "subblock" in parts:
        out.update(extras_subblock(w3, graphs))
    if "rates" in parts:
        out.update(extras_rates(w3, graphs))
    if "small" in parts:
        out.update(extras_step_small(graphs))
    if "persequence" in parts:
        out.update(extras_persequence(w3))
    if "v1" in parts:
        out.update(extras_v1())
    return out


def calibration_copy():
    """Plain device copy of CALIB_BYTES: what the HBM byte counters read for
    it calibrates them in a profiling run of a section."""
    src = torch.empty(CALIB_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def stored_traffic(kind: str):
    """Measured HBM bytes per launch from profiles/, while the kernel's
    sources still hash to the recorded value (else None)."""
    path = os.path.join(ROOT, "profiles", TRAFFIC[kind]["file"])
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_source_hash") != kernel_source_hash(kind):
        log(f"[bench] traffic record {TRAFFIC[kind]['file']} was measured on other sources of its kernels: "
            f"traffic reported as null (retake it with --traffic-from)")
        return None
    return rec.get("bytes_per_launch")


def extras_attn(c4, reps):
    from block_diffusion_decoding_amd import ops
    out = {}
    T = torch.bfloat16
    calibration_copy()
    # ---- attention, batch 32 x 16384 committed tokens
    log("[bench] long-context attention inputs")
    pre4 = bi.make_prefix(c4, 0)
    kc = torch.from_numpy(pre4.cache_k).to("cuda", T)
    vc = torch.from_numpy(pre4.cache_v).to("cuda", T)
    del pre4
    lens = torch.full((c4.B,), 16384, dtype=torch.int32, device="cuda")
    for n_q, name in ((8, "dualcache"), (32, "exact")):
        q = torch.randn(c4.B, n_q, c4.Hq, c4.d, device="cuda", dtype=T) * 0.02
        kb = torch.randn(c4.B, c4.D, c4.Hkv, c4.d, device="cuda", dtype=T) * 0.02
        vb = torch.randn_like(kb) * 0.02
        o = torch.empty_like(q)
        t = time_call(lambda: ops.bd_block_attn(q, kc, vc, lens, kb, vb, o, D=c4.D, q_off=0), reps)
        mean = t.mean
        nbytes = c4.B * (16384 + c4.D) * 2 * c4.Hkv * c4.d * 2 + 2 * c4.B * n_q * c4.Hq * c4.d * 2
        flops = 4 * c4.B * n_q * c4.Hq * c4.d * (16384 + c4.D)
        out[f"attn_long_{name}"] = {
            "shape": f"B=32 L=16384 n_q={n_q} Hq=28 Hkv=4 d=128 bf16", **t.record(),
            "bytes": nbytes, "GB/s": nbytes / mean / 1e9, "frac_hbm": nbytes / mean / 1e9 / HBM_PEAK_GBS,
            "TFLOP/s": flops / mean / 1e12, "traffic": stored_traffic(f"attn_{name}")}
        log(f"[bench] attention {name}: {mean * 1e6:.1f} us, {nbytes / mean / 1e9:.0f} GB/s")
    del kc, vc
    return out


def extras_long(c4, w3, graphs):
    out = {}
    # ---- fixed-schedule long-context block: 4 windows x 8 steps + commit
    log("[bench] long-context block loop")
    cfg4 = c4
    pre4 = bi.make_prefix(cfg4, 0)
    dec4 = make_decoder(cfg4, w3, pre4)
    del pre4
    if graphs:
        dec4.capture(cfg4.S, cfg4.tau)
    dec4.new_block()
    dec4.decode_block(cfg4.S, cfg4.tau, steps_per_window=8)          # warm-up block
    dec4.kv_len.fill_(16384)
    dec4.kv_len_host[:] = 16384
    dec4.new_block()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = dec4.decode_block(cfg4.S, cfg4.tau, steps_per_window=8)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    decoded = cfg4.B * cfg4.D - int(sum(bin(int(x)).count("1") for x in dec4.mask_bits.cpu().numpy().view(np.uint64)))
    out["long_block_loop"] = {"shape": "B=32 L=16384 block 32 sub-block 8, 8 steps/window + commit",
                              "ms": dt * 1e3, "steps": n, "decoded_tokens": decoded,
                              "tokens_per_s": decoded / dt, "steps_per_s": n / dt}
    log(f"[bench] long block: {dt * 1e3:.2f} ms, {decoded / dt:.0f} tokens/s")
    del dec4
    torch.cuda.empty_cache()
    return out


def extras_lm(w3, reps):
    from block_diffusion_decoding_amd import ops
    out = {}
    T = torch.bfloat16
    calibration_copy()
    # ---- vendor ceilings for streaming HBM traffic on this part: a 1 GiB
    # device copy (torch copy_, reads and writes 1 GiB) and a 1 GiB fp32 sum
    # (torch sum, reads 1 GiB): what a plain library streaming kernel reaches
    src = torch.empty(1 << 28, dtype=torch.float32, device="cuda").normal_()
    dst = torch.empty_like(src)
    tc = time_call(lambda: dst.copy_(src), reps)
    acc = torch.empty((), dtype=torch.float32, device="cuda")
    ts = time_call(lambda: torch.sum(src, dim=0, out=acc), reps)
    out["hbm_stream_ceiling"] = {
        "what": "vendor streaming kernels on 1 GiB: torch copy_ (1 GiB read + 1 GiB written) and torch.sum over "
                "fp32 (1 GiB read)",
        "copy_us": tc.mean * 1e6, "copy_GB/s": 2 * (1 << 30) / tc.mean / 1e9,
        "sum_us": ts.mean * 1e6, "sum_read_GB/s": (1 << 30) / ts.mean / 1e9,
        "frac_hbm_copy": 2 * (1 << 30) / tc.mean / 1e9 / HBM_PEAK_GBS,
        "frac_hbm_sum": (1 << 30) / ts.mean / 1e9 / HBM_PEAK_GBS}
    log(f"[bench] streaming ceilings: copy {2 * (1 << 30) / tc.mean / 1e9:.0f} GB/s, "
        f"sum {(1 << 30) / ts.mean / 1e9:.0f} GB/s")
    del src, dst
    # ---- LM head alone: 1024 rows on the 7B head (MFMA bound)
    Wlm = torch.from_numpy(w3.Wlm).to("cuda", T)
    for M, key in ((1024, "lmhead_7B_M1024"), (256, "lmhead_7B_M256"), (64, "lmhead_7B_M64")):
        h = torch.randn(M, 3584, device="cuda", dtype=T) * 0.05
        am = torch.empty(M, dtype=torch.int32, device="cuda")
        cf = torch.empty(M, dtype=torch.float32, device="cuda")
        t = time_call(lambda: ops.bd_lmhead_confidence(h, None, Wlm, am, cf), reps)
        mean = t.mean
        flops = 2.0 * M * 3584 * 152064
        nbytes = 152064 * 3584 * 2 + M * 3584 * 2 + 16 * M
        out[key] = {**t.record(), "TFLOP/s": flops / mean / 1e12,
                    "frac_mfma": flops / mean / 1e12 / BF16_PEAK_TFLOPS,
                    "GB/s": nbytes / mean / 1e9, "frac_hbm": nbytes / mean / 1e9 / HBM_PEAK_GBS}
        log(f"[bench] lm head M={M}: {mean * 1e6:.1f} us, {flops / mean / 1e12:.0f} TFLOP/s, "
            f"{nbytes / mean / 1e9:.0f} GB/s")
        if M == 1024:
            # the same product through the vendor GEMM (hipBLASLt via torch), logits
            # stored and no epilogue: a reference for the MFMA rate on this part
            y = torch.empty(M, 152064, device="cuda", dtype=T)
            tb = time_call(lambda: torch.matmul(h, Wlm.t(), out=y), reps)
            out["vendor_gemm_7B_M1024"] = {
                **tb.record(), "what": "torch.matmul(h [1024, 3584], Wlm^T) bf16 -> [1024, 152064] bf16 "
                                      "(hipBLASLt), the batched LM head's product without its epilogue",
                "TFLOP/s": flops / tb.mean / 1e12, "frac_mfma": flops / tb.mean / 1e12 / BF16_PEAK_TFLOPS}
            log(f"[bench] vendor GEMM M={M}: {tb.mean * 1e6:.1f} us, {flops / tb.mean / 1e12:.0f} TFLOP/s")
            # both on all-zero operands: the same instructions and memory traffic,
            # far less switching activity in the matrix units
            hz, Wz = torch.zeros_like(h), torch.zeros_like(Wlm)
            tz = time_call(lambda: ops.bd_lmhead_confidence(hz, None, Wz, am, cf), reps)
            tzb = time_call(lambda: torch.matmul(hz, Wz.t(), out=y), reps)
            out["lmhead_7B_M1024_zero_operands"] = {
                **tz.record(), "TFLOP/s": flops / tz.mean / 1e12, "frac_mfma": flops / tz.mean / 1e12 / BF16_PEAK_TFLOPS,
                "vendor_us": tzb.mean * 1e6,
                "vendor_TFLOP/s": flops / tzb.mean / 1e12,
                "what": "the 1024-row LM head and the vendor GEMM on all-zero h and W (same work, same bytes)"}
            log(f"[bench] zero operands M={M}: lm head {tz.mean * 1e6:.1f} us ({flops / tz.mean / 1e12:.0f} TFLOP/s), "
                f"vendor GEMM {tzb.mean * 1e6:.1f} us ({flops / tzb.mean / 1e12:.0f} TFLOP/s)")
            del y, hz, Wz
    # ---- the refinement step's call: the 64-row LM head fused with the
    # threshold unmask (8 sequences x window of 8); the window's mask bits are
    # restored before every call (one 64-byte device copy, timed with it), or
    # the calls would decode the window and then skip the LM head
    B, S, D = 8, 8, 32
    h = torch.randn(B * (1 + D), 3584, device="cuda", dtype=T) * 0.05
    ridx = torch.tensor([b * (1 + D) + 8 + r for b in range(B) for r in range(S)], dtype=torch.int32, device="cuda")
    am = torch.empty(B, S, dtype=torch.int32, device="cuda")
    cf = torch.empty(B, S, dtype=torch.float32, device="cuda")
    tok = torch.zeros(B, D, dtype=torch.int32, device="cuda")
    bits0 = torch.full((B,), -1, dtype=torch.int64, device="cuda")
    bits = bits0.clone()
    host = torch.zeros(B, dtype=torch.int64, pin_memory=True)

    def fused():
        bits.copy_(bits0)
        ops.bd_lmhead_unmask(h, ridx, Wlm, am, cf, tok, bits, win_lo=8, threshold=0.9, mask_bits_host=host)
    t = time_call(fused, reps)
    mean = t.mean
    nbytes = 152064 * 3584 * 2 + 64 * 3584 * 2 + 16 * 64
    out["lmhead_unmask_7B_B8_S8"] = {"us_with_bits_reset": mean * 1e6, **t.record(), "GB/s": nbytes / mean / 1e9,
                                     "frac_hbm": nbytes / mean / 1e9 / HBM_PEAK_GBS}
    log(f"[bench] lm head + unmask B=8 S=8: {mean * 1e6:.1f} us with the bits reset, {nbytes / mean / 1e9:.0f} GB/s")
    # ---- the 64-row LM head's load pattern alone (bd_probe_weight_stream: the
    # same global->LDS stages over the same weights, no arithmetic), with and
    # without the 64 rows of h per stage, at the LM head's 256 work-groups and
    # at 512: the floor of the load design, to set the LM head against
    h64 = torch.randn(64, 3584, device="cuda", dtype=T) * 0.05
    probe = {}
    for wgs in (256, 512):
        for with_x in (False, True):
            tp = time_call(lambda: ops.bd_probe_weight_stream(Wlm, h64 if with_x else None, work_groups=wgs), reps)
            probe[f"{'w_and_x' if with_x else 'w_only'}_{wgs}"] = {**tp.record(), "GB/s": Wlm.numel() * 2 / tp.mean / 1e9}
    out["lmhead_7B_M64_load_pattern"] = {**probe, "what": "bd_probe_weight_stream over the 7B head (1.09 GB): "
                                         "the streaming LM head's loads with no arithmetic; w_and_x adds its 64 "
                                         "rows of h to every stage"}
    log("[bench] lm head load pattern alone: " + ", ".join(f"{k} {v['us']:.1f} us" for k, v in probe.items()))
    del Wlm
    # ---- LM head alone: batch 1 on the 1.5B head (HBM bound)
    c2 = bi.C2
    W2 = torch.from_numpy(bi.normal(0, "Wlm", (c2.V, c2.hidden), 0.02, "bf16")).to("cuda", T)
    h = torch.randn(8, c2.hidden, device="cuda", dtype=T) * 0.05
    am = torch.empty(8, dtype=torch.int32, device="cuda")
    cf = torch.empty(8, dtype=torch.float32, device="cuda")
    t = time_call(lambda: ops.bd_lmhead_confidence(h, None, W2, am, cf), reps)
    mean = t.mean
    nbytes = c2.V * c2.hidden * 2 + 8 * c2.hidden * 2 + 16 * 8
    out["lmhead_1.5B_M8"] = {**t.record(), "GB/s": nbytes / mean / 1e9,
                             "frac_hbm": nbytes / mean / 1e9 / HBM_PEAK_GBS}
    log(f"[bench] lm head 1.5B M=8: {mean * 1e6:.1f} us, {nbytes / mean / 1e9:.0f} GB/s")
    return out


def cpu_baseline(cfg, w, pre, rate, n_steps):
    """fp64 oracle on the same seeded inputs: DualCache steps of window 1 of
    the same 8 sequences (the exact refresh step that builds the snapshot is
    not timed)."""
    from oracle import refine as R
    st = bi.make_block_state(cfg, 0, 1)
    plant, carry_plant, _ = bi.make_plants(cfg, 0, w, st, rate)
    m = R.Model.from_weights(w, cfg)
    seqs = R.seqs_from_inputs(m, cfg, pre, st, plant, carry_plant)
    for q in seqs:
        R.e_step(m, q, 1, cfg.S, cfg.tau, cfg.D)
    times = []
    for _ in range(n_steps):
        for q, b in zip(seqs, range(cfg.B)):
            q.tokens = st.tokens[b].astype(np.int64).copy()
            q.masked = st.masked[b].copy()
        t0 = time.perf_counter()
        for q in seqs:
            R.dc_step(m, q, 1, cfg.S, cfg.tau, cfg.D)
        times.append(time.perf_counter() - t0)
    sec = float(np.median(times))
    try:
        vendor = np.show_config(mode="dicts")["Build Dependencies"]["blas"]["name"]
    except Exception:  # pragma: no cover
        vendor = "unknown"
    return {"value": 1.0 / sec, "unit": "steps/s", "cores": _CORES, "kind": "oracle",
            "sample": f"{n_steps} DualCache refinement steps (window 1) of the same 8-sequence 7B-shape batch, "
                      f"fp64 NumPy ({vendor}), median {sec:.2f} s/step"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=60)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--rate", type=float, default=0.5, help="planted pass rate of masked rows")
    ap.add_argument("--reps", type=int, default=20, help="repetitions of the single-call measurements")
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--no-graphs", action="store_true", help="launch every step's kernels eagerly")
    ap.add_argument("--no-window-graphs", action="store_true",
                    help="replay one captured step at a time (a host wait after every step) instead of one "
                         "captured graph per window")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-steps", type=int, default=32,
                    help="DualCache steps of the oracle timed for cpu_baseline (about 10 s of host work)")
    ap.add_argument("--section", choices=("all", "attn", "long", "lm", "proj", "e2e", "train", "subblock", "rates",
                                          "small", "persequence", "v1", "oracle1"),
                    default="all", help="run only that measurement (for profiling) and print its JSON instead of the "
                                        "bench line (oracle1: the one-thread oracle, no GPU)")
    ap.add_argument("--e2e-blocks", type=int, default=None,
                    help="blocks generated by the end-to-end decode measurement (default: the workload's 16)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the traffic record of --traffic-kind (profiles/*_traffic.json) from two rocprofv3 "
                         "--pmc counter files of its section (FETCH_SIZE, WRITE_SIZE) and exit")
    ap.add_argument("--traffic-kind", choices=sorted(TRAFFIC), default="lm")
    args = ap.parse_args()
    if args.traffic_from:
        traffic_from(args.traffic_kind, *args.traffic_from)
        return
    if args.section == "oracle1":
        print(json.dumps(oracle_one_thread()), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: this implementation runs on a "
              "single GPU and has no multi-GPU path", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    import block_diffusion_decoding_amd as pkg
    pkg.load_library()

    cfg = bi.C3
    if args.section in ("e2e", "train", "v1", "small", "proj"):
        print(json.dumps(extras(None, args.reps, parts=(args.section,), graphs=not args.no_graphs,
                                e2e_blocks=args.e2e_blocks)), flush=True)
        return
    log("[bench] generating the 7B-shape workload")
    w = bi.make_weights(cfg, 0)
    if args.section != "all":
        print(json.dumps(extras(w, args.reps, parts=(args.section,), graphs=not args.no_graphs)), flush=True)
        return
    pre = bi.make_prefix(cfg, 0)
    n_blocks = 8
    dec = make_decoder(cfg, w, pre)
    plants = block_plants(cfg, w, args.rate, 0, n_blocks)
    if not args.no_graphs:
        dec.capture(cfg.S, cfg.tau)
    loop = Loop(dec, cfg, plants)
    windows = not args.no_graphs and not args.no_window_graphs
    loop.run(args.warmup, windows)
    torch.cuda.synchronize()
    # timed region: the headline loop (captured windows replayed as HIP graphs)
    s0, t0_tok, c0 = loop.steps, loop.tokens, loop.commits
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    loop.run(args.steps, windows)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    steps = loop.steps - s0
    tokens = loop.tokens - t0_tok
    steps_per_s = steps / elapsed
    log(f"[bench] {steps} steps in {elapsed * 1e3:.1f} ms: {steps_per_s:.1f} steps/s, "
        f"{tokens / elapsed:.0f} tokens/s, {loop.commits - c0} commits")
    # second pass of the same loop, steps launched one by one, with HIP events
    # around every LM-head launch (a kernel inside a graph replay cannot be
    # timed by events): the dominant kernel's launch durations
    timer = LaunchTimer()
    dec.lm_timer = timer
    torch.cuda.synchronize()
    for _ in range(args.steps):
        loop.step()
    torch.cuda.synchronize()
    lm_t = timer.seconds()
    dec.lm_timer = None
    log(f"[bench] LM head (bd_lmhead_unmask) {lm_t.mean() * 1e6:.1f} us mean, {np.median(lm_t) * 1e6:.1f} us median "
        f"over {len(lm_t)} launches of the loop")

    # roofline of the dominant kernel: LM head of the 7B step (B*S = 64 rows)
    M = cfg.B * cfg.S
    lm_bytes = cfg.V * cfg.hidden * 2 + M * cfg.hidden * 2 + 16 * M
    lm_mean = float(lm_t.mean())
    achieved = lm_bytes / lm_mean / 1e9
    traffic = stored_traffic("lm")
    # lockstep against a per-sequence window progression over the blocks the
    # loop finished (warm-up and timed): steps the batch took vs the most steps
    # any one sequence needed on its own schedule (what per-sequence progression
    # would take if a step mixing exact and DualCache rows cost the same)
    lock = sum(b[0] for b in loop.done_blocks)
    own = sum(b[1] for b in loop.done_blocks)
    progression = {"blocks": len(loop.done_blocks), "lockstep_steps": lock, "per_sequence_steps_bound": own,
                   "saving_bound": round(1 - own / lock, 4) if lock else None}
    # the whole DualCache step against HBM: every byte it must read once (LM head and projection
    # weights, the committed K/V of the batch at the loop's starting lengths plus the in-block rows)
    step_bytes = step_floor_bytes(cfg, pre.kv_len)
    floor_us = step_bytes / (HBM_PEAK_GBS * 1e9) * 1e6
    step_roofline = {"bound": "hbm", "bytes_per_dualcache_step": step_bytes, "floor_us_at_peak": round(floor_us, 1),
                     "us_per_step": round(elapsed / steps * 1e6, 1),
                     "frac": round(floor_us / (elapsed / steps * 1e6), 4),
                     "note": "LM head + QKV/O weights + the batch's K/V at the starting lengths, read once, "
                             "against the whole loop's time per step (exact steps, window ends and host waits "
                             "included)"}
    if windows:
        step_roofline["graphs"] = graph_costs(dec, cfg, plants[0])
        log(f"[bench] graphs: {json.dumps(step_roofline['graphs'])}")
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": "bd_lmhead_unmask (lm_stream_kernel<4, 4> + lm_merge_unmask_kernel: the LM head's final reduction "
                          "with the threshold unmask), 64 rows x 152064 x 3584",
                "algorithmic_bytes": lm_bytes, "launch_us_mean": round(lm_mean * 1e6, 2),
                "launch_us_median": round(float(np.median(lm_t)) * 1e6, 2),
                "timing": f"HIP events around each of {len(lm_t)} LM-head launches of a second pass of the same "
                          "loop (steps launched one by one) on the launch stream; a spin kernel before each start "
                          "event keeps the host ahead of the GPU, so no interval holds host launch time"}
    extra = {}
    if not args.no_extras:
        del dec
        torch.cuda.empty_cache()
        extra = extras(w, args.reps, e2e_blocks=args.e2e_blocks)
    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (fp64 oracle)")
        cpu = cpu_baseline(cfg, w, pre, args.rate, args.cpu_steps)
        log(f"[bench] oracle: {cpu['value']:.3f} steps/s on {cpu['cores']} cores")
        cpu.update(oracle_one_thread())
    line = {
        "metric": METRIC, "value": round(steps_per_s, 2), "unit": "steps/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(elapsed / steps * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "7B-shape refinement loop: 28q/4kv heads d128, hidden 3584, LM head 3584x152064, "
                               "batch 8, prefixes 1024-4096 (block-aligned), block 32, sub-block 8, tau 0.9, "
                               f"planted pass rate {args.rate}",
                   "global_batch": cfg.B, "block": cfg.D, "sub_block": cfg.S, "threshold": cfg.tau},
        "decoded_tokens_per_s": round(tokens / elapsed, 1),
        "tokens_per_step": round(tokens / steps, 3),
        "graphs": ("one per window" if windows else "one per step") if not args.no_graphs else None,
        "roofline": roofline,
        "step_roofline": step_roofline,
        "per_sequence_progression": progression,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
