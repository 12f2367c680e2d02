"""Seeded synthetic inputs for the block-diffusion refinement step.

This module is shared by the fp64 oracle (``oracle/``) and the HIP path
(``block_diffusion_decoding_amd``).  It holds workload shapes and random
draws only -- none of the method's arithmetic -- so that neither side has to
import the other.

Every array is drawn from ``numpy.random.PCG64``.  Large tensors are drawn in
fixed chunks of 2**22 elements; chunk ``c`` of tensor ``t`` for seed ``s``
uses the stream ``SeedSequence([s, t, c])``, so the values do not depend on
the number of threads used to draw them.  Floating-point values are
N(0, std^2) drawn in float32 and, for bf16 workloads, rounded to the nearest
bf16 (ties to even); they are stored as float32 arrays whose values are
exactly representable in the workload dtype, so both sides read identical
numbers (the oracle lifts them to float64 without rounding).

Shapes and value distributions follow the Qwen2.5-shaped configurations the
method was evaluated on ("Fast-dLLM v2: Efficient Block-Diffusion LLM"
notes, main-results table: Qwen2.5 1.5B / 7B Instruct adaptations; block
size 32 and sub-block size 8 from Key design 4; threshold 0.9 from Key
design 3).  The accuracy benchmarks the pages report on (GSM8K, HumanEval,
...) are not reproduced: random tokens and random-init weights stand in for
them.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

_CHUNK = 1 << 22

# Tensor ids: the second word of every SeedSequence, fixed forever so that a
# given (seed, tensor) pair always yields the same values.
TID = {
    "E": 1, "Wq": 2, "Wk": 3, "Wv": 4, "Wo": 5, "Wlm": 6,
    "lens": 10, "cache_k": 11, "cache_v": 12, "carry": 13,
    "prompt": 20, "committed": 21, "tokens": 22,
    "mask": 30, "plant": 40,
    # stand-alone operands for single-call tests
    "q": 50, "blk_k": 51, "blk_v": 52, "h": 53, "conf": 54,
    # multi-layer model (layer l uses tensor id base + 16 * l)
    "mE": 60, "mWlm": 61, "mprompt": 62, "x": 63, "pos": 64,
    "mWq": 1000, "mWk": 1001, "mWv": 1002, "mWo": 1003, "mWg": 1004, "mWu": 1005, "mWd": 1006,
    # training form
    "tx0": 70, "tmask": 71,
}
_LAYER_STRIDE = 16


# --------------------------------------------------------------------------
# workload configurations
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class Config:
    """One synthetic workload.

    B: batch; Hq/Hkv: query/KV heads; d: head dim; hidden = Hq*d; V: vocab
    (the [MASK] embedding is an extra row V that is never an LM-head class);
    D: block size; S: sub-block (window) size; tau: unmask threshold.
    prefix: 'prefill' (prompt + committed blocks computed by the model) or
    'synthetic' (random K/V cache rows).
    """
    name: str
    dtype: str              # 'f32' or 'bf16'
    B: int
    Hq: int
    Hkv: int
    d: int
    hidden: int
    V: int
    D: int = 32
    S: int = 8
    tau: float = 0.9
    std: float = 0.02
    prefix: str = "synthetic"
    # synthetic prefix: lengths L_b = D * U{len_lo_blocks..len_hi_blocks}
    len_lo_blocks: int = 0
    len_hi_blocks: int = 0
    cap: int = 0            # cache capacity (rows per sequence)
    # prefill prefix (tiny config): one 0-padded prompt block + committed blocks
    prompt_len: int = 0
    n_committed_blocks: int = 0
    # scale on the LM-head weights (tiny config: chosen so that ~30% of the
    # candidate rows pass the threshold)
    lm_scale: float = 1.0
    # planted peaked logits: offset gamma * Wlm[t] / |Wlm[t]|^2 on the row
    # that feeds a planted candidate
    plant_gamma: float = 30.0

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def np_dtype(self):
        return np.float32


# c1 lm_scale was chosen by tests/golden/make_tiny_scale.py, which runs the
# oracle on seed 0 (E-step and DC-step states) and picks the scale that puts
# ~30% of the candidate rows above the threshold with none within 2e-3 of it.
C1 = Config(name="c1", dtype="f32", B=1, Hq=4, Hkv=2, d=64, hidden=256,
            V=1024, prefix="prefill", prompt_len=20, n_committed_blocks=1,
            cap=192, lm_scale=1666.0)
C1_96 = replace(C1, name="c1-96", n_committed_blocks=2)
C2 = Config(name="c2", dtype="bf16", B=1, Hq=12, Hkv=2, d=128, hidden=1536,
            V=151936, len_lo_blocks=64, len_hi_blocks=64, cap=2048 + 32 * 8)
C3 = Config(name="c3", dtype="bf16", B=8, Hq=28, Hkv=4, d=128, hidden=3584,
            V=152064, len_lo_blocks=32, len_hi_blocks=128, cap=4096 + 32 * 8)
C4 = Config(name="c4", dtype="bf16", B=32, Hq=28, Hkv=4, d=128, hidden=3584,
            V=152064, len_lo_blocks=512, len_hi_blocks=512, cap=16384 + 32)

CONFIGS = {c.name: c for c in (C1, C1_96, C2, C3, C4)}


# --------------------------------------------------------------------------
# draws
# --------------------------------------------------------------------------
def _threads() -> int:
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:  # pragma: no cover
        return max(1, min(16, os.cpu_count() or 1))


def _rng(seed: int, tid: int, chunk: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tid, chunk])))


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round a float32 array in place to the nearest bf16 value (ties to even)."""
    assert x.dtype == np.float32
    u = x.view(np.uint32)
    flat = u.reshape(-1)
    for s in range(0, flat.size, _CHUNK):
        c = flat[s:s + _CHUNK]
        c += np.uint32(0x7FFF) + ((c >> np.uint32(16)) & np.uint32(1))
        c &= np.uint32(0xFFFF0000)
    return x


def normal(seed: int, name: str, shape, std: float, dtype: str, layer: int = 0) -> np.ndarray:
    """N(0, std^2) float32 array (bf16-representable when dtype == 'bf16');
    ``layer`` selects the draw of a per-layer tensor."""
    tid = TID[name] + _LAYER_STRIDE * layer
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    nchunks = (n + _CHUNK - 1) // _CHUNK

    def fill(c):
        sl = slice(c * _CHUNK, min(n, (c + 1) * _CHUNK))
        _rng(seed, tid, c).standard_normal(out=out[sl], dtype=np.float32)
        out[sl] *= np.float32(std)
        if dtype == "bf16":
            round_to_bf16(out[sl])

    if nchunks == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


def cast(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 copy of x, rounded to bf16 when dtype == 'bf16'."""
    y = np.array(x, dtype=np.float32, copy=True)
    return round_to_bf16(y) if dtype == "bf16" else y


@dataclass
class Weights:
    """One attention layer plus LM head, random-init N(0, std^2).

    E [V+1, hidden] (row V is the learnable [MASK] embedding), Wq [Hq*d,
    hidden], Wk/Wv [Hkv*d, hidden], Wo [hidden, Hq*d], Wlm [V, hidden]
    (out_features x in_features, row-major).
    """
    E: np.ndarray
    Wq: np.ndarray
    Wk: np.ndarray
    Wv: np.ndarray
    Wo: np.ndarray
    Wlm: np.ndarray


def make_weights(cfg: Config, seed: int) -> Weights:
    dt, s = cfg.dtype, cfg.std
    hq, hkv = cfg.Hq * cfg.d, cfg.Hkv * cfg.d
    E = normal(seed, "E", (cfg.V + 1, cfg.hidden), s, dt)
    Wq = normal(seed, "Wq", (hq, cfg.hidden), s, dt)
    Wk = normal(seed, "Wk", (hkv, cfg.hidden), s, dt)
    Wv = normal(seed, "Wv", (hkv, cfg.hidden), s, dt)
    Wo = normal(seed, "Wo", (cfg.hidden, hq), s, dt)
    Wlm = normal(seed, "Wlm", (cfg.V, cfg.hidden), s * cfg.lm_scale, dt)
    return Weights(E, Wq, Wk, Wv, Wo, Wlm)


@dataclass
class Prefix:
    """Context before the current block, per sequence.

    synthetic: kv_len [B], cache_k/cache_v [B, Hkv, cap, d] (rows >= kv_len
    are zero), carry [B, hidden] (hidden row of the last committed position).
    prefill: prompt [B, D] (0-padded on the left) and committed
    [B, n_committed_blocks * D] clean tokens; the cache and carry are then
    computed by the model.
    """
    kind: str
    kv_len: np.ndarray | None = None
    cache_k: np.ndarray | None = None
    cache_v: np.ndarray | None = None
    carry: np.ndarray | None = None
    prompt: np.ndarray | None = None
    committed: np.ndarray | None = None


def make_prefix(cfg: Config, seed: int) -> Prefix:
    B, D = cfg.B, cfg.D
    if cfg.prefix == "prefill":
        g = _rng(seed, TID["prompt"])
        prompt = np.zeros((B, D), dtype=np.int32)
        prompt[:, D - cfg.prompt_len:] = g.integers(0, cfg.V, size=(B, cfg.prompt_len))
        g = _rng(seed, TID["committed"])
        committed = g.integers(0, cfg.V, size=(B, cfg.n_committed_blocks * D)).astype(np.int32)
        return Prefix("prefill", prompt=prompt, committed=committed)
    g = _rng(seed, TID["lens"])
    nb = g.integers(cfg.len_lo_blocks, cfg.len_hi_blocks + 1, size=B)
    kv_len = (nb * D).astype(np.int32)
    assert kv_len.max() + D <= cfg.cap
    shape = (B, cfg.Hkv, cfg.cap, cfg.d)
    ck = normal(seed, "cache_k", shape, cfg.std, cfg.dtype)
    cv = normal(seed, "cache_v", shape, cfg.std, cfg.dtype)
    for b in range(B):
        ck[b, :, kv_len[b]:, :] = 0.0
        cv[b, :, kv_len[b]:, :] = 0.0
    carry = normal(seed, "carry", (B, cfg.hidden), cfg.std, cfg.dtype)
    return Prefix("synthetic", kv_len=kv_len, cache_k=ck, cache_v=cv, carry=carry)


@dataclass
class BlockState:
    """Token state of the current block.

    tokens [B, D] int32 (ids of unmasked positions; masked ids are 0),
    masked [B, D] bool, window: active sub-block index s (positions
    [s*S, (s+1)*S)), S: window length (S == D is exact mode).
    """
    tokens: np.ndarray
    masked: np.ndarray
    window: int
    S: int


def make_block_state(cfg: Config, seed: int, window: int, S: int | None = None,
                     n_masked: int | None = None, density: float | None = 0.5,
                     all_masked: bool = False) -> BlockState:
    """Block state at the start of a refinement step in window ``window``.

    Windows before it are decoded (uniform random tokens), windows after it
    are all [MASK].  Inside the window either exactly ``n_masked`` random
    positions or Bernoulli(density) positions (redrawn until one is masked)
    are masked.  ``all_masked`` gives a fresh block.
    """
    B, D = cfg.B, cfg.D
    S = cfg.S if S is None else S
    g = _rng(seed, TID["tokens"])
    tokens = g.integers(0, cfg.V, size=(B, D)).astype(np.int32)
    masked = np.zeros((B, D), dtype=bool)
    if all_masked:
        masked[:] = True
    else:
        lo, hi = window * S, (window + 1) * S
        masked[:, hi:] = True
        gm = _rng(seed, TID["mask"])
        for b in range(B):
            if n_masked is not None:
                pos = gm.choice(S, size=n_masked, replace=False)
                masked[b, lo + pos] = True
            else:
                while True:
                    m = gm.random(S) < density
                    if m.any():
                        break
                masked[b, lo:hi] = m
    tokens[masked] = 0
    return BlockState(tokens, masked, window, S)


def make_plants(cfg: Config, seed: int, wts: Weights, state: BlockState, rate: float,
                carry: np.ndarray | None = None):
    """Planted peaked logits for a controlled pass rate.

    For a seeded fraction ``rate`` of each sequence's candidate rows (masked
    positions of the active window), add gamma * Wlm[t] / |Wlm[t]|^2 (t
    uniform in [0, V)) to the input row that feeds the candidate: row j-1 of
    the block, or, for j == 0, the carry row.  The target logit then rises by
    about gamma, well above the log(9 V) needed for a confidence above 0.9.

    Returns (plant [B, D, hidden] float32 offsets for the block rows,
    carry_plant [B, hidden], planted [B, D] bool marking planted candidates).
    Offsets are rounded to the workload dtype.
    """
    B, D, S = cfg.B, cfg.D, state.S
    plant = np.zeros((B, D, cfg.hidden), dtype=np.float32)
    carry_plant = np.zeros((B, cfg.hidden), dtype=np.float32)
    planted = np.zeros((B, D), dtype=bool)
    g = _rng(seed, TID["plant"])
    lo = state.window * S
    for b in range(B):
        cand = [j for j in range(lo, lo + S) if state.masked[b, j]]
        k = int(round(rate * len(cand)))
        chosen = g.permutation(len(cand))[:k]
        for ci in sorted(chosen):
            j = cand[ci]
            t = int(g.integers(0, cfg.V))
            w = wts.Wlm[t].astype(np.float64)
            off = cfg.plant_gamma * w / float(w @ w)
            planted[b, j] = True
            if j == 0:
                carry_plant[b] += off.astype(np.float32)
            else:
                plant[b, j - 1] += off.astype(np.float32)
    if cfg.dtype == "bf16":
        round_to_bf16(plant)
        round_to_bf16(carry_plant)
    return plant, carry_plant, planted


def mask_bits(masked: np.ndarray) -> np.ndarray:
    """[B, D] bool -> [B] uint64 with bit j set when position j is [MASK]."""
    B, D = masked.shape
    assert D <= 64
    w = np.zeros(B, dtype=np.uint64)
    for j in range(D):
        w |= masked[:, j].astype(np.uint64) << np.uint64(j)
    return w


def bits_to_mask(bits: np.ndarray, D: int) -> np.ndarray:
    bits = np.asarray(bits, dtype=np.uint64)
    return np.stack([(bits >> np.uint64(j)) & np.uint64(1) for j in range(D)], axis=1).astype(bool)


# --------------------------------------------------------------------------
# multi-layer model (end-to-end decode)
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class ModelConfig:
    """A random-init Qwen2.5-shaped decoder for the end-to-end decode.

    n_layers layers of hidden size Hq*d with GQA (Hq/Hkv heads of dim d) and
    a SwiGLU MLP of width inter; vocab V (+ the [MASK] row of E).  B prompts
    of prompt_len uniform token ids (a whole number of blocks), n_blocks
    blocks of D generated in windows of S, threshold tau.  RMSNorm eps and
    RoPE theta are the Qwen2.5 family's (the pages do not give them; any
    values are valid for random weights).  cap = cache rows per sequence.
    lm_scale scales the LM-head weights (tiny configs: so that some
    candidates pass the threshold).
    """
    name: str
    dtype: str
    B: int
    n_layers: int
    Hq: int
    Hkv: int
    d: int
    hidden: int
    inter: int
    V: int
    prompt_len: int
    n_blocks: int
    D: int = 32
    S: int = 8
    tau: float = 0.9
    std: float = 0.02
    eps: float = 1e-6
    theta: float = 1e6
    lm_scale: float = 1.0

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def cap(self) -> int:
        return self.prompt_len + self.n_blocks * self.D


# end-to-end Qwen2.5-1.5B shape: 16 prompts of 512 ids, 512 new tokens
C5 = ModelConfig(name="c5", dtype="bf16", B=16, n_layers=28, Hq=12, Hkv=2, d=128, hidden=1536,
                 inter=8960, V=151936, prompt_len=512, n_blocks=16)
# small models the oracle runs in seconds (tests)
M1 = ModelConfig(name="m1", dtype="f32", B=2, n_layers=2, Hq=4, Hkv=2, d=64, hidden=256, inter=512,
                 V=1024, prompt_len=64, n_blocks=2, lm_scale=100.0)
M2 = ModelConfig(name="m2", dtype="bf16", B=2, n_layers=2, Hq=4, Hkv=2, d=128, hidden=512, inter=768,
                 V=2048, prompt_len=64, n_blocks=1, lm_scale=100.0)
MODEL_CONFIGS = {c.name: c for c in (C5, M1, M2)}


@dataclass
class LayerWeights:
    """Wq [Hq*d, hid], Wk/Wv [Hkv*d, hid], Wo [hid, Hq*d], Wg/Wu [inter,
    hid], Wd [hid, inter] (out x in, row-major)."""
    Wq: np.ndarray
    Wk: np.ndarray
    Wv: np.ndarray
    Wo: np.ndarray
    Wg: np.ndarray
    Wu: np.ndarray
    Wd: np.ndarray


@dataclass
class ModelWeights:
    E: np.ndarray
    layers: list
    Wlm: np.ndarray


def make_model_weights(cfg: ModelConfig, seed: int) -> ModelWeights:
    dt, s = cfg.dtype, cfg.std
    hq, hkv, hid, I = cfg.Hq * cfg.d, cfg.Hkv * cfg.d, cfg.hidden, cfg.inter
    E = normal(seed, "mE", (cfg.V + 1, hid), s, dt)
    layers = []
    for l in range(cfg.n_layers):
        layers.append(LayerWeights(
            normal(seed, "mWq", (hq, hid), s, dt, l), normal(seed, "mWk", (hkv, hid), s, dt, l),
            normal(seed, "mWv", (hkv, hid), s, dt, l), normal(seed, "mWo", (hid, hq), s, dt, l),
            normal(seed, "mWg", (I, hid), s, dt, l), normal(seed, "mWu", (I, hid), s, dt, l),
            normal(seed, "mWd", (hid, I), s, dt, l)))
    Wlm = normal(seed, "mWlm", (cfg.V, hid), s * cfg.lm_scale, dt)
    return ModelWeights(E, layers, Wlm)


def make_prompts(cfg: ModelConfig, seed: int) -> np.ndarray:
    """[B, prompt_len] int32 uniform token ids."""
    return _rng(seed, TID["mprompt"]).integers(0, cfg.V, size=(cfg.B, cfg.prompt_len)).astype(np.int32)


# --------------------------------------------------------------------------
# training form (forward pass and loss value of the 2L layout)
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class TrainConfig:
    """A batch of S training sequences of L tokens for the one-layer model
    (fields as Config); each sample also enters in its complementary view,
    so 2S sequences of 2L rows are attended.  mask_p: probability that a
    position is masked in the first view."""
    name: str
    dtype: str
    S: int
    L: int
    Hq: int
    Hkv: int
    d: int
    hidden: int
    V: int
    D: int = 32
    mask_p: float = 0.5
    std: float = 0.02
    lm_scale: float = 1.0

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv


# small cases the oracle runs in seconds (tests; lm_scale makes the logits
# O(1) so that a wrong source row or target changes the loss visibly) and
# the 1.5B-shaped layer the benchmark times (L 2048, 4 samples = 8 views)
T1 = TrainConfig(name="t1", dtype="f32", S=2, L=96, Hq=4, Hkv=2, d=64, hidden=256, V=1024, lm_scale=300.0)
T2 = TrainConfig(name="t2", dtype="bf16", S=2, L=128, Hq=12, Hkv=2, d=128, hidden=1536, V=4096, lm_scale=100.0)
T3 = TrainConfig(name="t3", dtype="bf16", S=4, L=2048, Hq=12, Hkv=2, d=128, hidden=1536, V=151936)
TRAIN_CONFIGS = {c.name: c for c in (T1, T2, T3)}


def make_train_batch(cfg: TrainConfig, seed: int):
    """x0 [S, L] int32 uniform token ids; m [S, L] bool, Bernoulli(mask_p):
    the first view's mask (the second view masks the complement)."""
    x0 = _rng(seed, TID["tx0"]).integers(0, cfg.V, size=(cfg.S, cfg.L)).astype(np.int32)
    m = _rng(seed, TID["tmask"]).random((cfg.S, cfg.L)) < cfg.mask_p
    return x0, m
