"""GPU parity of v1-style decoding of a full-attention model with the
block-wise DualCache (block_diffusion_decoding_amd/v1.py) against the oracle
(oracle/v1.py): whole generations, step by step with teacher forcing (after
each step the GPU block state is set to the oracle's decisions)."""
import numpy as np
import pytest
import torch

import bd_inputs as bi
from gpu_util import DEV, TOL, lm_stats_close, say, tdt, unmask_close
from oracle import refine as R
from oracle import v1 as V1

pytestmark = pytest.mark.gpu

CASES = {"tiny-f32": (bi.T1, 2, 32, 96), "1.5B-layer-bf16": (bi.T2, 2, 64, 64)}


@pytest.mark.parametrize("case,mode", [("tiny-f32", "dual"), ("tiny-f32", "exact"), ("1.5B-layer-bf16", "dual")])
def test_v1_generation_teacher_forced(case, mode):
    cfg, B, P, gen = CASES[case]
    say(f"[v1] {case} {mode}")
    from block_diffusion_decoding_amd.v1 import FullAttnDecoder
    w = bi.make_weights(cfg, 11)
    model = R.Model.from_weights(w, cfg)
    prompts = bi.make_train_batch(cfg, 11)[0][:B, :P]
    D, tau, rtol = cfg.D, 0.9, TOL[cfg.dtype]
    dec = FullAttnDecoder({k: torch.from_numpy(getattr(w, k)) for k in ("E", "Wq", "Wk", "Wv", "Wo", "Wlm")},
                          B, P, gen, cfg.Hq, cfg.Hkv, cfg.d, D, dtype=tdt(cfg.dtype), device=DEV)
    dec.set_prompts(prompts)
    seqs = [V1.new_sequence(prompts[b], gen) for b in range(B)]
    n_steps, passes = 0, 0
    for k in range(gen // D):
        lo = P + k * D
        dec.begin_block(k)
        first = True
        while any(q.masked[lo:lo + D].any() for q in seqs):
            kind = "E" if (first or mode == "exact") else "DC"
            before = np.stack([q.masked[lo:lo + D] for q in seqs])
            res = [(V1.exact_step(model, q, k, D, tau) if kind == "E" else V1.dual_step(model, q, k, D, tau))
                   for q in seqs]
            (dec.exact_step(tau) if kind == "E" else dec.dual_step(tau))
            torch.cuda.synchronize()
            what = f"block {k} step {n_steps} {kind}"
            am, cf = dec.argmax.cpu().numpy(), dec.conf.cpu().numpy()
            mx, lse = dec.max_logit.cpu().numpy(), dec.lse.cpu().numpy()
            for b, r in enumerate(res):
                lm_stats_close(am[b], cf[b], mx[b], lse[b], R.lm_logits(model.Wlm, r.src), rtol, f"{what} seq {b}")
            got = ((dec.mask_bits_host()[:, None] >> np.arange(D, dtype=np.uint64)) & np.uint64(1)).astype(bool)
            ref = np.stack([q.masked[lo:lo + D] for q in seqs])
            unmask_close(got, ref, before, [r.conf for r in res], 0, tau, rtol, what, got_conf_win=cf)
            passes += int((before & ~ref).sum())
            # teacher forcing: the oracle's block state
            dec.tok_blk.copy_(torch.from_numpy(np.stack([q.tokens[lo:lo + D] for q in seqs]).astype(np.int32)))
            bits = (ref.astype(np.uint64) << np.arange(D, dtype=np.uint64)).sum(axis=1)
            dec.bits_blk.copy_(torch.from_numpy(bits.astype(np.uint64).view(np.int64)))
            first = False
            n_steps += 1
    say(f"    {n_steps} steps, {passes} tokens")
    assert passes == B * gen
    got_tokens = dec.tokens_host()
    for b, q in enumerate(seqs):
        assert np.array_equal(got_tokens[b], q.tokens.astype(np.int32))


def test_whole_sequence_attention_at_the_benchmark_shape_sampled():
    """The refresh pass of the v1 benchmark (4 sequences of 512 positions,
    12q/2kv heads d 128: one block spanning the sequence, no cache) on sampled
    (sequence, row, head) outputs computed one by one in fp64 over all keys."""
    from block_diffusion_decoding_amd import ops
    say("[v1] whole-sequence attention, sampled")
    B, T, Hq, Hkv, d = 4, 512, 12, 2, 128
    g = torch.Generator(device=DEV)
    g.manual_seed(22)
    q = torch.randn(B, T, Hq, d, generator=g, device=DEV).to(torch.bfloat16)
    k = torch.randn(B, T, Hkv, d, generator=g, device=DEV).to(torch.bfloat16)
    v = torch.randn(B, T, Hkv, d, generator=g, device=DEV).to(torch.bfloat16)
    out = torch.zeros_like(q)
    ops.bd_block_attn(q, None, None, torch.zeros(B, dtype=torch.int32, device=DEV), k, v, out, D=T, q_off=0)
    torch.cuda.synchronize()
    rng = np.random.default_rng(22)
    for s, p, h in [(int(rng.integers(B)), int(rng.integers(T)), int(rng.integers(Hq))) for _ in range(32)]:
        kvh = h // (Hq // Hkv)
        qv = q[s, p, h].float().cpu().numpy().astype(np.float64)
        K = k[s, :, kvh].float().cpu().numpy().astype(np.float64)
        V = v[s, :, kvh].float().cpu().numpy().astype(np.float64)
        sc = K @ qv / np.sqrt(d)
        pr = np.exp(sc - sc.max())
        ref = (pr / pr.sum()) @ V
        got = out[s, p, h].float().cpu().numpy().astype(np.float64)
        err = np.linalg.norm(got - ref) / np.linalg.norm(ref)
        assert err <= TOL["bf16"], f"sequence {s} row {p} head {h}: rel err {err:.3g}"
