// C-ABI entry points of libbd (declared in include/bd.h): argument checks on
// the host, workspace carving, then the launchers of the kernel files.
#include <cstdint>

#include "bd_launch.h"

namespace {

thread_local int g_last_hip_error = 0;

bd_status hip_status(hipError_t e) { return bd_hip_status(e); }

bool valid_dtype(bd_dtype dt) { return dt == BD_F32 || dt == BD_BF16; }

bool valid_rows(const bd_rows& r) { return r.group >= 1 && r.stride >= 0 && r.offset >= 0; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// A guard is optional; when given its words must be there and aligned.
bool valid_guard(const bd_guard* g) {
  return g == nullptr || (g->bits != nullptr && (reinterpret_cast<uintptr_t>(g->bits) & 7u) == 0 && g->n >= 1 &&
                          g->n <= 4096);
}

}  // namespace

bd_status bd_hip_status(hipError_t e) {
  if (e == hipSuccess) return BD_OK;
  g_last_hip_error = static_cast<int>(e);
  return BD_EHIP;
}

bd_status bd_block_attn_check(bd_dtype dt, int B, int Hq, int Hkv, int d, int D, const void* q, int n_q, int q_off,
                              const void* k_cache, const void* v_cache, const int32_t* kv_len, int cap,
                              const void* k_blk, const void* v_blk, int n_blk, float scale, const void* o) {
  if (!valid_dtype(dt) || B < 0 || n_q < 0) return BD_EINVAL;
  if (B == 0 || n_q == 0) return BD_OK;
  if (Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || D < 1 || n_blk < 1 || n_blk % D != 0 || q_off < 0 ||
      q_off + n_q > n_blk || cap < 0)
    return BD_EINVAL;
  if (d != 64 && d != 128) return BD_EUNSUPPORTED;
  if (!q || !kv_len || !k_blk || !v_blk || !o || (cap > 0 && (!k_cache || !v_cache))) return BD_EINVAL;
  if (!aligned16(q) || !aligned16(k_blk) || !aligned16(v_blk) || !aligned16(o) ||
      (cap > 0 && (!aligned16(k_cache) || !aligned16(v_cache))))
    return BD_EINVAL;
  if (!(scale == scale)) return BD_EINVAL;
  return BD_OK;
}

extern "C" {

const char* bd_version(void) { return "libbd 0.1 (gfx950)"; }

const char* bd_status_string(bd_status s) {
  switch (s) {
    case BD_OK: return "ok";
    case BD_EINVAL: return "invalid argument";
    case BD_EUNSUPPORTED: return "unsupported";
    case BD_ECAPACITY: return "cache capacity exceeded";
    case BD_EHIP: return "HIP runtime error";
    case BD_ESCRATCH: return "needs more scratch than the library's static buffer holds";
  }
  return "unknown status";
}

int bd_last_hip_error(void) { return g_last_hip_error; }

// ---------------------------------------------------------------------------
size_t bd_block_attn_workspace_size(bd_dtype dt, int B, int Hq, int Hkv, int d, int n_q, int cap, int n_blk) {
  if (!valid_dtype(dt) || B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || n_q <= 0 || cap < 0 || n_blk <= 0)
    return 0;
  return bd_attn_plan(dt, B, Hq, Hkv, d, n_q, cap, n_blk).ws_bytes;
}

bd_status bd_block_attn(bd_dtype dt, int B, int Hq, int Hkv, int d, int D, const void* q, int n_q, int q_off,
                        const void* k_cache, const void* v_cache, const int32_t* kv_len, int cap,
                        const void* k_blk, const void* v_blk, int n_blk, float scale, void* o, float* lse,
                        void* workspace, size_t ws_bytes, void* stream) {
  return bd_block_attn_guarded(dt, B, Hq, Hkv, d, D, q, n_q, q_off, k_cache, v_cache, kv_len, cap, k_blk, v_blk,
                               n_blk, scale, o, lse, workspace, ws_bytes, nullptr, stream);
}

bd_status bd_block_attn_guarded(bd_dtype dt, int B, int Hq, int Hkv, int d, int D, const void* q, int n_q,
                                int q_off, const void* k_cache, const void* v_cache, const int32_t* kv_len, int cap,
                                const void* k_blk, const void* v_blk, int n_blk, float scale, void* o, float* lse,
                                void* workspace, size_t ws_bytes, const bd_guard* guard, void* stream) {
  if (!valid_guard(guard)) return BD_EINVAL;
  const bd_status chk = bd_block_attn_check(dt, B, Hq, Hkv, d, D, q, n_q, q_off, k_cache, v_cache, kv_len, cap,
                                            k_blk, v_blk, n_blk, scale, o);
  if (chk != BD_OK || B == 0 || n_q == 0) return chk;
  const BdAttnPlan p = bd_attn_plan(dt, B, Hq, Hkv, d, n_q, cap, n_blk);
  if (p.ws_bytes > 0 && (workspace == nullptr || ws_bytes < p.ws_bytes || !aligned16(workspace)))
    return BD_EINVAL;
  BdAttnArgs a{};
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.kv_len = kv_len;
  a.k_blk = k_blk;
  a.v_blk = v_blk;
  a.o = o;
  a.lse = lse;
  a.part_o = p.ws_bytes ? reinterpret_cast<float*>(static_cast<char*>(workspace) + p.part_o) : nullptr;
  a.part_ml = p.ws_bytes ? reinterpret_cast<float*>(static_cast<char*>(workspace) + p.part_ml) : nullptr;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = Hq / Hkv;
  a.d = d;
  a.D = D;
  a.n_q = n_q;
  a.q_off = q_off;
  a.cap = cap;
  a.n_blk = n_blk;
  a.epc = 1;
  a.scale = scale;
  a.guard = guard;
  return hip_status(bd_attn_launch(dt, p, a, static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------------------
size_t bd_lmhead_workspace_size(bd_dtype dt, int M, int hidden, int V) {
  if (!valid_dtype(dt) || M <= 0 || hidden <= 0 || V <= 0) return 0;
  return bd_lm_plan(dt, M, hidden, V).ws_bytes;
}

static bd_status lm_common(bd_dtype dt, int M, int hidden, int V, const void* h_src, int n_src,
                           const int32_t* row_idx, const int32_t* out_pos, const int32_t* m_dev, int n_out,
                           const void* w, int32_t* argmax, float* conf, float* max_logit, float* lse, float* logits,
                           void* workspace, size_t ws_bytes, void* stream, const BdLmUnmask* um = nullptr) {
  if (!valid_dtype(dt) || M < 0) return BD_EINVAL;
  if (M == 0) return BD_OK;
  if (hidden <= 0 || V <= 0 || n_src <= 0 || !h_src || !w || !argmax || !conf) return BD_EINVAL;
  if (row_idx == nullptr && n_src < M) return BD_EINVAL;
  if (dt == BD_BF16 && (hidden % 256 != 0 || !aligned16(h_src) || !aligned16(w))) return BD_EUNSUPPORTED;
  const BdLmPlan p = bd_lm_plan(dt, M, hidden, V);
  if (workspace == nullptr || ws_bytes < p.ws_bytes || !aligned16(workspace)) return BD_EINVAL;
  const size_t n = (size_t)M * p.nvt;
  BdLmArgs a{};
  a.h = h_src;
  a.n_src = n_src;
  a.row_idx = row_idx;
  a.w = w;
  a.argmax = argmax;
  a.conf = conf;
  a.max_logit = max_logit;
  a.lse = lse;
  a.logits = logits;
  a.M = M;
  a.hidden = hidden;
  a.V = V;
  a.pmax = static_cast<float*>(workspace);
  a.psum = a.pmax + n;
  a.pidx = reinterpret_cast<int32_t*>(a.psum + n);
  a.m_dev = m_dev;
  a.out_pos = out_pos;
  a.n_out = n_out;
  return hip_status(bd_lm_launch(dt, p, a, static_cast<hipStream_t>(stream), um));
}

bd_status bd_lmhead_confidence(bd_dtype dt, int M, int hidden, int V, const void* h_src, int n_src,
                               const int32_t* row_idx, const void* w, int32_t* argmax, float* conf,
                               float* max_logit, float* lse, float* logits, void* workspace, size_t ws_bytes,
                               void* stream) {
  return lm_common(dt, M, hidden, V, h_src, n_src, row_idx, nullptr, nullptr, 0, w, argmax, conf, max_logit, lse,
                   logits, workspace, ws_bytes, stream);
}

bd_status bd_lmhead_unmask_next(bd_dtype dt, int B, int D, int win_lo, int win_len, int hidden, int V,
                                const void* h_src, int n_src, const int32_t* row_idx, const void* w, float threshold,
                                const float* threshold_dev, int32_t* argmax, float* conf, float* max_logit, float* lse,
                                int32_t* tokens, uint64_t* mask_bits, int32_t* n_unmasked, int32_t* unmasked_pos,
                                uint64_t* mask_bits_host, const bd_next_rows* next, void* workspace,
                                size_t ws_bytes, void* stream) {
  if (B < 0) return BD_EINVAL;
  if (B == 0) return BD_OK;
  if (D < 1 || D > 64 || win_lo < 0 || win_len < 1 || win_len > 64 || win_lo + win_len > D) return BD_EINVAL;
  if ((long)B * win_len > 64 || !tokens || !mask_bits) return BD_EINVAL;
  if (threshold_dev == nullptr && !(threshold == threshold)) return BD_EINVAL;
  BdLmUnmask um{B, D, win_lo, win_len, threshold, threshold_dev, tokens, mask_bits, n_unmasked, unmasked_pos,
                mask_bits_host, nullptr, nullptr, nullptr, 0, 0, 0};
  if (next != nullptr) {
    if (!valid_dtype(dt) || !next->embedding || !next->x) return BD_EINVAL;
    if (hidden % (dt == BD_BF16 ? 8 : 4) != 0 || !aligned16(next->embedding) || !aligned16(next->x) ||
        (next->plant && !aligned16(next->plant)))
      return BD_EUNSUPPORTED;
    um.emb = next->embedding;
    um.plant = next->plant;
    um.x = next->x;
    um.hidden = hidden;
    um.V = V;
    um.f32 = dt == BD_F32 ? 1 : 0;
  }
  return lm_common(dt, B * win_len, hidden, V, h_src, n_src, row_idx, nullptr, nullptr, 0, w, argmax, conf,
                   max_logit, lse, nullptr, workspace, ws_bytes, stream, &um);
}

bd_status bd_lmhead_unmask(bd_dtype dt, int B, int D, int win_lo, int win_len, int hidden, int V, const void* h_src,
                           int n_src, const int32_t* row_idx, const void* w, float threshold,
                           const float* threshold_dev, int32_t* argmax, float* conf, float* max_logit, float* lse,
                           int32_t* tokens, uint64_t* mask_bits, int32_t* n_unmasked, int32_t* unmasked_pos,
                           uint64_t* mask_bits_host, void* workspace, size_t ws_bytes, void* stream) {
  return bd_lmhead_unmask_next(dt, B, D, win_lo, win_len, hidden, V, h_src, n_src, row_idx, w, threshold,
                               threshold_dev, argmax, conf, max_logit, lse, tokens, mask_bits, n_unmasked,
                               unmasked_pos, mask_bits_host, nullptr, workspace, ws_bytes, stream);
}

bd_status bd_lmhead_confidence_rows(bd_dtype dt, int M, int hidden, int V, const void* h_src, int n_src,
                                    const int32_t* row_idx, const int32_t* out_pos, const int32_t* m_dev, int n_out,
                                    const void* w, int32_t* argmax, float* conf, float* max_logit, float* lse,
                                    float* logits, void* workspace, size_t ws_bytes, void* stream) {
  if (M > 0 && (m_dev == nullptr || row_idx == nullptr || out_pos == nullptr || n_out < 0)) return BD_EINVAL;
  return lm_common(dt, M, hidden, V, h_src, n_src, row_idx, out_pos, m_dev, n_out, w, argmax, conf, max_logit,
                   lse, logits, workspace, ws_bytes, stream);
}

// ---------------------------------------------------------------------------
bd_status bd_candidate_rows(int B, int win_lo, int win_len, const uint64_t* mask_bits, int rows_per_seq,
                            int32_t* row_idx, int32_t* out_pos, int32_t* count, void* stream) {
  if (B < 0) return BD_EINVAL;
  if (B == 0) return BD_OK;
  if (win_lo < 0 || win_len < 1 || win_len > 64 || win_lo + win_len > 64) return BD_EINVAL;
  if (rows_per_seq < win_lo + win_len || (long)B * win_len > 4096) return BD_EINVAL;
  if (!mask_bits || !row_idx || !out_pos || !count) return BD_EINVAL;
  return hip_status(bd_candidates_launch(B, win_lo, win_len, mask_bits, rows_per_seq, row_idx, out_pos, count,
                                         static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------------------
bd_status bd_threshold_unmask(int B, int D, int win_lo, int win_len, const float* conf, const int32_t* argmax,
                              float threshold, int32_t* tokens, uint64_t* mask_bits, int32_t* n_unmasked,
                              int32_t* unmasked_pos, void* stream) {
  if (B < 0) return BD_EINVAL;
  if (B == 0) return BD_OK;
  if (D < 1 || D > 64 || win_lo < 0 || win_len < 1 || win_len > 64 || win_lo + win_len > D) return BD_EINVAL;
  if (!conf || !argmax || !tokens || !mask_bits || !(threshold == threshold)) return BD_EINVAL;
  return hip_status(bd_unmask_launch(B, D, win_lo, win_len, conf, argmax, threshold, nullptr, tokens, mask_bits,
                                     n_unmasked, unmasked_pos, static_cast<hipStream_t>(stream)));
}

bd_status bd_threshold_unmask_tau(int B, int D, int win_lo, int win_len, const float* conf, const int32_t* argmax,
                                  const float* threshold, int32_t* tokens, uint64_t* mask_bits, int32_t* n_unmasked,
                                  int32_t* unmasked_pos, void* stream) {
  if (B < 0) return BD_EINVAL;
  if (B == 0) return BD_OK;
  if (D < 1 || D > 64 || win_lo < 0 || win_len < 1 || win_len > 64 || win_lo + win_len > D) return BD_EINVAL;
  if (!conf || !argmax || !tokens || !mask_bits || !threshold) return BD_EINVAL;
  return hip_status(bd_unmask_launch(B, D, win_lo, win_len, conf, argmax, 0.f, threshold, tokens, mask_bits,
                                     n_unmasked, unmasked_pos, static_cast<hipStream_t>(stream)));
}

bd_status bd_threshold_unmask_windows(int B, int D, int win_len, const int32_t* win_lo, const float* conf,
                                      const int32_t* argmax, float threshold, int32_t* tokens, uint64_t* mask_bits,
                                      int32_t* n_unmasked, int32_t* unmasked_pos, void* stream) {
  if (B < 0) return BD_EINVAL;
  if (B == 0) return BD_OK;
  if (D < 1 || D > 64 || win_len < 1 || win_len > D) return BD_EINVAL;
  if (!win_lo || !conf || !argmax || !tokens || !mask_bits || !(threshold == threshold)) return BD_EINVAL;
  return hip_status(bd_unmask_launch(B, D, 0, win_len, conf, argmax, threshold, nullptr, tokens, mask_bits,
                                     n_unmasked, unmasked_pos, static_cast<hipStream_t>(stream), win_lo));
}

bd_status bd_persequence_schedule(int B, int D, int S, const uint64_t* mask_bits, int32_t* win, int32_t* opening,
                                  int32_t* ran, uint64_t* restore, uint64_t* save, uint64_t* save_h,
                                  int32_t* row_idx, int32_t* win_lo, int32_t* kinds, int32_t* live, void* stream) {
  if (B < 0) return BD_EINVAL;
  if (B == 0) return BD_OK;
  if (S < 1 || D < S || D > 63 || D % S != 0 || (long)B * (1 + D) * 2 > INT32_MAX) return BD_EINVAL;
  if (!mask_bits || !win || !opening || !ran || !restore || !save || !save_h || !row_idx || !win_lo)
    return BD_EINVAL;
  return hip_status(bd_persequence_schedule_launch(B, D, S, mask_bits, win, opening, ran, restore, save, save_h,
                                                   row_idx, win_lo, kinds, live, static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------------------
bd_status bd_copy_rows(int B, int n_rows, int row_bytes, const uint64_t* row_mask, const void* src0, void* dst0,
                       const void* src1, void* dst1, void* stream) {
  if (B < 0 || n_rows < 0) return BD_EINVAL;
  if (B == 0 || n_rows == 0) return BD_OK;
  if (n_rows > 64 || row_bytes <= 0 || row_bytes % 16 != 0 || !row_mask || !src0 || !dst0) return BD_EINVAL;
  if ((src1 == nullptr) != (dst1 == nullptr)) return BD_EINVAL;
  if (!aligned16(src0) || !aligned16(dst0) || (src1 && (!aligned16(src1) || !aligned16(dst1)))) return BD_EINVAL;
  return hip_status(bd_copy_rows_launch(B, n_rows, row_bytes, row_mask, src0, dst0, src1, dst1,
                                        static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------------------
bd_status bd_kv_append(bd_dtype dt, int B, int Hkv, int d, int cap, void* k_cache, void* v_cache, int32_t* kv_len,
                       const int32_t* kv_len_host, const void* k_blk, const void* v_blk, int n_blk, int n_rows,
                       void* stream) {
  if (!valid_dtype(dt) || B < 0 || n_rows < 0) return BD_EINVAL;
  if (B == 0 || n_rows == 0) return BD_OK;
  if (Hkv <= 0 || d <= 0 || cap <= 0 || n_blk < n_rows || !k_cache || !v_cache || !kv_len || !k_blk || !v_blk)
    return BD_EINVAL;
  if ((d * (dt == BD_F32 ? 4 : 2)) % 16 != 0 || !aligned16(k_cache) || !aligned16(v_cache) ||
      !aligned16(k_blk) || !aligned16(v_blk))
    return BD_EINVAL;
  if (kv_len_host != nullptr)
    for (int b = 0; b < B; ++b)
      if (kv_len_host[b] < 0 || (long)kv_len_host[b] + n_rows > cap) return BD_ECAPACITY;
  return hip_status(bd_append_launch(dt, B, Hkv, d, cap, k_cache, v_cache, kv_len, k_blk, v_blk, n_blk, n_rows,
                                     static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------------------
bd_status bd_embed_rows(bd_dtype dt, int B, int D, int row_off, int n_rows, int hidden, int V, const void* E,
                        const int32_t* tokens, const uint64_t* mask_bits, const void* plant, void* x,
                        void* stream) {
  if (!valid_dtype(dt) || B < 0 || n_rows < 0) return BD_EINVAL;
  if (B == 0 || n_rows == 0) return BD_OK;
  if (D < 1 || (mask_bits != nullptr && D > 64) || row_off < 0 || row_off + n_rows > D || hidden <= 0 || V <= 0 ||
      !E || !tokens || !x)
    return BD_EINVAL;
  if (hidden % (dt == BD_BF16 ? 8 : 4) != 0 || !aligned16(E) || !aligned16(x) || (plant && !aligned16(plant)))
    return BD_EUNSUPPORTED;
  return hip_status(bd_embed_launch(dt, B, D, row_off, n_rows, hidden, V, E, tokens, mask_bits, plant, x,
                                    static_cast<hipStream_t>(stream)));
}

static bd_status gemm_common(bd_dtype dt, int M, int K, const void* x, bd_rows xr, const BdGemmSeg* segs, int nseg,
                             int mode, const BdGemmRope* rope, const BdGemmNorm* post_norm, void* workspace,
                             size_t ws_bytes, void* stream, const bd_guard* guard = nullptr,
                             float in_norm_eps = -1.f) {
  if (!valid_dtype(dt) || M < 0 || !valid_guard(guard)) return BD_EINVAL;
  if (M == 0) return BD_OK;
  if (K <= 0 || !x || !valid_rows(xr)) return BD_EINVAL;
  int N[3];
  for (int i = 0; i < nseg; ++i) {
    if (segs[i].N <= 0 || !segs[i].w || !segs[i].y || !valid_rows(segs[i].yr)) return BD_EINVAL;
    if (segs[i].res && !valid_rows(segs[i].rr)) return BD_EINVAL;
    N[i] = segs[i].N;
  }
  if (mode == BD_GEMM_ROPE) {
    const int d = rope->d;
    if (d <= 0 || d % 8 != 0 || N[0] % d != 0 || N[1] % d != 0 || rope->n_rows <= 0 || M % rope->n_rows != 0 ||
        rope->pos_off < 0 || !rope->pos_base || !(rope->theta > 1.f))
      return BD_EINVAL;
  }
  if (dt == BD_BF16) {
    if (K % 256 != 0 || !aligned16(x)) return BD_EUNSUPPORTED;
    for (int i = 0; i < nseg; ++i)
      if (!aligned16(segs[i].w)) return BD_EUNSUPPORTED;
  }
  BdGemmPlan p = bd_gemm_plan(dt, M, K, N, nseg, mode);
  if (in_norm_eps >= 0.f && p.kw_nt != 0) {  // the input norm rides on the streaming kernel instead
    p.kw_nt = p.kw_mt = 0;
    p.ny = (M + p.MT * 16 - 1) / (p.MT * 16);
  }
  if (p.ws_bytes > 0 && (workspace == nullptr || ws_bytes < p.ws_bytes || !aligned16(workspace)))
    return BD_EINVAL;
  return hip_status(bd_gemm_launch(dt, p, M, K, x, xr, segs, nseg, mode, rope, post_norm, workspace,
                                   static_cast<hipStream_t>(stream), guard, in_norm_eps));
}

size_t bd_linear_workspace_size(bd_dtype dt, int M, int N, int K) {
  if (!valid_dtype(dt) || M <= 0 || N <= 0 || K <= 0) return 0;
  return bd_gemm_plan(dt, M, K, &N, 1, BD_GEMM_PLAIN).ws_bytes;
}

size_t bd_qkv_proj_workspace_size(bd_dtype dt, int M, int K, int Nq, int Nkv) {
  if (!valid_dtype(dt) || M <= 0 || K <= 0 || Nq <= 0 || Nkv <= 0) return 0;
  const int N[3] = {Nq, Nkv, Nkv};
  return bd_gemm_plan(dt, M, K, N, 3, BD_GEMM_PLAIN).ws_bytes;
}

size_t bd_qkv_proj_rope_workspace_size(bd_dtype dt, int M, int K, int Nq, int Nkv) {
  if (!valid_dtype(dt) || M <= 0 || K <= 0 || Nq <= 0 || Nkv <= 0) return 0;
  const int N[3] = {Nq, Nkv, Nkv};
  return bd_gemm_plan(dt, M, K, N, 3, BD_GEMM_ROPE).ws_bytes;
}

bd_status bd_linear(bd_dtype dt, int M, int N, int K, const void* x, bd_rows xr, const void* w, const void* res,
                    bd_rows rr, void* y, bd_rows yr, void* workspace, size_t ws_bytes, void* stream) {
  BdGemmSeg seg{w, y, yr, res, rr, N};
  return gemm_common(dt, M, K, x, xr, &seg, 1, BD_GEMM_PLAIN, nullptr, nullptr, workspace, ws_bytes, stream);
}

bd_status bd_linear_guarded(bd_dtype dt, int M, int N, int K, const void* x, bd_rows xr, const void* w,
                            const void* res, bd_rows rr, void* y, bd_rows yr, void* workspace, size_t ws_bytes,
                            const bd_guard* guard, void* stream) {
  BdGemmSeg seg{w, y, yr, res, rr, N};
  return gemm_common(dt, M, K, x, xr, &seg, 1, BD_GEMM_PLAIN, nullptr, nullptr, workspace, ws_bytes, stream, guard);
}

bd_status bd_linear_residual_rmsnorm(bd_dtype dt, int M, int N, int K, const void* x, bd_rows xr, const void* w,
                                     void* y, bd_rows yr, float eps, void* h, bd_rows hr, void* workspace,
                                     size_t ws_bytes, void* stream) {
  if (!h || !valid_rows(hr) || !(eps >= 0.f)) return BD_EINVAL;
  BdGemmSeg seg{w, y, yr, y, yr, N};
  const BdGemmNorm norm{h, hr, eps};
  return gemm_common(dt, M, K, x, xr, &seg, 1, BD_GEMM_PLAIN, nullptr, &norm, workspace, ws_bytes, stream);
}

bd_status bd_qkv_proj(bd_dtype dt, int M, int K, const void* x, bd_rows xr, const void* wq, int Nq, void* q,
                      bd_rows qr, const void* wk, const void* wv, int Nkv, void* k, bd_rows kr, void* v, bd_rows vr,
                      void* workspace, size_t ws_bytes, void* stream) {
  const bd_rows none{1, 1, 0};
  BdGemmSeg segs[3] = {{wq, q, qr, nullptr, none, Nq}, {wk, k, kr, nullptr, none, Nkv},
                       {wv, v, vr, nullptr, none, Nkv}};
  return gemm_common(dt, M, K, x, xr, segs, 3, BD_GEMM_PLAIN, nullptr, nullptr, workspace, ws_bytes, stream);
}

bd_status bd_qkv_proj_guarded(bd_dtype dt, int M, int K, const void* x, bd_rows xr, const void* wq, int Nq, void* q,
                              bd_rows qr, const void* wk, const void* wv, int Nkv, void* k, bd_rows kr, void* v,
                              bd_rows vr, void* workspace, size_t ws_bytes, const bd_guard* guard, void* stream) {
  const bd_rows none{1, 1, 0};
  BdGemmSeg segs[3] = {{wq, q, qr, nullptr, none, Nq}, {wk, k, kr, nullptr, none, Nkv},
                       {wv, v, vr, nullptr, none, Nkv}};
  return gemm_common(dt, M, K, x, xr, segs, 3, BD_GEMM_PLAIN, nullptr, nullptr, workspace, ws_bytes, stream, guard);
}

bd_status bd_qkv_proj_rope(bd_dtype dt, int M, int K, const void* x, bd_rows xr, const void* wq, int Nq, void* q,
                           bd_rows qr, const void* wk, const void* wv, int Nkv, void* k, bd_rows kr, void* v,
                           bd_rows vr, int d, const int32_t* pos_base, int n_rows, int pos_off, float theta,
                           void* workspace, size_t ws_bytes, void* stream) {
  const bd_rows none{1, 1, 0};
  BdGemmSeg segs[3] = {{wq, q, qr, nullptr, none, Nq}, {wk, k, kr, nullptr, none, Nkv},
                       {wv, v, vr, nullptr, none, Nkv}};
  const BdGemmRope rope{pos_base, n_rows, pos_off, d, theta};
  return gemm_common(dt, M, K, x, xr, segs, 3, BD_GEMM_ROPE, &rope, nullptr, workspace, ws_bytes, stream);
}

bd_status bd_gate_up_swiglu(bd_dtype dt, int M, int K, const void* x, bd_rows xr, const void* w_gu, int inter,
                            void* a, bd_rows ar, void* stream) {
  const bd_rows none{1, 1, 0};
  BdGemmSeg seg{w_gu, a, ar, nullptr, none, inter};
  return gemm_common(dt, M, K, x, xr, &seg, 1, BD_GEMM_SWIGLU, nullptr, nullptr, nullptr, 0, stream);
}

bd_status bd_gate_up_swiglu_rmsnorm(bd_dtype dt, int M, int K, const void* x, bd_rows xr, float eps,
                                    const void* w_gu, int inter, void* a, bd_rows ar, void* stream) {
  if (!(eps >= 0.f)) return BD_EINVAL;
  const bd_rows none{1, 1, 0};
  BdGemmSeg seg{w_gu, a, ar, nullptr, none, inter};
  return gemm_common(dt, M, K, x, xr, &seg, 1, BD_GEMM_SWIGLU, nullptr, nullptr, nullptr, 0, stream, nullptr, eps);
}

// ---------------------------------------------------------------------------
bd_status bd_rmsnorm(bd_dtype dt, int M, int hidden, const void* x, bd_rows xr, float eps, void* y, bd_rows yr,
                     void* stream) {
  if (!valid_dtype(dt) || M < 0) return BD_EINVAL;
  if (M == 0) return BD_OK;
  if (hidden <= 0 || !x || !y || !valid_rows(xr) || !valid_rows(yr) || !(eps >= 0.f)) return BD_EINVAL;
  return hip_status(bd_rmsnorm_launch(dt, M, hidden, x, xr, eps, y, yr, static_cast<hipStream_t>(stream)));
}

bd_status bd_rope(bd_dtype dt, int B, int n_rows, int H, int d, void* x, bd_rows xr, const int32_t* pos_base,
                  int pos_off, float theta, void* stream) {
  if (!valid_dtype(dt) || B < 0 || n_rows < 0) return BD_EINVAL;
  if (B == 0 || n_rows == 0) return BD_OK;
  if (H <= 0 || d <= 0 || d % 2 != 0 || pos_off < 0 || !x || !pos_base || !valid_rows(xr) || !(theta > 1.f))
    return BD_EINVAL;
  return hip_status(bd_rope_launch(dt, B, n_rows, H, d, x, xr, pos_base, pos_off, theta,
                                   static_cast<hipStream_t>(stream)));
}

bd_status bd_swiglu(bd_dtype dt, int M, int inter, const void* gu, bd_rows gr, void* a, bd_rows ar, void* stream) {
  if (!valid_dtype(dt) || M < 0) return BD_EINVAL;
  if (M == 0) return BD_OK;
  if (inter <= 0 || !gu || !a || !valid_rows(gr) || !valid_rows(ar)) return BD_EINVAL;
  return hip_status(bd_swiglu_launch(dt, M, inter, gu, gr, a, ar, static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------------------
size_t bd_train_attn_workspace_size(bd_dtype dt, int S, int L, int D, int Hq, int Hkv, int d) {
  if (!valid_dtype(dt) || S <= 0 || L <= 0 || D < 1 || L % D != 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 ||
      (d != 64 && d != 128))
    return 0;
  return bd_train_plan(dt, S, L, D, Hq, Hkv, d).ws_bytes;
}

bd_status bd_train_attn(bd_dtype dt, int S, int L, int D, int Hq, int Hkv, int d, const void* q, const void* k,
                        const void* v, float scale, void* o, void* workspace, size_t ws_bytes, void* stream) {
  if (!valid_dtype(dt) || S < 0 || L < 0) return BD_EINVAL;
  if (S == 0 || L == 0) return BD_OK;
  if (D < 1 || L % D != 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || !q || !k || !v || !o || !(scale == scale))
    return BD_EINVAL;
  if (d != 64 && d != 128) return BD_EUNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return BD_EINVAL;
  const BdTrainPlan p = bd_train_plan(dt, S, L, D, Hq, Hkv, d);
  if (workspace == nullptr || ws_bytes < p.ws_bytes || !aligned16(workspace)) return BD_EINVAL;
  return hip_status(bd_train_attn_launch(dt, p, S, L, D, Hq, Hkv, d, q, k, v, scale, o, workspace,
                                         static_cast<hipStream_t>(stream)));
}

bd_status bd_masked_nll(bd_dtype dt, int M, int hidden, int V, const void* h_src, int n_src, const int32_t* row_idx,
                        const void* w, const int32_t* target, const float* lse, float* nll, float* loss_sum,
                        void* stream) {
  if (!valid_dtype(dt) || M < 0) return BD_EINVAL;
  if (M == 0) return BD_OK;
  if (hidden <= 0 || V <= 0 || n_src <= 0 || !h_src || !w || !target || !lse || !nll) return BD_EINVAL;
  if (hidden % (dt == BD_BF16 ? 8 : 4) != 0 || !aligned16(h_src) || !aligned16(w)) return BD_EUNSUPPORTED;
  return hip_status(bd_nll_launch(dt, M, hidden, V, h_src, n_src, row_idx, w, target, lse, nll, loss_sum,
                                  static_cast<hipStream_t>(stream)));
}

}  // extern "C"
