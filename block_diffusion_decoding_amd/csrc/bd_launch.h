// Host-side launchers of the libbd kernels (internal; the C ABI is bd.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/bd.h"

// ---- shared by the C-ABI files --------------------------------------------
// BD_OK for hipSuccess; otherwise records the error for bd_last_hip_error()
// and returns BD_EHIP.
bd_status bd_hip_status(hipError_t e);

// Host-side argument checks of bd_block_attn (BD_OK also for empty work).
bd_status bd_block_attn_check(bd_dtype dt, int B, int Hq, int Hkv, int d, int D, const void* q, int n_q, int q_off,
                              const void* k_cache, const void* v_cache, const int32_t* kv_len, int cap,
                              const void* k_blk, const void* v_blk, int n_blk, float scale, const void* o);

// ---- attention -----------------------------------------------------------
struct BdAttnPlan {
  int R;          // query rows per (sequence, KV head) = n_q * G
  int QT;         // 16-row query tiles
  int qpw;        // query tiles per wave
  int nqg;        // query-tile groups (work items along the query rows)
  int chunk;      // keys per work item
  int nchunks;    // key chunks (max over sequences)
  int stream_nt;  // committed K/V loaded with the non-temporal hint (bf16)
  int light;      // small call: short stage ring, two work-groups per CU (bf16)
  size_t part_o;  // workspace offsets / sizes in bytes
  size_t part_ml;
  size_t ws_bytes;
};

BdAttnPlan bd_attn_plan(bd_dtype dt, int B, int Hq, int Hkv, int d, int n_q, int cap, int n_blk);

struct BdAttnArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* kv_len;
  const void* k_blk;
  const void* v_blk;
  void* o;
  float* lse;
  float* part_o;
  float* part_ml;
  int B, Hq, Hkv, G, d, D, n_q, q_off, cap, n_blk;
  int epc;  // entries per cache slab (1: entry b owns slab b)
  float scale;
  const bd_guard* guard;  // optional (bd_guard)
};

hipError_t bd_attn_launch(bd_dtype dt, const BdAttnPlan& p, const BdAttnArgs& a, hipStream_t s);

// ---- LM head ---------------------------------------------------------------
struct BdLmPlan {
  int cols_per_wg;  // vocabulary columns per work-group (at most, streaming kernel)
  int nvt;          // work-groups along V (partials per row)
  int passes;       // streaming kernel: passes over a work-group's column range
  int rows_per_wg;  // rows of h per work-group
  int nmb;          // row blocks
  size_t ws_bytes;  // partial (max, argmax, sum) per (row, tile)
};

BdLmPlan bd_lm_plan(bd_dtype dt, int M, int hidden, int V);

struct BdLmArgs {
  const void* h;
  int n_src;
  const int32_t* row_idx;
  const void* w;
  int32_t* argmax;
  float* conf;
  float* max_logit;
  float* lse;
  float* logits;
  int M, hidden, V;
  float* pmax;
  int32_t* pidx;
  float* psum;
  const int32_t* m_dev;    // device row count (rows >= it are skipped), or NULL = M
  const int32_t* out_pos;  // output slot of row m, or NULL = m
  int n_out;               // output slots when out_pos is given
};

// Threshold unmask fused into the LM head's merge: rows m = b * win_len + r
// (window entry r of sequence b), one work-group per sequence.
struct BdLmUnmask {
  int B, D, win_lo, win_len;
  float threshold;
  const float* threshold_dev;  // [B] per-sequence threshold, or NULL = threshold
  int32_t* tokens;
  uint64_t* mask_bits;
  int32_t* n_unmasked;
  int32_t* unmasked_pos;
  uint64_t* bits_out;          // second copy of the new mask bits, or NULL
  // next step's input rows (x != NULL): the row of every position unmasked
  // here becomes E[token] (+ plant), x / plant [B, D, hidden], E [V+1, hidden]
  const void* emb;
  const void* plant;
  void* x;
  int hidden, V, f32;
};

// um != NULL: the merge also applies the threshold rule (a.M = B * win_len,
// no row list compaction).
hipError_t bd_lm_launch(bd_dtype dt, const BdLmPlan& p, const BdLmArgs& a, hipStream_t s,
                        const BdLmUnmask* um = nullptr);
hipError_t bd_candidates_launch(int B, int win_lo, int win_len, const uint64_t* mask_bits, int rows_per_seq,
                                int32_t* row_idx, int32_t* out_pos, int32_t* count, hipStream_t s);

// ---- projections -------------------------------------------------------------
struct BdGemmSeg {
  const void* w;   // [N, K]
  void* y;         // rows of N elements
  bd_rows yr;
  const void* res; // optional residual, rows of N elements
  bd_rows rr;
  int N;
};

// Epilogue variants of the projection GEMM.
enum BdGemmMode {
  BD_GEMM_PLAIN = 0,   // y = x W^T (+ res)
  BD_GEMM_ROPE = 1,    // segments 0 and 1 (q, k) rotated after the product
  BD_GEMM_SWIGLU = 2,  // one segment: W = [gate; up] (2N rows), y = silu(x Wg^T) * (x Wu^T)
};

// Rotary embedding of the q and k segments (BD_GEMM_ROPE): logical row m is
// at position pos_base[m / n_rows] + pos_off + m % n_rows; head dim d.
struct BdGemmRope {
  const int32_t* pos_base;
  int n_rows, pos_off, d;
  float theta;
};

struct BdGemmPlan {
  int MT;                 // 16-row tiles per work-group
  int NTW;                // 16-column tiles per pass
  int ny;                 // row blocks
  int T;                  // 16-column tiles over all segments
  int G;                  // tiles per scheduling unit (2 in SwiGLU mode: a gate and an up tile)
  int nwg;                // persistent work-groups per (row block, K slice)
  int passes;             // passes per work-group
  int ksplit;             // K slices
  int big_ct;             // > 0: 256-row x (big_ct*16)-column tiles instead (large M)
  int kw_nt;              // > 0: K split over the waves of a work-group, kw_nt tiles and kw_mt row tiles each
  int kw_mt;
  size_t ws_bytes;        // workspace: fp32 partial sums [ksplit][M][T*16]
};

BdGemmPlan bd_gemm_plan(bd_dtype dt, int M, int K, const int* N, int nseg, int mode);

// RMSNorm (unit gains) of a one-segment projection's output rows, after the
// residual: h[hr(m)] = y[yr(m)] / sqrt(mean y^2 + eps).
struct BdGemmNorm {
  void* h;
  bd_rows hr;
  float eps;
};

// guard: optional (bd_guard), honoured by every kernel of the launch.
// in_norm_eps >= 0 (SwiGLU mode only): the rows of x are RMS-normalised
// (unit gains) before the product; not with the K split over waves.
hipError_t bd_gemm_launch(bd_dtype dt, const BdGemmPlan& p, int M, int K, const void* x, bd_rows xr,
                          const BdGemmSeg* segs, int nseg, int mode, const BdGemmRope* rope,
                          const BdGemmNorm* post_norm, void* workspace, hipStream_t s,
                          const bd_guard* guard = nullptr, float in_norm_eps = -1.f);

hipError_t bd_embed_launch(bd_dtype dt, int B, int D, int row_off, int n_rows, int hidden, int V,
                           const void* E, const int32_t* tokens, const uint64_t* mask_bits,
                           const void* plant, void* x, hipStream_t s);

// ---- unmask / append ---------------------------------------------------------
hipError_t bd_unmask_launch(int B, int D, int win_lo, int win_len, const float* conf,
                            const int32_t* argmax, float threshold, const float* threshold_dev,
                            int32_t* tokens, uint64_t* mask_bits, int32_t* n_unmasked,
                            int32_t* unmasked_pos, hipStream_t s, const int32_t* win_lo_dev = nullptr);
hipError_t bd_persequence_schedule_launch(int B, int D, int S, const uint64_t* mask_bits, int32_t* win,
                                         int32_t* opening, int32_t* ran, uint64_t* restore, uint64_t* save,
                                         uint64_t* save_h, int32_t* row_idx, int32_t* win_lo, int32_t* kinds,
                                         int32_t* live, hipStream_t s);
hipError_t bd_copy_rows_launch(int B, int n_rows, int row_bytes, const uint64_t* row_mask, const void* src0,
                               void* dst0, const void* src1, void* dst1, hipStream_t s);

hipError_t bd_append_launch(bd_dtype dt, int B, int Hkv, int d, int cap, void* k_cache,
                            void* v_cache, int32_t* kv_len, const void* k_blk, const void* v_blk,
                            int n_blk, int n_rows, hipStream_t s);

// ---- training form (train.hip) ------------------------------------------------
struct BdTrainPlan {
  BdAttnPlan attn;      // the step kernel over S*2*(L/D) entries
  size_t cache_bytes;   // one of the clean K / V caches [S, Hkv, L, d]
  size_t len_off;       // int32 cached length per entry
  size_t attn_off;      // attention partials
  size_t ws_bytes;
};

BdTrainPlan bd_train_plan(bd_dtype dt, int S, int L, int D, int Hq, int Hkv, int d);
hipError_t bd_train_attn_launch(bd_dtype dt, const BdTrainPlan& p, int S, int L, int D, int Hq, int Hkv, int d,
                                const void* q, const void* k, const void* v, float scale, void* o,
                                void* workspace, hipStream_t s);
hipError_t bd_nll_launch(bd_dtype dt, int M, int hidden, int V, const void* h, int n_src, const int32_t* row_idx,
                         const void* w, const int32_t* target, const float* lse, float* nll, float* loss,
                         hipStream_t s);

// ---- layer pieces of the multi-layer model (model_ops.hip) --------------------
hipError_t bd_rmsnorm_launch(bd_dtype dt, int M, int hidden, const void* x, bd_rows xr, float eps, void* y,
                             bd_rows yr, hipStream_t s);
hipError_t bd_rope_launch(bd_dtype dt, int B, int n_rows, int H, int d, void* x, bd_rows xr, const int32_t* pos_base,
                          int pos_off, float theta, hipStream_t s);
hipError_t bd_swiglu_launch(bd_dtype dt, int M, int inter, const void* gu, bd_rows gr, void* a, bd_rows ar,
                            hipStream_t s);
