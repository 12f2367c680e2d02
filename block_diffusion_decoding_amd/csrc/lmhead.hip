// LM head with token shift and fused softmax statistics.
//
// Method: "Fast-dLLM v2: Efficient Block-Diffusion LLM" notes, Key design 2
// (token shift: the prediction for masked position i is read from the output
// row of position i-1, expressed here by a row index per output row) and Key
// design 3 (confidence-threshold unmasking needs, per candidate, the predicted
// token and its probability); "Fast-dLLM" v1 article, Core technique 2 (the
// confidence of a position is the probability the model gives its token).
//
// The logits h W^T are never written to memory (unless a debug dump is
// requested).  Each work-group reduces its tile of logits to, per row,
// (max, lowest argmax, sum of exp(l - max)); a second kernel folds the tiles
// of a row in a fixed order into argmax, max, log-sum-exp and
// confidence = exp(max - lse).
//
// bf16, up to 64 rows: streaming MFMA GEMM (stream_gemm.h), weights
// streamed once from HBM through a 3-stage asynchronous global->LDS pipeline.
// bf16, more rows (a whole batch's window or block, where the product is
// MFMA-bound): 256-row work-group tiles, see lm_big_kernel.
// fp32: plain VALU kernel.
//
// With a device-side row count (bd_lmhead_confidence_rows: the masked
// candidates listed first by bd_candidate_rows) rows past the count are
// skipped -- whole row blocks exit, and the 256-row kernel skips the loads
// and MFMAs of its row tiles past the count -- and the merge writes each
// row's statistics to its output slot.
#include <climits>

#include "bd_device.h"
#include "bd_launch.h"
#include "stream_gemm.h"

namespace {

constexpr int kThreads = 256;
// bf16 tiling; defaults chosen by measurement, overridable at build time.
#ifndef BD_LM_NTW
#define BD_LM_NTW 8
#endif
#ifndef BD_LM_NS
#define BD_LM_NS 3
#endif
constexpr int kNTW = BD_LM_NTW;  // 16-column tiles per work-group (bf16)
constexpr int kNS = BD_LM_NS;    // pipeline stages (bf16)
constexpr int kF32Rows = 16;  // rows per work-group (fp32)

struct LmK {
  const uint16_t* h;
  int n_src;
  const int32_t* row_idx;
  const uint16_t* w;
  float* logits;
  int M, hidden, V, nvt;
  float* pmax;
  int32_t* pidx;
  float* psum;
  const int32_t* m_dev;  // device row count, or NULL
};

// Rows taken: min(M, *m_dev) when a device count is given (the row list of
// the masked candidates), else M.
__device__ __forceinline__ int lm_rows(const int32_t* m_dev, int M) {
  if (m_dev == nullptr) return M;
  const int c = *m_dev;
  return c < 0 ? 0 : (c < M ? c : M);
}

__device__ __forceinline__ const uint16_t* lm_row(const LmK& a, int m, int Meff) {
  if (m >= Meff) return nullptr;
  const int r = a.row_idx ? a.row_idx[m] : m;
  if (r < 0 || r >= a.n_src) return nullptr;
  return a.h + (size_t)r * a.hidden;
}

template <int MT>
__global__ __launch_bounds__(kThreads, 2) void lm_bf16_kernel(LmK a) {
  using C = bd_stream::Cfg<MT, kNTW, kNS>;
  __shared__ uint4 sbuf[C::NS * C::STAGE_U4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int wm = wave % C::WM, wn = wave / C::WM;
  const int m0 = blockIdx.y * MT * 16;
  const int n0 = blockIdx.x * kNTW * 16;
  const int Meff = lm_rows(a.m_dev, a.M);
  if (m0 >= Meff) return;  // the whole row block is past the row count

  bd_f32x4 acc[C::MTW][C::NTP];
  auto xrow = [&](int m) { return lm_row(a, m, Meff); };
  bd_stream::mainloop<C>(xrow, a.h, m0, a.w, a.V, a.hidden, n0, sbuf, acc);

  // rows m0 + (wm*MTW + i)*16 + 4g + r, columns n0 + (wn*NTP + j)*16 + l16
  if (a.logits != nullptr) {  // debug dump of the raw logits (tests only)
#pragma unroll
    for (int i = 0; i < C::MTW; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + (wm * C::MTW + i) * 16 + 4 * g + r;
#pragma unroll
        for (int j = 0; j < C::NTP; ++j) {
          const int col = n0 + (wn * C::NTP + j) * 16 + l16;
          if (m < Meff && col < a.V) a.logits[(size_t)m * a.V + col] = acc[i][j][r];
        }
      }
  }
  const bool ragged = n0 + kNTW * 16 > a.V;  // only the last column block
  int col[C::NTP];
#pragma unroll
  for (int j = 0; j < C::NTP; ++j) col[j] = n0 + (wn * C::NTP + j) * 16 + l16;
  BdArgStat* red = reinterpret_cast<BdArgStat*>(sbuf);  // [WN][MT*16]
#pragma unroll
  for (int i = 0; i < C::MTW; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float v[C::NTP];
#pragma unroll
      for (int j = 0; j < C::NTP; ++j) v[j] = (ragged && col[j] >= a.V) ? BD_NEG_INF : acc[i][j][r];
      const BdArgStat st = bd_row16_stat(v, col);
      if (l16 == 0) red[wn * (MT * 16) + (wm * C::MTW + i) * 16 + 4 * g + r] = st;
    }
  }
  __syncthreads();
  if (tid < MT * 16 && m0 + tid < Meff) {
    BdArgStat st = red[tid];
#pragma unroll
    for (int w = 1; w < C::WN; ++w) st = bd_stat_combine(st, red[w * (MT * 16) + tid]);
    const size_t pi = (size_t)(m0 + tid) * a.nvt + blockIdx.x;
    a.pmax[pi] = st.m;
    a.pidx[pi] = st.i;
    a.psum[pi] = st.s;
  }
}

// ---------------------------------------------------------------------------
// Large-M bf16 LM head: each work-group computes a 256-row x (CT*16)-column
// tile of the logits with 8 waves and reduces it to per-row partials.
//   CT = 16 (more than 256 rows, MFMA-bound): 2 x 4 waves of 128 x 64, two
//            64 KiB stages;
//   CT = 8  (up to 256 rows, HBM-bound): 4 x 2 waves of 64 x 64, three
//            48 KiB stages (two in flight) and twice the work-groups, so the
//            weight stream has more bytes in flight and a shorter tail.
// K is walked in 64-wide chunks filled by whole-line DMA (the tile layout of
// stream_gemm.h: a 16-row x 64-k tile is 2 KiB, two instructions of 8 rows x
// 128 B, XOR-swizzled k-blocks).  Work order: the row blocks of one column
// block are consecutive on one XCD, so a W column block is fetched from HBM
// once and re-read from that XCD's L2.
constexpr int kBigRows = 256, kBigThreads = 512;
#ifndef BD_LM_NARROW_MAX_ROWS
#define BD_LM_NARROW_MAX_ROWS 256
#endif
constexpr int kNarrowMaxRows = BD_LM_NARROW_MAX_ROWS;  // up to this many rows: 256 x 128 tiles

template <int CT>
struct Big {
  static constexpr int WR = CT == 16 ? 2 : 4;       // waves along the rows
  static constexpr int WC = 8 / WR;                 // waves along the columns
  static constexpr int MW = kBigRows / 16 / WR;     // row tiles per wave
  static constexpr int NWT = CT / WC;               // column tiles per wave
  static constexpr int NS = CT == 16 ? 2 : 3;       // stages
  static constexpr int TILES = kBigRows / 16 + CT;  // 16-row tiles per stage
  static constexpr int FR = 2 * TILES;              // DMA instructions per stage
  static constexpr int LW = FR / 8;                 // per wave
  static constexpr int STAGE_U4 = FR * 64;
  static_assert(MW % 4 == 0 && NWT == 4 && FR % 8 == 0, "wave tiling");
};

template <int CT>
__global__ __launch_bounds__(kBigThreads, 1) void lm_big_kernel(LmK a, int rb_count, int cb_count) {
  using P = Big<CT>;
  __shared__ uint4 sbuf[P::NS * P::STAGE_U4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int wr = wave % P::WR, wc = wave / P::WR;
  // XCD-aware order: work-group w runs on XCD w % 8; the (w / 8)-th work-group
  // of an XCD takes row block q % rb_count of column block 8 * (q / rb_count) + xcd.
  const int xcd = blockIdx.x & 7, q = blockIdx.x >> 3;
  const int rb = q % rb_count, cb = 8 * (q / rb_count) + xcd;
  if (cb >= cb_count) return;
  const int m0 = rb * kBigRows, n0 = cb * CT * 16;
  const int nch = a.hidden / 64;
  const int Meff = lm_rows(a.m_dev, a.M);
  if (m0 >= Meff) return;  // the whole row block is past the row count

  // DMA sources: instruction f covers rows 8*(f%2)..+7 of stage tile f/2;
  // tiles 0..15 are X row tiles, the next CT are W column tiles.
  const int lrow = lane >> 3, lkb = (lane & 7) ^ lrow;
  const uint16_t* src[P::LW];
#pragma unroll
  for (int i = 0; i < P::LW; ++i) {
    const int f = wave + 8 * i, t = f >> 1, r = 8 * (f & 1) + lrow;
    if (t < kBigRows / 16) {
      const uint16_t* p = lm_row(a, m0 + t * 16 + r, Meff);
      src[i] = (p ? p : a.h) + 8 * lkb;
    } else {
      const int col = n0 + (t - kBigRows / 16) * 16 + r;
      src[i] = a.w + (size_t)(col < a.V ? col : 0) * a.hidden + 8 * lkb;
    }
  }
  // X tiles past the row count are not loaded (their MFMAs are skipped);
  // the number of loads this wave issues per stage is then a wave-uniform
  // value and the pipeline waits select the matching immediate.
  const int live_tiles = (Meff - m0 + 15) / 16;
  bool ld[P::LW];
  int issued = 0;
#pragma unroll
  for (int i = 0; i < P::LW; ++i) {
    const int t = (wave + 8 * i) >> 1;
    ld[i] = t >= kBigRows / 16 || t < live_tiles;
    issued += ld[i] ? 1 : 0;
  }
  auto issue = [&](int ch) {
    uint4* st = sbuf + (ch % P::NS) * P::STAGE_U4;
#pragma unroll
    for (int i = 0; i < P::LW; ++i)
      if (ld[i])
        __builtin_amdgcn_global_load_lds((bd_stream::glb_void_t*)(src[i] + (size_t)ch * 64),
                                         (bd_stream::lds_void_t*)(st + (wave + 8 * i) * 64), 16, 0, 0);
  };
  auto wait_later_stage = [&]() {  // vmcnt <= loads of one stage
    switch (issued) {
      case 0: __builtin_amdgcn_s_waitcnt(bd_stream::vmcnt_imm(0)); break;
      case 1: __builtin_amdgcn_s_waitcnt(bd_stream::vmcnt_imm(1)); break;
      case 2: __builtin_amdgcn_s_waitcnt(bd_stream::vmcnt_imm(2)); break;
      case 3: __builtin_amdgcn_s_waitcnt(bd_stream::vmcnt_imm(3)); break;
      case 4: __builtin_amdgcn_s_waitcnt(bd_stream::vmcnt_imm(4)); break;
      case 5: __builtin_amdgcn_s_waitcnt(bd_stream::vmcnt_imm(5)); break;
      case 6: __builtin_amdgcn_s_waitcnt(bd_stream::vmcnt_imm(6)); break;
      case 7: __builtin_amdgcn_s_waitcnt(bd_stream::vmcnt_imm(7)); break;
      default: __builtin_amdgcn_s_waitcnt(bd_stream::vmcnt_imm(8)); break;
    }
  };
  static_assert(P::LW <= 8, "wait immediates");

  bd_f32x4 acc[P::MW][P::NWT];
#pragma unroll
  for (int i = 0; i < P::MW; ++i)
#pragma unroll
    for (int j = 0; j < P::NWT; ++j) acc[i][j] = bd_f32x4{0.f, 0.f, 0.f, 0.f};
  const uint32_t sbase = bd_stream::lds_addr(sbuf);
  const uint32_t fo[2] = {(uint32_t)bd_stream::frag_offset(lane, 0), (uint32_t)bd_stream::frag_offset(lane, 1)};
  // Row tiles are dealt to the row waves in turn (tile i of this wave is row
  // tile i*WR + wr), so that the waves sharing a SIMD get equal shares when
  // rows past the count are skipped.  First X / W tile as a byte offset.
  const uint32_t xt0 = wr * 2048, wt0 = (kBigRows / 16 + wc * P::NWT) * 2048;
  constexpr int XS = P::WR * 2048;  // byte stride between this wave's X tiles
  // this wave's 16-row tiles that hold rows below the count (MFMAs of the
  // others are skipped: the candidate rows are listed first)
  const int live = min(P::MW, max(0, (live_tiles - wr + P::WR - 1) / P::WR));

#pragma unroll
  for (int c = 0; c < P::NS - 1; ++c)
    if (c < nch) issue(c);
  for (int ch = 0; ch < nch; ++ch) {
    // chunks issued so far: min(nch, ch + NS - 1); keep the later ones in flight
    if (P::NS == 3 && ch + 1 < nch) wait_later_stage();
    else __builtin_amdgcn_s_waitcnt(bd_stream::vmcnt_imm(0));
    bd_stream::pipe_barrier();  // chunk ch in LDS everywhere; the slot of ch - 1 is free
    if (ch + P::NS - 1 < nch) issue(ch + P::NS - 1);
    const uint32_t st = sbase + (ch % P::NS) * P::STAGE_U4 * 16;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      uint4 wb[4], xa[4];
      bd_stream::lds_frags_4x4<XS>(st + xt0 + fo[ks], st + wt0 + fo[ks], xa, wb);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (i < live)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = bd_mfma16(xa[i], wb[j], acc[i][j]);
#pragma unroll
      for (int i0 = 4; i0 < P::MW; i0 += 4) {
        if (i0 >= live) break;
        bd_stream::lds_frags_4<XS>(st + xt0 + i0 * XS + fo[ks], xa);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (i0 + i < live)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i0 + i][j] = bd_mfma16(xa[i], wb[j], acc[i0 + i][j]);
      }
    }
  }
  __syncthreads();  // the stages become the reduction buffer

  // acc[i][j][r]: row m0 + (i*WR + wr)*16 + 4g + r, column n0 + wc*NWT*16 + 16j + l16
  if (a.logits != nullptr) {  // debug dump of the raw logits (tests only)
#pragma unroll
    for (int i = 0; i < P::MW; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + (i * P::WR + wr) * 16 + 4 * g + r;
#pragma unroll
        for (int j = 0; j < P::NWT; ++j) {
          const int col = n0 + (wc * P::NWT + j) * 16 + l16;
          if (m < Meff && col < a.V) a.logits[(size_t)m * a.V + col] = acc[i][j][r];
        }
      }
  }
  const bool ragged = n0 + CT * 16 > a.V;  // only the last column block
  int col[P::NWT];
#pragma unroll
  for (int j = 0; j < P::NWT; ++j) col[j] = n0 + (wc * P::NWT + j) * 16 + l16;
  BdArgStat* red = reinterpret_cast<BdArgStat*>(sbuf);  // [WC column waves][256 rows]
#pragma unroll
  for (int i = 0; i < P::MW; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float v[P::NWT];
#pragma unroll
      for (int j = 0; j < P::NWT; ++j) v[j] = (ragged && col[j] >= a.V) ? BD_NEG_INF : acc[i][j][r];
      const BdArgStat st = bd_row16_stat(v, col);
      if (l16 == 0) red[wc * kBigRows + (i * P::WR + wr) * 16 + 4 * g + r] = st;
    }
  }
  __syncthreads();
  if (tid < kBigRows && m0 + tid < Meff) {
    BdArgStat st = red[tid];
#pragma unroll
    for (int w = 1; w < P::WC; ++w) st = bd_stat_combine(st, red[w * kBigRows + tid]);
    const size_t pi = (size_t)(m0 + tid) * a.nvt + cb;
    a.pmax[pi] = st.m;
    a.pidx[pi] = st.i;
    a.psum[pi] = st.s;
  }
}

struct LmF {
  const float* h;
  int n_src;
  const int32_t* row_idx;
  const float* w;
  float* logits;
  int M, hidden, V, nvt;
  float* pmax;
  int32_t* pidx;
  float* psum;
  const int32_t* m_dev;
};

__global__ __launch_bounds__(kThreads) void lm_f32_kernel(LmF a) {
  __shared__ float sh[kF32Rows][kThreads];
  __shared__ BdArgStat red[kThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = blockIdx.x * kThreads + tid;
  const int m0 = blockIdx.y * kF32Rows;
  const int Meff = lm_rows(a.m_dev, a.M);
  if (m0 >= Meff) return;
  const float* hrow[kF32Rows];
#pragma unroll
  for (int r = 0; r < kF32Rows; ++r) {
    const int m = m0 + r;
    const int src = (m < Meff) ? (a.row_idx ? a.row_idx[m] : m) : -1;
    hrow[r] = (src >= 0 && src < a.n_src) ? a.h + (size_t)src * a.hidden : nullptr;
  }
  float acc[kF32Rows];
#pragma unroll
  for (int r = 0; r < kF32Rows; ++r) acc[r] = 0.f;
  for (int k0 = 0; k0 < a.hidden; k0 += kThreads) {
    const int kn = min(kThreads, a.hidden - k0);
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kF32Rows; ++r) sh[r][tid] = (hrow[r] != nullptr && tid < kn) ? hrow[r][k0 + tid] : 0.f;
    __syncthreads();
    if (col < a.V) {
      const float* wr = a.w + (size_t)col * a.hidden + k0;
      for (int kk = 0; kk < kn; ++kk) {
        const float wv = wr[kk];
#pragma unroll
        for (int r = 0; r < kF32Rows; ++r) acc[r] += sh[r][kk] * wv;
      }
    }
  }
#pragma unroll
  for (int r = 0; r < kF32Rows; ++r) {
    const int m = m0 + r;
    if (a.logits != nullptr && m < Meff && col < a.V) a.logits[(size_t)m * a.V + col] = acc[r];
    BdArgStat st = (col < a.V) ? BdArgStat{acc[r], col, 1.f} : BdArgStat{BD_NEG_INF, INT_MAX, 0.f};
    for (int off = 1; off < 64; off <<= 1) st = bd_stat_combine(st, bd_stat_shfl_xor(st, off));
    __syncthreads();
    if (lane == 0) red[wave] = st;
    __syncthreads();
    if (tid == 0 && m < Meff) {
      BdArgStat t = red[0];
      for (int w = 1; w < kThreads / 64; ++w) t = bd_stat_combine(t, red[w]);
      const size_t pi = (size_t)m * a.nvt + blockIdx.x;
      a.pmax[pi] = t.m;
      a.pidx[pi] = t.i;
      a.psum[pi] = t.s;
    }
  }
}

// Fold the tiles of each row; one work-group per row.  Each thread keeps up to
// kMergePer of the row's tile statistics in registers: the row max is found
// first, then every tile's sum is scaled with one exp2 and the argmax is the
// lowest column among the tiles that reach the max.  The order of the sums
// is fixed, so the result is deterministic.
constexpr int kMergePer = 8;

__device__ __forceinline__ float block_max(float v, float* sh) {
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  v = sh[0];
  for (int w = 1; w < kThreads / 64; ++w) v = fmaxf(v, sh[w]);
  return v;
}

__global__ __launch_bounds__(kThreads) void lm_merge_kernel(const int32_t* row_idx, int n_src, int M,
                                                            int nvt, const float* pmax, const int32_t* pidx,
                                                            const float* psum, int32_t* argmax, float* conf,
                                                            float* max_logit, float* lse, const int32_t* m_dev,
                                                            const int32_t* out_pos, int n_out) {
  __shared__ float shm[kThreads / 64];
  __shared__ float shs[kThreads / 64];
  __shared__ int shi[kThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = blockIdx.x;
  if (m >= lm_rows(m_dev, M)) return;
  const int om = out_pos ? out_pos[m] : m;  // output slot of this row
  if (out_pos != nullptr && (om < 0 || om >= n_out)) return;
  const size_t rowb = (size_t)m * nvt;
  float mx = BD_NEG_INF, s = 0.f;
  int idx = INT_MAX;
  if (nvt <= kMergePer * kThreads) {
    float pm[kMergePer], ps[kMergePer];
    int pi[kMergePer];
#pragma unroll
    for (int u = 0; u < kMergePer; ++u) {
      const int t = tid + u * kThreads;
      const bool ok = t < nvt;
      pm[u] = ok ? pmax[rowb + t] : BD_NEG_INF;
      ps[u] = ok ? psum[rowb + t] : 0.f;
      pi[u] = ok ? pidx[rowb + t] : INT_MAX;
    }
#pragma unroll
    for (int u = 0; u < kMergePer; ++u) mx = fmaxf(mx, pm[u]);
    mx = block_max(mx, shm);
    const float mu = (mx == BD_NEG_INF) ? 0.f : mx;
#pragma unroll
    for (int u = 0; u < kMergePer; ++u) {
      s += ps[u] * bd_exp2((pm[u] - mu) * BD_LOG2E);
      if (pm[u] == mx && pm[u] != BD_NEG_INF) idx = min(idx, pi[u]);
    }
  } else {  // very large vocabularies: pairwise combines over a strided loop
    BdArgStat st{BD_NEG_INF, INT_MAX, 0.f};
    for (int t = tid; t < nvt; t += kThreads) st = bd_stat_combine(st, BdArgStat{pmax[rowb + t], pidx[rowb + t], psum[rowb + t]});
    mx = block_max(st.m, shm);
    const float mu = (mx == BD_NEG_INF) ? 0.f : mx;
    s = (st.m == BD_NEG_INF) ? 0.f : st.s * bd_exp2((st.m - mu) * BD_LOG2E);
    if (st.m == mx && st.m != BD_NEG_INF) idx = st.i;
  }
  for (int off = 32; off > 0; off >>= 1) {
    s += __shfl_xor(s, off);
    idx = min(idx, __shfl_xor(idx, off));
  }
  if (lane == 0) {
    shs[wave] = s;
    shi[wave] = idx;
  }
  __syncthreads();
  if (tid != 0) return;
  for (int w = 1; w < kThreads / 64; ++w) {
    s += shs[w];
    idx = min(idx, shi[w]);
  }
  const int src = row_idx ? row_idx[m] : m;
  const bool ok = src >= 0 && src < n_src && s > 0.f;
  const float nan = __builtin_nanf("");
  argmax[om] = ok ? idx : -1;
  conf[om] = ok ? 1.f / s : nan;
  if (max_logit != nullptr) max_logit[om] = ok ? mx : nan;
  if (lse != nullptr) lse[om] = ok ? mx + bd_log2(s) * BD_LN2 : nan;
}

}  // namespace

BdLmPlan bd_lm_plan(bd_dtype dt, int M, int hidden, int V) {
  BdLmPlan p{};
  if (dt == BD_F32) {
    p.cols_per_wg = kThreads;
    p.rows_per_wg = kF32Rows;
  } else if (M > 64) {
    p.cols_per_wg = (M > kNarrowMaxRows ? 16 : 8) * 16;
    p.rows_per_wg = kBigRows;
  } else {
    p.cols_per_wg = kNTW * 16;
    const int mt = (M + 15) / 16;
    p.rows_per_wg = 16 * (mt <= 1 ? 1 : (mt == 2 ? 2 : 4));
  }
  p.nvt = (V + p.cols_per_wg - 1) / p.cols_per_wg;
  p.nmb = (M + p.rows_per_wg - 1) / p.rows_per_wg;
  p.ws_bytes = (size_t)M * p.nvt * (2 * sizeof(float) + sizeof(int32_t));
  (void)hidden;
  return p;
}

hipError_t bd_lm_launch(bd_dtype dt, const BdLmPlan& p, const BdLmArgs& x, hipStream_t s) {
  const dim3 grid(p.nvt, p.nmb);
  if (dt == BD_F32) {
    LmF a{static_cast<const float*>(x.h), x.n_src, x.row_idx, static_cast<const float*>(x.w), x.logits,
          x.M, x.hidden, x.V, p.nvt, x.pmax, x.pidx, x.psum, x.m_dev};
    hipLaunchKernelGGL(lm_f32_kernel, grid, dim3(kThreads), 0, s, a);
  } else {
    LmK a{static_cast<const uint16_t*>(x.h), x.n_src, x.row_idx, static_cast<const uint16_t*>(x.w), x.logits,
          x.M, x.hidden, x.V, p.nvt, x.pmax, x.pidx, x.psum, x.m_dev};
    switch (p.rows_per_wg / 16) {
      case kBigRows / 16: {
        const int cb8 = (p.nvt + 7) / 8 * 8;  // column blocks rounded up to whole XCD rounds
        if (p.cols_per_wg == 256)
          hipLaunchKernelGGL(lm_big_kernel<16>, dim3(cb8 * p.nmb), dim3(kBigThreads), 0, s, a, p.nmb, p.nvt);
        else
          hipLaunchKernelGGL(lm_big_kernel<8>, dim3(cb8 * p.nmb), dim3(kBigThreads), 0, s, a, p.nmb, p.nvt);
        break;
      }
      case 1: hipLaunchKernelGGL(lm_bf16_kernel<1>, grid, dim3(kThreads), 0, s, a); break;
      case 2: hipLaunchKernelGGL(lm_bf16_kernel<2>, grid, dim3(kThreads), 0, s, a); break;
      default: hipLaunchKernelGGL(lm_bf16_kernel<4>, grid, dim3(kThreads), 0, s, a); break;
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(lm_merge_kernel, dim3(x.M), dim3(kThreads), 0, s, x.row_idx, x.n_src, x.M,
                     p.nvt, x.pmax, x.pidx, x.psum, x.argmax, x.conf, x.max_logit, x.lse, x.m_dev, x.out_pos,
                     x.n_out);
  return hipGetLastError();
}
