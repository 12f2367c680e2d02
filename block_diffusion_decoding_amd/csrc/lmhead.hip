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
// bf16, more rows (the exact step of a whole batch, where the product is
// MFMA-bound): 256 x 256 work-group tiles, see lm_big_kernel.
// fp32: plain VALU kernel.
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
};

__device__ __forceinline__ const uint16_t* lm_row(const LmK& a, int m) {
  if (m >= a.M) return nullptr;
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

  bd_f32x4 acc[C::MTW][C::NTP];
  auto xrow = [&](int m) { return lm_row(a, m); };
  bd_stream::mainloop<C>(xrow, a.h, m0, a.w, a.V, a.hidden, n0, sbuf, acc);

  // rows m0 + (wm*MTW + i)*16 + 4g + r, columns n0 + (wn*NTP + j)*16 + l16
  BdArgStat* red = reinterpret_cast<BdArgStat*>(sbuf);  // [WN][MT*16]
#pragma unroll
  for (int i = 0; i < C::MTW; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int rl = (wm * C::MTW + i) * 16 + 4 * g + r;
      BdArgStat st{BD_NEG_INF, INT_MAX, 0.f};
#pragma unroll
      for (int j = 0; j < C::NTP; ++j) {
        const int col = n0 + (wn * C::NTP + j) * 16 + l16;
        const float v = acc[i][j][r];
        if (col < a.V && v > st.m) {
          st.m = v;
          st.i = col;
        }
      }
      float s = 0.f;
#pragma unroll
      for (int j = 0; j < C::NTP; ++j) {
        const int col = n0 + (wn * C::NTP + j) * 16 + l16;
        if (col < a.V) s += bd_exp2((acc[i][j][r] - st.m) * BD_LOG2E);
      }
      st.s = s;
      if (a.logits != nullptr && m0 + rl < a.M) {
#pragma unroll
        for (int j = 0; j < C::NTP; ++j) {
          const int col = n0 + (wn * C::NTP + j) * 16 + l16;
          if (col < a.V) a.logits[(size_t)(m0 + rl) * a.V + col] = acc[i][j][r];
        }
      }
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) st = bd_stat_combine(st, bd_stat_shfl_xor(st, off));
      if (l16 == 0) red[wn * (MT * 16) + rl] = st;
    }
  }
  __syncthreads();
  if (tid < MT * 16 && m0 + tid < a.M) {
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
// Large-M bf16 LM head: each work-group computes a 256-row x 256-column tile of
// the logits with 8 waves (2 along the rows x 4 along the columns, 128 x 64
// each, 32 MFMA accumulators per wave) and reduces it to per-row partials.
// K is walked in 64-wide chunks through two 64 KiB LDS stages filled by
// whole-line DMA (the tile layout of stream_gemm.h: a 16-row x 64-k tile is
// 2 KiB, two instructions of 8 rows x 128 B, XOR-swizzled k-blocks).  Work
// order: the row blocks of one column block are consecutive on one XCD, so a
// W column block is fetched from HBM once and re-read from that XCD's L2.
constexpr int kBigRows = 256, kBigCols = 256, kBigThreads = 512;
constexpr int kBigTiles = (kBigRows + kBigCols) / 16;  // 16-row tiles per stage
constexpr int kBigFR = 2 * kBigTiles;                   // DMA instructions per stage
constexpr int kBigLW = kBigFR / 8;                      // per wave
constexpr int kBigStageU4 = kBigFR * 64;

__global__ __launch_bounds__(kBigThreads, 1) void lm_big_kernel(LmK a, int rb_count, int cb_count) {
  __shared__ uint4 sbuf[2 * kBigStageU4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int wr = wave & 1, wc = wave >> 1;
  // XCD-aware order: work-group w runs on XCD w % 8; the (w / 8)-th work-group
  // of an XCD takes row block q % rb_count of column block 8 * (q / rb_count) + xcd.
  const int xcd = blockIdx.x & 7, q = blockIdx.x >> 3;
  const int rb = q % rb_count, cb = 8 * (q / rb_count) + xcd;
  if (cb >= cb_count) return;
  const int m0 = rb * kBigRows, n0 = cb * kBigCols;
  const int nch = a.hidden / 64;

  // DMA sources: instruction f covers rows 8*(f%2)..+7 of stage tile f/2;
  // tiles 0..15 are X row tiles, 16..31 W column tiles.
  const int lrow = lane >> 3, lkb = (lane & 7) ^ lrow;
  const uint16_t* src[kBigLW];
#pragma unroll
  for (int i = 0; i < kBigLW; ++i) {
    const int f = wave + 8 * i, t = f >> 1, r = 8 * (f & 1) + lrow;
    if (t < kBigRows / 16) {
      const uint16_t* p = lm_row(a, m0 + t * 16 + r);
      src[i] = (p ? p : a.h) + 8 * lkb;
    } else {
      const int col = n0 + (t - kBigRows / 16) * 16 + r;
      src[i] = a.w + (size_t)(col < a.V ? col : 0) * a.hidden + 8 * lkb;
    }
  }
  auto issue = [&](int ch) {
    uint4* st = sbuf + (ch & 1) * kBigStageU4;
#pragma unroll
    for (int i = 0; i < kBigLW; ++i)
      __builtin_amdgcn_global_load_lds((bd_stream::glb_void_t*)(src[i] + (size_t)ch * 64),
                                       (bd_stream::lds_void_t*)(st + (wave + 8 * i) * 64), 16, 0, 0);
  };

  bd_f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = bd_f32x4{0.f, 0.f, 0.f, 0.f};
  const uint32_t sbase = bd_stream::lds_addr(sbuf);
  const uint32_t fo[2] = {(uint32_t)bd_stream::frag_offset(lane, 0), (uint32_t)bd_stream::frag_offset(lane, 1)};
  const uint32_t xt0 = wr * 8 * 2048, wt0 = (kBigRows / 16 + wc * 4) * 2048;  // this wave's first X / W tile

  issue(0);
  for (int ch = 0; ch < nch; ++ch) {
    __builtin_amdgcn_s_waitcnt(bd_stream::vmcnt_imm(0));
    bd_stream::pipe_barrier();  // chunk ch in LDS everywhere; the other stage is free
    if (ch + 1 < nch) issue(ch + 1);
    const uint32_t st = sbase + (ch & 1) * kBigStageU4 * 16;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      uint4 wb[4], xa[4];
      bd_stream::lds_frags_4x4(st + xt0 + fo[ks], st + wt0 + fo[ks], xa, wb);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = bd_mfma16(xa[i], wb[j], acc[i][j]);
      bd_stream::lds_frags_4(st + xt0 + 4 * 2048 + fo[ks], xa);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[4 + i][j] = bd_mfma16(xa[i], wb[j], acc[4 + i][j]);
    }
  }
  __syncthreads();  // the stages become the reduction buffer

  // acc[i][j][r]: row m0 + wr*128 + 16i + 4g + r, column n0 + wc*64 + 16j + l16
  BdArgStat* red = reinterpret_cast<BdArgStat*>(sbuf);  // [4 column waves][256 rows]
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int rl = wr * 128 + 16 * i + 4 * g + r;
      BdArgStat st{BD_NEG_INF, INT_MAX, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = n0 + wc * 64 + 16 * j + l16;
        const float v = acc[i][j][r];
        if (col < a.V && v > st.m) {
          st.m = v;
          st.i = col;
        }
      }
      float sum = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = n0 + wc * 64 + 16 * j + l16;
        if (col < a.V) sum += bd_exp2((acc[i][j][r] - st.m) * BD_LOG2E);
      }
      st.s = sum;
      if (a.logits != nullptr && m0 + rl < a.M) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int col = n0 + wc * 64 + 16 * j + l16;
          if (col < a.V) a.logits[(size_t)(m0 + rl) * a.V + col] = acc[i][j][r];
        }
      }
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) st = bd_stat_combine(st, bd_stat_shfl_xor(st, off));
      if (l16 == 0) red[wc * kBigRows + rl] = st;
    }
  }
  __syncthreads();
  if (tid < kBigRows && m0 + tid < a.M) {
    BdArgStat st = red[tid];
#pragma unroll
    for (int w = 1; w < 4; ++w) st = bd_stat_combine(st, red[w * kBigRows + tid]);
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
};

__global__ __launch_bounds__(kThreads) void lm_f32_kernel(LmF a) {
  __shared__ float sh[kF32Rows][kThreads];
  __shared__ BdArgStat red[kThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = blockIdx.x * kThreads + tid;
  const int m0 = blockIdx.y * kF32Rows;
  const float* hrow[kF32Rows];
#pragma unroll
  for (int r = 0; r < kF32Rows; ++r) {
    const int m = m0 + r;
    const int src = (m < a.M) ? (a.row_idx ? a.row_idx[m] : m) : -1;
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
    if (a.logits != nullptr && m < a.M && col < a.V) a.logits[(size_t)m * a.V + col] = acc[r];
    BdArgStat st = (col < a.V) ? BdArgStat{acc[r], col, 1.f} : BdArgStat{BD_NEG_INF, INT_MAX, 0.f};
    for (int off = 1; off < 64; off <<= 1) st = bd_stat_combine(st, bd_stat_shfl_xor(st, off));
    __syncthreads();
    if (lane == 0) red[wave] = st;
    __syncthreads();
    if (tid == 0 && m < a.M) {
      BdArgStat t = red[0];
      for (int w = 1; w < kThreads / 64; ++w) t = bd_stat_combine(t, red[w]);
      const size_t pi = (size_t)m * a.nvt + blockIdx.x;
      a.pmax[pi] = t.m;
      a.pidx[pi] = t.i;
      a.psum[pi] = t.s;
    }
  }
}

// Fold the tiles of each row in a fixed order; one work-group per row.
__global__ __launch_bounds__(kThreads) void lm_merge_kernel(const int32_t* row_idx, int n_src, int M,
                                                            int nvt, const float* pmax, const int32_t* pidx,
                                                            const float* psum, int32_t* argmax, float* conf,
                                                            float* max_logit, float* lse) {
  __shared__ BdArgStat red[kThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = blockIdx.x;
  BdArgStat st{BD_NEG_INF, INT_MAX, 0.f};
  for (int t = tid; t < nvt; t += kThreads) {
    const size_t pi = (size_t)m * nvt + t;
    st = bd_stat_combine(st, BdArgStat{pmax[pi], pidx[pi], psum[pi]});
  }
  for (int off = 32; off > 0; off >>= 1) st = bd_stat_combine(st, bd_stat_shfl_xor(st, off));
  if (lane == 0) red[wave] = st;
  __syncthreads();
  if (tid != 0) return;
  st = red[0];
  for (int w = 1; w < kThreads / 64; ++w) st = bd_stat_combine(st, red[w]);
  const int src = row_idx ? row_idx[m] : m;
  const bool ok = src >= 0 && src < n_src && st.s > 0.f;
  const float nan = __builtin_nanf("");
  argmax[m] = ok ? st.i : -1;
  conf[m] = ok ? 1.f / st.s : nan;
  if (max_logit != nullptr) max_logit[m] = ok ? st.m : nan;
  if (lse != nullptr) lse[m] = ok ? st.m + bd_log2(st.s) * BD_LN2 : nan;
}

}  // namespace

BdLmPlan bd_lm_plan(bd_dtype dt, int M, int hidden, int V) {
  BdLmPlan p{};
  if (dt == BD_F32) {
    p.cols_per_wg = kThreads;
    p.rows_per_wg = kF32Rows;
  } else if (M > 64) {
    p.cols_per_wg = kBigCols;
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
          x.M, x.hidden, x.V, p.nvt, x.pmax, x.pidx, x.psum};
    hipLaunchKernelGGL(lm_f32_kernel, grid, dim3(kThreads), 0, s, a);
  } else {
    LmK a{static_cast<const uint16_t*>(x.h), x.n_src, x.row_idx, static_cast<const uint16_t*>(x.w), x.logits,
          x.M, x.hidden, x.V, p.nvt, x.pmax, x.pidx, x.psum};
    switch (p.rows_per_wg / 16) {
      case kBigRows / 16: {
        const int cb8 = (p.nvt + 7) / 8 * 8;  // column blocks rounded up to whole XCD rounds
        hipLaunchKernelGGL(lm_big_kernel, dim3(cb8 * p.nmb), dim3(kBigThreads), 0, s, a, p.nmb, p.nvt);
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
                     p.nvt, x.pmax, x.pidx, x.psum, x.argmax, x.conf, x.max_logit, x.lse);
  return hipGetLastError();
}
