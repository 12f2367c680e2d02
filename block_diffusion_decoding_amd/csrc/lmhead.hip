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
// bf16: streaming MFMA GEMM (stream_gemm.h), weights streamed once from HBM
// through a 3-stage asynchronous global->LDS pipeline, up to 64 rows per
// work-group.  fp32: plain VALU kernel.
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
