// Support kernels of the refinement step: input rows and projections.
//
// Input rows: "Fast-dLLM v2: Efficient Block-Diffusion LLM" notes, Key design 2
// -- a masked position takes the learnable [MASK] embedding.  Projections:
// the Q/K/V projections of the block rows (fresh rows write their K/V into
// the in-block buffer, Key design 3) and the attention output projection
// with its residual.
//
// bf16 projections use the skinny MFMA core of skinny_gemm.h with a plain
// store epilogue; up to three weight matrices (Q, K, V) share one launch.
#include "bd_device.h"
#include "bd_launch.h"
#include "skinny_gemm.h"

namespace {

constexpr int kThreads = 256;
constexpr int kNT = 1;
constexpr int kKC = 256;
constexpr int kMaxSeg = 3;

struct GemmK {
  const uint16_t* x;
  bd_rows xr;
  int M, K, nseg;
  const uint16_t* w[kMaxSeg];
  uint16_t* y[kMaxSeg];
  const uint16_t* res[kMaxSeg];
  bd_rows yr[kMaxSeg];
  bd_rows rr[kMaxSeg];
  int N[kMaxSeg];
  int wg_begin[kMaxSeg + 1];
};

template <int MT>
__global__ __launch_bounds__(kThreads) void gemm_bf16_kernel(GemmK a) {
  using XS = bd_skinny::XStage<MT, kKC>;
  __shared__ uint4 sX[2 * XS::LDS_U4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int bx = blockIdx.x;
  const int seg = (a.nseg > 2 && bx >= a.wg_begin[2]) ? 2 : (a.nseg > 1 && bx >= a.wg_begin[1]) ? 1 : 0;
  const int N = a.N[seg];
  const int col0 = ((bx - a.wg_begin[seg]) * 4 + wave) * kNT * 16;
  const int m0 = blockIdx.y * MT * 16;

  auto xrow = [&](int m) -> const uint16_t* {
    return m < a.M ? a.x + (size_t)bd_map_row(a.xr, m) * a.K : nullptr;
  };
  bd_f32x4 acc[MT][kNT];
  bd_skinny::mainloop<MT, kNT, kKC>(xrow, m0, a.w[seg], N, a.K, col0, sX, acc);

  uint16_t* y = a.y[seg];
  const uint16_t* res = a.res[seg];
  const bd_rows yr = a.yr[seg], rr = a.rr[seg];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + mt * 16 + 4 * g + r;
      if (m >= a.M) continue;
      const size_t yrow = (size_t)bd_map_row(yr, m) * N;
      const size_t rrow = res ? (size_t)bd_map_row(rr, m) * N : 0;
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) {
        const int col = col0 + nt * 16 + l16;
        if (col >= N) continue;
        float v = acc[mt][nt][r];
        if (res) v += bd_bf2f(res[rrow + col]);
        y[yrow + col] = (uint16_t)bd_f2bf(v);
      }
    }
}

struct GemmF {
  const float* x;
  bd_rows xr;
  int M, K;
  const float* w;
  float* y;
  const float* res;
  bd_rows yr, rr;
  int N;
};

__global__ __launch_bounds__(kThreads) void gemm_f32_kernel(GemmF a) {
  const int n = blockIdx.x * kThreads + threadIdx.x;
  const int m = blockIdx.y;
  if (n >= a.N) return;
  const float* xr = a.x + (size_t)bd_map_row(a.xr, m) * a.K;
  const float* wr = a.w + (size_t)n * a.K;
  float acc = 0.f;
  for (int k = 0; k < a.K; ++k) acc += xr[k] * wr[k];
  if (a.res) acc += a.res[(size_t)bd_map_row(a.rr, m) * a.N + n];
  a.y[(size_t)bd_map_row(a.yr, m) * a.N + n] = acc;
}

// Input rows of the block: E[token] or the [MASK] row, plus an optional offset.
template <typename T>
__global__ __launch_bounds__(kThreads) void embed_kernel(int D, int row_off, int n_rows, int hidden, int V,
                                                         const T* E, const int32_t* tokens,
                                                         const uint64_t* mask_bits, const T* plant, T* x) {
  const int i = blockIdx.x, b = blockIdx.y;
  const int pos = row_off + i;
  const bool masked = mask_bits != nullptr && ((mask_bits[b] >> pos) & 1ull);
  const int tok = tokens[(size_t)b * D + pos];
  const bool ok = masked || (tok >= 0 && tok < V);
  const T* er = E + (size_t)(masked ? V : (ok ? tok : 0)) * hidden;
  const T* pr = plant ? plant + ((size_t)b * D + pos) * hidden : nullptr;
  T* xr = x + ((size_t)b * n_rows + i) * hidden;
  for (int e = threadIdx.x; e < hidden; e += kThreads) {
    float v;
    if constexpr (sizeof(T) == 2) {
      v = bd_bf2f(er[e]);
      if (pr) v += bd_bf2f(pr[e]);
      xr[e] = ok ? (T)bd_f2bf(v) : (T)0x7fc0u;
    } else {
      v = er[e];
      if (pr) v += pr[e];
      xr[e] = ok ? v : __builtin_nanf("");
    }
  }
}

}  // namespace

hipError_t bd_gemm_launch(bd_dtype dt, int M, int K, const void* x, bd_rows xr, const BdGemmSeg* segs,
                          int nseg, hipStream_t s) {
  if (dt == BD_F32) {
    for (int i = 0; i < nseg; ++i) {
      GemmF a{static_cast<const float*>(x), xr, M, K, static_cast<const float*>(segs[i].w),
              static_cast<float*>(segs[i].y), static_cast<const float*>(segs[i].res), segs[i].yr, segs[i].rr,
              segs[i].N};
      hipLaunchKernelGGL(gemm_f32_kernel, dim3((segs[i].N + kThreads - 1) / kThreads, M), dim3(kThreads), 0, s,
                         a);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  GemmK a{};
  a.x = static_cast<const uint16_t*>(x);
  a.xr = xr;
  a.M = M;
  a.K = K;
  a.nseg = nseg;
  const int cols_per_wg = 4 * kNT * 16;
  int wg = 0;
  for (int i = 0; i < nseg; ++i) {
    a.w[i] = static_cast<const uint16_t*>(segs[i].w);
    a.y[i] = static_cast<uint16_t*>(segs[i].y);
    a.res[i] = static_cast<const uint16_t*>(segs[i].res);
    a.yr[i] = segs[i].yr;
    a.rr[i] = segs[i].rr;
    a.N[i] = segs[i].N;
    a.wg_begin[i] = wg;
    wg += (segs[i].N + cols_per_wg - 1) / cols_per_wg;
  }
  for (int i = nseg; i <= kMaxSeg; ++i) a.wg_begin[i] = wg;
  const int mt = (M + 15) / 16;
  const int MT = mt > 4 ? 4 : mt;
  const dim3 grid(wg, (M + MT * 16 - 1) / (MT * 16));
  switch (MT) {
    case 1: hipLaunchKernelGGL(gemm_bf16_kernel<1>, grid, dim3(kThreads), 0, s, a); break;
    case 2: hipLaunchKernelGGL(gemm_bf16_kernel<2>, grid, dim3(kThreads), 0, s, a); break;
    case 3: hipLaunchKernelGGL(gemm_bf16_kernel<3>, grid, dim3(kThreads), 0, s, a); break;
    default: hipLaunchKernelGGL(gemm_bf16_kernel<4>, grid, dim3(kThreads), 0, s, a); break;
  }
  return hipGetLastError();
}

hipError_t bd_embed_launch(bd_dtype dt, int B, int D, int row_off, int n_rows, int hidden, int V, const void* E,
                           const int32_t* tokens, const uint64_t* mask_bits, const void* plant, void* x,
                           hipStream_t s) {
  const dim3 grid(n_rows, B);
  if (dt == BD_F32)
    hipLaunchKernelGGL(embed_kernel<float>, grid, dim3(kThreads), 0, s, D, row_off, n_rows, hidden, V,
                       static_cast<const float*>(E), tokens, mask_bits, static_cast<const float*>(plant),
                       static_cast<float*>(x));
  else
    hipLaunchKernelGGL(embed_kernel<uint16_t>, grid, dim3(kThreads), 0, s, D, row_off, n_rows, hidden, V,
                       static_cast<const uint16_t*>(E), tokens, mask_bits, static_cast<const uint16_t*>(plant),
                       static_cast<uint16_t*>(x));
  return hipGetLastError();
}
