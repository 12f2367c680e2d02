// Support kernels of the refinement step: input rows and projections.
//
// Input rows: "Fast-dLLM v2: Efficient Block-Diffusion LLM" notes, Key design 2
// -- a masked position takes the learnable [MASK] embedding.  Projections:
// the Q/K/V projections of the block rows (fresh rows write their K/V into
// the in-block buffer, Key design 3) and the attention output projection
// with its residual.
//
// bf16 projections use the streaming MFMA core of stream_gemm.h with a plain
// store epilogue (plus residual); up to three weight matrices (Q, K, V) share
// one launch, and K is split over work-groups when the column tiles alone
// cannot fill the GPU.
#include "bd_device.h"
#include "bd_launch.h"
#include "stream_gemm.h"

namespace {

constexpr int kThreads = 256;
// Tiling; defaults chosen by measurement, overridable at build time.
#ifndef BD_GEMM_NTW
#define BD_GEMM_NTW 4
#endif
#ifndef BD_GEMM_TARGET_WGS
#define BD_GEMM_TARGET_WGS 512
#endif
#ifndef BD_GEMM_MIN_CHUNKS
#define BD_GEMM_MIN_CHUNKS 4
#endif
#ifndef BD_GEMM_NTW_M64
#define BD_GEMM_NTW_M64 4
#endif
// 16-column tiles per work-group: narrower at 64 rows (more column work-groups,
// a smaller K split, half the partial sums to add)
__host__ __device__ constexpr int ntw_for(int MT) { return MT == 4 ? BD_GEMM_NTW_M64 : BD_GEMM_NTW; }
#ifndef BD_GEMM_NS
#define BD_GEMM_NS 3
#endif
constexpr int kNS = BD_GEMM_NS;          // pipeline stages
constexpr int kMaxSeg = 3;
constexpr int kTargetWGs = BD_GEMM_TARGET_WGS;
constexpr int kMinChunksPerSplit = BD_GEMM_MIN_CHUNKS;

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
  int ksplit;
  float* part;    // [tiles][ksplit][MT*16 x 64] fp32 partial sums (ksplit > 1)
};

__device__ __forceinline__ void gemm_store(const GemmK& a, int seg, int m, int col, float v) {
  const int N = a.N[seg];
  if (a.res[seg]) v += bd_bf2f(a.res[seg][(size_t)bd_map_row(a.rr[seg], m) * N + col]);
  a.y[seg][(size_t)bd_map_row(a.yr[seg], m) * N + col] = (uint16_t)bd_f2bf(v);
}

// One (column tile, row tile, K slice) per work-group.  With a K split the
// slices write fp32 partial tiles that gemm_reduce_kernel adds in slice order
// (a separate launch: cross-XCD visibility inside one kernel would need
// device-scope fences, i.e. L2 write-backs, per work-group).
template <int MT>
__global__ __launch_bounds__(kThreads, 2) void gemm_bf16_kernel(GemmK a) {
  constexpr int kNTW = ntw_for(MT);
  using C = bd_stream::Cfg<MT, kNTW, kNS>;
  constexpr int TILE = MT * 16 * kNTW * 16;
  __shared__ uint4 sbuf[C::NS * C::STAGE_U4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int wm = wave % C::WM, wn = wave / C::WM;
  const int bx = blockIdx.x;
  const int seg = (a.nseg > 2 && bx >= a.wg_begin[2]) ? 2 : (a.nseg > 1 && bx >= a.wg_begin[1]) ? 1 : 0;
  const int N = a.N[seg];
  const int n0 = (bx - a.wg_begin[seg]) * kNTW * 16;
  const int m0 = blockIdx.y * MT * 16;
  const int z = blockIdx.z;
  const int nch = a.K / C::KC;
  const int c0 = z * nch / a.ksplit, c1 = (z + 1) * nch / a.ksplit;

  auto xidx = [](int m) { return m; };
  auto xptr = [&](int m, int) -> const uint16_t* {
    return m < a.M ? a.x + (size_t)bd_map_row(a.xr, m) * a.K : nullptr;
  };
  bd_f32x4 acc[C::MTW][C::NTP];
  bd_stream::mainloop<C>(xidx, xptr, a.x, m0, a.w[seg], N, a.K, n0, sbuf, acc, c0 * C::KC, c1 - c0);

  if (a.ksplit == 1) {
#pragma unroll
    for (int i = 0; i < C::MTW; ++i)
#pragma unroll
      for (int j = 0; j < C::NTP; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = m0 + (wm * C::MTW + i) * 16 + 4 * g + r;
          const int col = n0 + (wn * C::NTP + j) * 16 + l16;
          if (m < a.M && col < N) gemm_store(a, seg, m, col, acc[i][j][r]);
        }
    return;
  }
  const int tile = blockIdx.y * gridDim.x + bx;
  float* pt = a.part + ((size_t)tile * a.ksplit + z) * TILE;
#pragma unroll
  for (int i = 0; i < C::MTW; ++i)
#pragma unroll
    for (int j = 0; j < C::NTP; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        pt[((wm * C::MTW + i) * 16 + 4 * g + r) * (kNTW * 16) + (wn * C::NTP + j) * 16 + l16] = acc[i][j][r];
}

// Adds the K slices of every tile in slice order, then residual and store.
template <int MT>
__global__ __launch_bounds__(kThreads) void gemm_reduce_kernel(GemmK a) {
  constexpr int kNTW = ntw_for(MT);
  constexpr int TILE = MT * 16 * kNTW * 16;
  const int bx = blockIdx.x;
  const int seg = (a.nseg > 2 && bx >= a.wg_begin[2]) ? 2 : (a.nseg > 1 && bx >= a.wg_begin[1]) ? 1 : 0;
  const int N = a.N[seg];
  const int n0 = (bx - a.wg_begin[seg]) * kNTW * 16;
  const int m0 = blockIdx.y * MT * 16;
  const float* p0 = a.part + (size_t)(blockIdx.y * gridDim.x + bx) * a.ksplit * TILE;
  // blockIdx.z: which 16-row group of the tile this work-group adds
  for (int e = blockIdx.z * 16 * kNTW * 16 + threadIdx.x * 4; e < (blockIdx.z + 1) * 16 * kNTW * 16;
       e += kThreads * 4) {
    const int m = m0 + e / (kNTW * 16), col = n0 + e % (kNTW * 16);
    if (m >= a.M) break;
    float4 v = *reinterpret_cast<const float4*>(p0 + e);
    for (int zz = 1; zz < a.ksplit; ++zz) {
      const float4 w = *reinterpret_cast<const float4*>(p0 + (size_t)zz * TILE + e);
      v.x += w.x;
      v.y += w.y;
      v.z += w.z;
      v.w += w.w;
    }
    const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (col + u < N) gemm_store(a, seg, m, col + u, vv[u]);
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
  constexpr int PER = 16 / sizeof(T);  // elements per 16-byte access
  for (int e = threadIdx.x * PER; e < hidden; e += kThreads * PER) {
    uint4 ev = *reinterpret_cast<const uint4*>(er + e);
    uint4 out;
    if constexpr (sizeof(T) == 2) {
      uint4 pv = pr ? *reinterpret_cast<const uint4*>(pr + e) : make_uint4(0, 0, 0, 0);
      const uint32_t* ew = reinterpret_cast<const uint32_t*>(&ev);
      const uint32_t* pw = reinterpret_cast<const uint32_t*>(&pv);
      uint32_t* ow = reinterpret_cast<uint32_t*>(&out);
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        if (!ok) {
          ow[h] = 0x7fc07fc0u;
        } else if (pr) {
          ow[h] = bd_pack_bf2(bd_bf2f(ew[h] & 0xffffu) + bd_bf2f(pw[h] & 0xffffu),
                              bd_bf2f(ew[h] >> 16) + bd_bf2f(pw[h] >> 16));
        } else {
          ow[h] = ew[h];
        }
      }
    } else {
      float4 f = __builtin_bit_cast(float4, ev);
      if (pr) {
        const float4 p = *reinterpret_cast<const float4*>(pr + e);
        f.x += p.x; f.y += p.y; f.z += p.z; f.w += p.w;
      }
      if (!ok) f = make_float4(__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""));
      out = __builtin_bit_cast(uint4, f);
    }
    *reinterpret_cast<uint4*>(xr + e) = out;
  }
}

}  // namespace

BdGemmPlan bd_gemm_plan(bd_dtype dt, int M, int K, const int* N, int nseg) {
  BdGemmPlan p{};
  if (dt == BD_F32) return p;
  const int mt = (M + 15) / 16;
  p.MT = mt <= 1 ? 1 : (mt == 2 ? 2 : 4);
  const int kNTW = ntw_for(p.MT);
  p.nx = 0;
  for (int i = 0; i < nseg; ++i) p.nx += (N[i] + kNTW * 16 - 1) / (kNTW * 16);
  p.ny = (M + p.MT * 16 - 1) / (p.MT * 16);
  const int nch = K / 64;
  const long base = (long)p.nx * p.ny;
  int ks = (int)((kTargetWGs + base - 1) / base);
  const int maxks = nch / kMinChunksPerSplit;
  ks = ks > maxks ? maxks : ks;
  p.ksplit = ks < 1 ? 1 : ks;
  if (p.ksplit > 1) p.ws_bytes = (size_t)p.nx * p.ny * p.ksplit * p.MT * 16 * kNTW * 16 * sizeof(float);
  return p;
}

hipError_t bd_gemm_launch(bd_dtype dt, const BdGemmPlan& p, int M, int K, const void* x, bd_rows xr,
                          const BdGemmSeg* segs, int nseg, void* workspace, hipStream_t s) {
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
  int wg = 0;
  for (int i = 0; i < nseg; ++i) {
    a.w[i] = static_cast<const uint16_t*>(segs[i].w);
    a.y[i] = static_cast<uint16_t*>(segs[i].y);
    a.res[i] = static_cast<const uint16_t*>(segs[i].res);
    a.yr[i] = segs[i].yr;
    a.rr[i] = segs[i].rr;
    a.N[i] = segs[i].N;
    a.wg_begin[i] = wg;
    wg += (segs[i].N + ntw_for(p.MT) * 16 - 1) / (ntw_for(p.MT) * 16);
  }
  for (int i = nseg; i <= kMaxSeg; ++i) a.wg_begin[i] = wg;
  a.ksplit = p.ksplit;
  a.part = p.ksplit > 1 ? static_cast<float*>(workspace) : nullptr;
  const dim3 grid(wg, p.ny, p.ksplit);
  switch (p.MT) {
    case 1: hipLaunchKernelGGL(gemm_bf16_kernel<1>, grid, dim3(kThreads), 0, s, a); break;
    case 2: hipLaunchKernelGGL(gemm_bf16_kernel<2>, grid, dim3(kThreads), 0, s, a); break;
    default: hipLaunchKernelGGL(gemm_bf16_kernel<4>, grid, dim3(kThreads), 0, s, a); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.ksplit == 1) return e;
  const dim3 rgrid(wg, p.ny, p.MT);
  switch (p.MT) {
    case 1: hipLaunchKernelGGL(gemm_reduce_kernel<1>, rgrid, dim3(kThreads), 0, s, a); break;
    case 2: hipLaunchKernelGGL(gemm_reduce_kernel<2>, rgrid, dim3(kThreads), 0, s, a); break;
    default: hipLaunchKernelGGL(gemm_reduce_kernel<4>, rgrid, dim3(kThreads), 0, s, a); break;
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
