// Layer pieces of the multi-layer decode beyond one attention layer:
// RMSNorm, rotary position embedding and the SwiGLU gate.
//
// The pages name the model family (Qwen2.5-style decoders adapted to block
// diffusion: "Fast-dLLM v2: Efficient Block-Diffusion LLM" notes, main-results
// table) but not its layer equations; these kernels implement that family's
// usual pieces: pre-norm RMSNorm with unit gains, rotate-half rotary embedding
// of queries and keys at absolute positions, and a SwiGLU MLP gate.  All are
// memory-bound elementwise or row-wise passes; they read and write each
// element once (bf16 or fp32 storage, fp32 arithmetic).
#include <cmath>

#include "bd_device.h"
#include "bd_launch.h"

namespace {

constexpr int kThreads = 256;

template <typename T>
__device__ __forceinline__ float ld(const T* p, size_t i);
template <>
__device__ __forceinline__ float ld<float>(const float* p, size_t i) { return p[i]; }
template <>
__device__ __forceinline__ float ld<uint16_t>(const uint16_t* p, size_t i) { return bd_bf2f(p[i]); }
template <typename T>
__device__ __forceinline__ void st(T* p, size_t i, float v);
template <>
__device__ __forceinline__ void st<float>(float* p, size_t i, float v) { p[i] = v; }
template <>
__device__ __forceinline__ void st<uint16_t>(uint16_t* p, size_t i, float v) { p[i] = (uint16_t)bd_f2bf(v); }

// y[yr(m)] = x[xr(m)] / sqrt(mean_k x^2 + eps): one wave per row, the sum of
// squares in fp32 over the row, then a second pass scales and stores (each
// element is read before it is written by the same lane, so x may be y).
template <typename T>
__global__ __launch_bounds__(kThreads) void rmsnorm_kernel(int M, int hidden, const T* x, bd_rows xr, float eps,
                                                           T* y, bd_rows yr) {
  const int m = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (m >= M) return;
  const T* xp = x + (size_t)bd_map_row(xr, m) * hidden;
  T* yp = y + (size_t)bd_map_row(yr, m) * hidden;
  float ss = 0.f;
  for (int k = lane; k < hidden; k += 64) {
    const float v = ld(xp, k);
    ss += v * v;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
  const float inv = 1.f / __builtin_sqrtf(ss / (float)hidden + eps);
  for (int k = lane; k < hidden; k += 64) st(yp, k, ld(xp, k) * inv);
}

// Rotary embedding in place: logical row m = b*n_rows + i (buffer row
// xr(m)) is at position pos_base[b] + pos_off + i; head h's dims j and
// j + d/2 (j < d/2) rotate by pos * theta^(-2j/d).  One thread per pair.
// The angle and its sine/cosine are taken in fp64 (positions reach the
// thousands, where an fp32 angle would lose ~1e-4 rad); the rotation in fp32.
template <typename T>
__global__ __launch_bounds__(kThreads) void rope_kernel(int B, int n_rows, int H, int d, T* x, bd_rows xr,
                                                        const int32_t* pos_base, int pos_off, double log2_theta) {
  const int half = d >> 1;
  const size_t total = (size_t)B * n_rows * H * half;
  const size_t t = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (t >= total) return;
  const int j = (int)(t % half);
  const int h = (int)((t / half) % H);
  const int m = (int)(t / ((size_t)half * H));
  const int b = m / n_rows, i = m % n_rows;
  const double pos = (double)(pos_base[b] + pos_off + i);
  const double ang = pos * exp2(-(2.0 * j / d) * log2_theta);
  double sn, cs;
  sincos(ang, &sn, &cs);
  T* row = x + (size_t)bd_map_row(xr, m) * ((size_t)H * d) + (size_t)h * d;
  const float x1 = ld(row, j), x2 = ld(row, j + half);
  const float c = (float)cs, s = (float)sn;
  st(row, j, x1 * c - x2 * s);
  st(row, j + half, x2 * c + x1 * s);
}

// a[ar(m), n] = silu(gu[gr(m), n]) * gu[gr(m), inter + n], silu(z) = z / (1 + e^-z):
// the rows of gu hold the gate projection, then the up projection.
template <typename T>
__global__ __launch_bounds__(kThreads) void swiglu_kernel(int M, int inter, const T* gu, bd_rows gr, T* a,
                                                          bd_rows ar) {
  const size_t total = (size_t)M * inter;
  const size_t t = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (t >= total) return;
  const int n = (int)(t % inter), m = (int)(t / inter);
  const T* g = gu + (size_t)bd_map_row(gr, m) * (2 * (size_t)inter);
  const float z = ld(g, n), u = ld(g, (size_t)inter + n);
  st(a + (size_t)bd_map_row(ar, m) * inter, n, z / (1.f + __expf(-z)) * u);
}

unsigned grid_for(size_t n) { return (unsigned)((n + kThreads - 1) / kThreads); }

}  // namespace

hipError_t bd_rmsnorm_launch(bd_dtype dt, int M, int hidden, const void* x, bd_rows xr, float eps, void* y,
                             bd_rows yr, hipStream_t s) {
  const dim3 grid((unsigned)((M + kThreads / 64 - 1) / (kThreads / 64)));
  if (dt == BD_F32)
    hipLaunchKernelGGL(rmsnorm_kernel<float>, grid, dim3(kThreads), 0, s, M, hidden, static_cast<const float*>(x),
                       xr, eps, static_cast<float*>(y), yr);
  else
    hipLaunchKernelGGL(rmsnorm_kernel<uint16_t>, grid, dim3(kThreads), 0, s, M, hidden,
                       static_cast<const uint16_t*>(x), xr, eps, static_cast<uint16_t*>(y), yr);
  return hipGetLastError();
}

hipError_t bd_rope_launch(bd_dtype dt, int B, int n_rows, int H, int d, void* x, bd_rows xr, const int32_t* pos_base,
                          int pos_off, float theta, hipStream_t s) {
  const size_t total = (size_t)B * n_rows * H * (d / 2);
  const double l2 = std::log2((double)theta);
  if (dt == BD_F32)
    hipLaunchKernelGGL(rope_kernel<float>, dim3(grid_for(total)), dim3(kThreads), 0, s, B, n_rows, H, d,
                       static_cast<float*>(x), xr, pos_base, pos_off, l2);
  else
    hipLaunchKernelGGL(rope_kernel<uint16_t>, dim3(grid_for(total)), dim3(kThreads), 0, s, B, n_rows, H, d,
                       static_cast<uint16_t*>(x), xr, pos_base, pos_off, l2);
  return hipGetLastError();
}

hipError_t bd_swiglu_launch(bd_dtype dt, int M, int inter, const void* gu, bd_rows gr, void* a, bd_rows ar,
                            hipStream_t s) {
  const size_t total = (size_t)M * inter;
  if (dt == BD_F32)
    hipLaunchKernelGGL(swiglu_kernel<float>, dim3(grid_for(total)), dim3(kThreads), 0, s, M, inter,
                       static_cast<const float*>(gu), gr, static_cast<float*>(a), ar);
  else
    hipLaunchKernelGGL(swiglu_kernel<uint16_t>, dim3(grid_for(total)), dim3(kThreads), 0, s, M, inter,
                       static_cast<const uint16_t*>(gu), gr, static_cast<uint16_t*>(a), ar);
  return hipGetLastError();
}
