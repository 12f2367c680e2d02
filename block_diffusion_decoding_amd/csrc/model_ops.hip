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

// 16-byte vectors: 8 bf16 or 4 fp32 elements, unpacked to fp32.
template <typename T>
struct Vec;
template <>
struct Vec<uint16_t> {
  static constexpr int n = 8;
  static __device__ __forceinline__ void unpack(const uint4& u, float* f) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ uint4 pack(const float* f) {
    return make_uint4(bd_pack_bf2(f[0], f[1]), bd_pack_bf2(f[2], f[3]), bd_pack_bf2(f[4], f[5]),
                      bd_pack_bf2(f[6], f[7]));
  }
};
template <>
struct Vec<float> {
  static constexpr int n = 4;
  static __device__ __forceinline__ void unpack(const uint4& u, float* f) {
    f[0] = __uint_as_float(u.x);
    f[1] = __uint_as_float(u.y);
    f[2] = __uint_as_float(u.z);
    f[3] = __uint_as_float(u.w);
  }
  static __device__ __forceinline__ uint4 pack(const float* f) {
    return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3]));
  }
};

// The same normalisation in one pass when rows are whole 16-byte vectors and
// a row fits in R vectors per lane: every load of the row is in flight at
// once, the row stays in registers for the scaling, stores go out as 16-byte
// vectors.
constexpr int kNormR = 8;
template <typename T>
__global__ __launch_bounds__(kThreads) void rmsnorm_vec_kernel(int M, int nvec, const T* x, bd_rows xr, float eps,
                                                               T* y, bd_rows yr, float inv_hidden) {
  constexpr int VN = Vec<T>::n;
  const int m = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (m >= M) return;
  const uint4* xp = reinterpret_cast<const uint4*>(x + (size_t)bd_map_row(xr, m) * ((size_t)nvec * VN));
  uint4* yp = reinterpret_cast<uint4*>(y + (size_t)bd_map_row(yr, m) * ((size_t)nvec * VN));
  uint4 u[kNormR];
#pragma unroll
  for (int r = 0; r < kNormR; ++r)
    if (lane + 64 * r < nvec) u[r] = xp[lane + 64 * r];
  float ss = 0.f;
#pragma unroll
  for (int r = 0; r < kNormR; ++r)
    if (lane + 64 * r < nvec) {
      float f[VN];
      Vec<T>::unpack(u[r], f);
#pragma unroll
      for (int e = 0; e < VN; ++e) ss += f[e] * f[e];
    }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
  const float inv = 1.f / __builtin_sqrtf(ss * inv_hidden + eps);
#pragma unroll
  for (int r = 0; r < kNormR; ++r)
    if (lane + 64 * r < nvec) {
      float f[VN];
      Vec<T>::unpack(u[r], f);
#pragma unroll
      for (int e = 0; e < VN; ++e) f[e] *= inv;
      yp[lane + 64 * r] = Vec<T>::pack(f);
    }
}

// Rotary embedding in place: logical row m = b*n_rows + i (buffer row
// xr(m)) is at position pos_base[b] + pos_off + i; head h's dims j and
// j + d/2 (j < d/2) rotate by pos * theta^(-2j/d).  One thread per (row,
// group of kRopeHeads heads, pair index j): the angle does not depend on the
// head, so a thread takes its sine and cosine once and rotates the pair in
// each head of its group, all loads ahead of the stores.  The angle and its
// sine/cosine are taken in fp64 (positions reach the thousands, where an fp32
// angle would lose ~1e-4 rad); the rotation in fp32.
constexpr int kRopeHeads = 4;
template <typename T>
__global__ __launch_bounds__(kThreads) void rope_kernel(int B, int n_rows, int H, int d, T* x, bd_rows xr,
                                                        const int32_t* pos_base, int pos_off, double log2_theta) {
  const int half = d >> 1;
  const int ng = (H + kRopeHeads - 1) / kRopeHeads;
  const size_t total = (size_t)B * n_rows * ng * half;
  const size_t t = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (t >= total) return;
  const int j = (int)(t % half);
  const int hg = (int)((t / half) % ng);
  const int m = (int)(t / ((size_t)half * ng));
  const int b = m / n_rows, i = m % n_rows;
  const double pos = (double)(pos_base[b] + pos_off + i);
  const double ang = pos * exp2(-(2.0 * j / d) * log2_theta);
  double sn, cs;
  sincos(ang, &sn, &cs);
  const float c = (float)cs, s = (float)sn;
  const int h0 = hg * kRopeHeads;
  T* row = x + (size_t)bd_map_row(xr, m) * ((size_t)H * d) + (size_t)h0 * d + j;
  float x1[kRopeHeads], x2[kRopeHeads];
#pragma unroll
  for (int u = 0; u < kRopeHeads; ++u)
    if (h0 + u < H) {
      x1[u] = ld(row, (size_t)u * d);
      x2[u] = ld(row, (size_t)u * d + half);
    }
#pragma unroll
  for (int u = 0; u < kRopeHeads; ++u)
    if (h0 + u < H) {
      st(row, (size_t)u * d, x1[u] * c - x2[u] * s);
      st(row, (size_t)u * d + half, x2[u] * c + x1[u] * s);
    }
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

// The same gate on 16-byte vectors (inter a multiple of the vector width).
template <typename T>
__global__ __launch_bounds__(kThreads) void swiglu_vec_kernel(int M, int nvec, const T* gu, bd_rows gr, T* a,
                                                              bd_rows ar) {
  constexpr int VN = Vec<T>::n;
  const size_t total = (size_t)M * nvec;
  const size_t t = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (t >= total) return;
  const int v = (int)(t % nvec), m = (int)(t / nvec);
  const uint4* g = reinterpret_cast<const uint4*>(gu + (size_t)bd_map_row(gr, m) * (2 * (size_t)nvec * VN));
  const uint4 ug = g[v], uu = g[nvec + v];
  float z[VN], u[VN];
  Vec<T>::unpack(ug, z);
  Vec<T>::unpack(uu, u);
#pragma unroll
  for (int e = 0; e < VN; ++e) z[e] = z[e] / (1.f + __expf(-z[e])) * u[e];
  reinterpret_cast<uint4*>(a + (size_t)bd_map_row(ar, m) * ((size_t)nvec * VN))[v] = Vec<T>::pack(z);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

unsigned grid_for(size_t n) { return (unsigned)((n + kThreads - 1) / kThreads); }

}  // namespace

hipError_t bd_rmsnorm_launch(bd_dtype dt, int M, int hidden, const void* x, bd_rows xr, float eps, void* y,
                             bd_rows yr, hipStream_t s) {
  const dim3 grid((unsigned)((M + kThreads / 64 - 1) / (kThreads / 64)));
  const int vn = dt == BD_F32 ? 4 : 8;
  if (hidden % vn == 0 && hidden <= 64 * kNormR * vn && aligned16(x) && aligned16(y)) {
    const int nvec = hidden / vn;
    if (dt == BD_F32)
      hipLaunchKernelGGL(rmsnorm_vec_kernel<float>, grid, dim3(kThreads), 0, s, M, nvec,
                         static_cast<const float*>(x), xr, eps, static_cast<float*>(y), yr, 1.f / (float)hidden);
    else
      hipLaunchKernelGGL(rmsnorm_vec_kernel<uint16_t>, grid, dim3(kThreads), 0, s, M, nvec,
                         static_cast<const uint16_t*>(x), xr, eps, static_cast<uint16_t*>(y), yr,
                         1.f / (float)hidden);
    return hipGetLastError();
  }
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
  const size_t total = (size_t)B * n_rows * ((H + kRopeHeads - 1) / kRopeHeads) * (d / 2);
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
  const int vn = dt == BD_F32 ? 4 : 8;
  if (inter % vn == 0 && aligned16(gu) && aligned16(a)) {
    const int nvec = inter / vn;
    const unsigned g = grid_for((size_t)M * nvec);
    if (dt == BD_F32)
      hipLaunchKernelGGL(swiglu_vec_kernel<float>, dim3(g), dim3(kThreads), 0, s, M, nvec,
                         static_cast<const float*>(gu), gr, static_cast<float*>(a), ar);
    else
      hipLaunchKernelGGL(swiglu_vec_kernel<uint16_t>, dim3(g), dim3(kThreads), 0, s, M, nvec,
                         static_cast<const uint16_t*>(gu), gr, static_cast<uint16_t*>(a), ar);
    return hipGetLastError();
  }
  const size_t total = (size_t)M * inter;
  if (dt == BD_F32)
    hipLaunchKernelGGL(swiglu_kernel<float>, dim3(grid_for(total)), dim3(kThreads), 0, s, M, inter,
                       static_cast<const float*>(gu), gr, static_cast<float*>(a), ar);
  else
    hipLaunchKernelGGL(swiglu_kernel<uint16_t>, dim3(grid_for(total)), dim3(kThreads), 0, s, M, inter,
                       static_cast<const uint16_t*>(gu), gr, static_cast<uint16_t*>(a), ar);
  return hipGetLastError();
}
