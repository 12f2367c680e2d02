// Training form of block diffusion (forward pass and loss value): attention
// over the 2L layout and the token-shift cross-entropy terms.
//
// "Fast-dLLM v2: Efficient Block-Diffusion LLM" notes, Key design 2: the
// noisy sequence x_t (masked positions replaced by [MASK]) and the clean x_0
// are concatenated into 2L positions and attended under one hybrid mask; the
// loss is the cross-entropy of the masked tokens, each predicted from the
// logits of the position before it.
//
// The attention reuses the refinement-step kernel (attn.hip).  Under the 2L
// mask, the D noisy rows of block b see exactly their own noisy block and
// the clean rows of blocks < b, and the D clean rows of block b see their
// own clean block and the clean rows of blocks < b: both are "a block over a
// prefix cache" with the clean rows of the sample as the cache and the
// block's own D rows as the in-block keys (all visible).  So every (sample,
// half, block) is one entry of the step kernel, entries of one sample share
// one cache slab, and entry (s, h, b) has b*D cached rows.  Its in-block rows
// are rows [b*D, b*D + D) of that half: in the [S, 2L, H, d] layout these are
// consecutive D-row groups, entry e owning rows e*D .. e*D + D - 1, so q, the
// in-block K/V and o need no copy.  Only the clean K/V are rewritten once
// into the cache layout [S, Hkv, L, d] (a (sample, KV head) slab is one
// contiguous stream, as for the inference cache).
#include "bd_device.h"
#include "bd_launch.h"

namespace {

constexpr int kThreads = 256;

// Clean K/V rows L .. 2L-1 of each sample -> cache [S, Hkv, L, d], one thread
// per 16 bytes; threads e < E also write entry e's cached length.
template <typename T>
__global__ __launch_bounds__(kThreads) void train_prep_kernel(int S, int L, int D, int Hkv, int d, const T* k,
                                                              const T* v, T* kc, T* vc, int32_t* kv_len) {
  constexpr int VN = 16 / sizeof(T);
  const size_t t = (size_t)blockIdx.x * kThreads + threadIdx.x;
  const int nb = L / D;
  if (t < (size_t)S * 2 * nb) kv_len[t] = (int)(t % nb) * D;
  const int dv = d / VN;
  const size_t total = (size_t)S * L * Hkv * dv;
  if (t >= total) return;
  const int e = (int)(t % dv);
  const int h = (int)((t / dv) % Hkv);
  const int r = (int)((t / ((size_t)dv * Hkv)) % L);
  const int s = (int)(t / ((size_t)dv * Hkv * L));
  const size_t src = (((size_t)s * 2 * L + L + r) * Hkv + h) * d + (size_t)e * VN;
  const size_t dst = (((size_t)s * Hkv + h) * L + r) * d + (size_t)e * VN;
  *reinterpret_cast<uint4*>(kc + dst) = *reinterpret_cast<const uint4*>(k + src);
  *reinterpret_cast<uint4*>(vc + dst) = *reinterpret_cast<const uint4*>(v + src);
}

template <typename T>
__device__ __forceinline__ void unpack16(const uint4& u, float* f);
template <>
__device__ __forceinline__ void unpack16<uint16_t>(const uint4& u, float* f) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
template <>
__device__ __forceinline__ void unpack16<float>(const uint4& u, float* f) {
  f[0] = __uint_as_float(u.x);
  f[1] = __uint_as_float(u.y);
  f[2] = __uint_as_float(u.z);
  f[3] = __uint_as_float(u.w);
}

// nll[m] = lse[m] - h[row(m)] . w[target[m]] (fp32 dot product), one wave per
// row; an invalid row index or target gives NaN.
template <typename T>
__global__ __launch_bounds__(kThreads) void nll_kernel(int M, int hidden, int V, const T* h, int n_src,
                                                       const int32_t* row_idx, const T* w, const int32_t* target,
                                                       const float* lse, float* nll) {
  constexpr int VN = 16 / sizeof(T);
  const int m = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (m >= M) return;
  const int r = row_idx ? row_idx[m] : m;
  const int tg = target[m];
  if (r < 0 || r >= n_src || tg < 0 || tg >= V) {
    if (lane == 0) nll[m] = __builtin_nanf("");
    return;
  }
  const uint4* hp = reinterpret_cast<const uint4*>(h + (size_t)r * hidden);
  const uint4* wp = reinterpret_cast<const uint4*>(w + (size_t)tg * hidden);
  float acc = 0.f;
  for (int i = lane; i < hidden / VN; i += 64) {
    float a[VN], b[VN];
    unpack16<T>(hp[i], a);
    unpack16<T>(wp[i], b);
#pragma unroll
    for (int e = 0; e < VN; ++e) acc += a[e] * b[e];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (lane == 0) nll[m] = lse[m] - acc;
}

// loss[0] = sum of nll[0 .. M-1]: one work-group, fp64 partial sums in a
// fixed order (thread t adds rows t, t + 256, ...; then a fixed tree).
__global__ __launch_bounds__(kThreads) void nll_sum_kernel(int M, const float* nll, float* loss) {
  __shared__ double part[kThreads];
  double s = 0.0;
  for (int m = threadIdx.x; m < M; m += kThreads) s += (double)nll[m];
  part[threadIdx.x] = s;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) loss[0] = (float)part[0];
}

unsigned grid_for(size_t n) { return (unsigned)((n + kThreads - 1) / kThreads); }
size_t round256(size_t n) { return (n + 255) / 256 * 256; }

}  // namespace

BdTrainPlan bd_train_plan(bd_dtype dt, int S, int L, int D, int Hq, int Hkv, int d) {
  BdTrainPlan p{};
  const int E = S * 2 * (L / D);
  p.attn = bd_attn_plan(dt, E, Hq, Hkv, d, D, L, D);
  const size_t elem = dt == BD_F32 ? 4 : 2;
  p.cache_bytes = round256((size_t)S * Hkv * L * d * elem);
  p.len_off = 2 * p.cache_bytes;
  p.attn_off = p.len_off + round256((size_t)E * sizeof(int32_t));
  p.ws_bytes = p.attn_off + p.attn.ws_bytes;
  return p;
}

hipError_t bd_train_attn_launch(bd_dtype dt, const BdTrainPlan& p, int S, int L, int D, int Hq, int Hkv, int d,
                                const void* q, const void* k, const void* v, float scale, void* o,
                                void* workspace, hipStream_t s) {
  char* ws = static_cast<char*>(workspace);
  void* kc = ws;
  void* vc = ws + p.cache_bytes;
  int32_t* kv_len = reinterpret_cast<int32_t*>(ws + p.len_off);
  const int E = S * 2 * (L / D);
  const size_t vn = dt == BD_F32 ? 4 : 8;
  size_t n = (size_t)S * L * Hkv * (d / vn);
  n = n > (size_t)E ? n : (size_t)E;
  if (dt == BD_F32)
    hipLaunchKernelGGL(train_prep_kernel<float>, dim3(grid_for(n)), dim3(kThreads), 0, s, S, L, D, Hkv, d,
                       static_cast<const float*>(k), static_cast<const float*>(v), static_cast<float*>(kc),
                       static_cast<float*>(vc), kv_len);
  else
    hipLaunchKernelGGL(train_prep_kernel<uint16_t>, dim3(grid_for(n)), dim3(kThreads), 0, s, S, L, D, Hkv, d,
                       static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), static_cast<uint16_t*>(kc),
                       static_cast<uint16_t*>(vc), kv_len);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  BdAttnArgs a{};
  a.q = q;
  a.k_cache = kc;
  a.v_cache = vc;
  a.kv_len = kv_len;
  a.k_blk = k;   // entry e's D in-block rows are rows e*D .. of the [S*2L, Hkv, d] layout
  a.v_blk = v;
  a.o = o;
  a.lse = nullptr;
  char* aw = ws + p.attn_off;
  a.part_o = p.attn.ws_bytes ? reinterpret_cast<float*>(aw + p.attn.part_o) : nullptr;
  a.part_ml = p.attn.ws_bytes ? reinterpret_cast<float*>(aw + p.attn.part_ml) : nullptr;
  a.B = E;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = Hq / Hkv;
  a.d = d;
  a.D = D;
  a.n_q = D;
  a.q_off = 0;
  a.cap = L;
  a.n_blk = D;
  a.epc = 2 * (L / D);
  a.scale = scale;
  return bd_attn_launch(dt, p.attn, a, s);
}

hipError_t bd_nll_launch(bd_dtype dt, int M, int hidden, int V, const void* h, int n_src, const int32_t* row_idx,
                         const void* w, const int32_t* target, const float* lse, float* nll, float* loss,
                         hipStream_t s) {
  const dim3 grid((unsigned)((M + kThreads / 64 - 1) / (kThreads / 64)));
  if (dt == BD_F32)
    hipLaunchKernelGGL(nll_kernel<float>, grid, dim3(kThreads), 0, s, M, hidden, V, static_cast<const float*>(h),
                       n_src, row_idx, static_cast<const float*>(w), target, lse, nll);
  else
    hipLaunchKernelGGL(nll_kernel<uint16_t>, grid, dim3(kThreads), 0, s, M, hidden, V,
                       static_cast<const uint16_t*>(h), n_src, row_idx, static_cast<const uint16_t*>(w), target,
                       lse, nll);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || loss == nullptr) return e;
  hipLaunchKernelGGL(nll_sum_kernel, dim3(1), dim3(kThreads), 0, s, M, nll, loss);
  return hipGetLastError();
}
