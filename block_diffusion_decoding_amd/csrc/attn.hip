// Hybrid-mask grouped-query attention of one block-diffusion refinement step.
//
// Method: "Fast-dLLM v2: Efficient Block-Diffusion LLM" notes, Framework and
// Key design 2 -- attention is bidirectional inside a block and causal across
// blocks, and the queries of the current block see every committed position
// plus the whole current block (masked positions included); Key design 3 --
// committed blocks are read from a block-level KV cache and, in a DualCache
// step, the in-block K/V outside the active sub-block come from a snapshot.
//
// bf16 path (MFMA): one work-group handles (sequence b, KV head, key chunk,
// query-tile group).  The G query heads that share a KV head and the n_q fresh
// block rows form R = n_q * G query rows; this is what turns the grouped-query
// attention into a real contraction for v_mfma_f32_16x16x32_bf16.  K and V
// tiles of KT keys are staged through LDS (K row-major with an XOR swizzle,
// V transposed) with a register prefetch of the next tile; the scores are
// computed transposed (S^T = K Q^T) so that the probabilities land in the B
// operand layout of the P.V product without any data movement; the softmax is
// an online (running max) softmax in base 2.  Key chunks of one (sequence, KV
// head) are merged by a second kernel when a sequence needs more than one.
//
// fp32 path: a plain VALU kernel (one work-group per query row and head),
// used for the tiny fp32 workload.
#include <climits>

#include "bd_device.h"
#include "bd_launch.h"

namespace {

constexpr int kThreads = 256;
constexpr int kKT = 64;         // keys per LDS tile (bf16 path)
constexpr int kXcd = 8;         // work-groups are dispatched round-robin over 8 XCDs
constexpr int kMinChunk = 512;  // keys per work item, lower bound
constexpr int kTargetWGs = 1024;

struct AttnK {
  const uint16_t* q;
  const uint16_t* kc;
  const uint16_t* vc;
  const int32_t* kv_len;
  const uint16_t* kb;
  const uint16_t* vb;
  uint16_t* o;
  float* lse;
  float* part_o;
  float* part_ml;
  int B, Hq, Hkv, G, D, n_q, q_off, cap, n_blk;
  int R, QT, nqg, chunk, nchunks, n_units;
  float scale_log2;
};

__device__ __forceinline__ uint32_t half16(const uint4& v, int e) {
  const uint32_t w = (e < 2) ? v.x : (e < 4) ? v.y : (e < 6) ? v.z : v.w;
  return (e & 1) ? (w >> 16) : (w & 0xffffu);
}

template <int DH, int KT, int QPW>
__global__ __launch_bounds__(kThreads) void attn_bf16_kernel(AttnK a) {
  constexpr int KCH = DH / 8;         // 16-byte chunks per key row
  constexpr int VP = KT + 4;          // row pitch (elements) of the transposed V tile
  constexpr int NKL = KT * KCH / kThreads;
  constexpr int NVT = (KT / 4) * KCH; // V tasks: 4 keys x 8 head-dim elements
  constexpr int KS = DH / 32;         // MFMA K-steps over the head dim
  constexpr int NKT = KT / 16;        // 16-key tiles per LDS tile
  static_assert(NKL >= 1 && KT * KCH % kThreads == 0, "K tile split");
  static_assert(NVT <= kThreads, "V tile split");

  __shared__ uint4 sK[2][KT * KCH];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][DH * VP];

  // ---- work item (XCD-aware: the query groups of one key chunk share an XCD)
  const int wid = blockIdx.x;
  const int xcd = wid % kXcd;
  const int t8 = wid / kXcd;
  const int qg = t8 % a.nqg;
  const int unit = (t8 / a.nqg) * kXcd + xcd;
  if (unit >= a.n_units) return;
  const int c = unit % a.nchunks;
  const int bh = unit / a.nchunks;
  const int kvh = bh % a.Hkv;
  const int b = bh / a.Hkv;

  int L = a.kv_len[b];
  L = L < 0 ? 0 : (L > a.cap ? a.cap : L);
  const int T = L + a.n_blk;
  const int kbeg = c * a.chunk;
  if (kbeg >= T) return;
  const int kend = min(T, kbeg + a.chunk);
  const bool single = (kbeg == 0 && kend == T);
  const int ntiles = (kend - kbeg + KT - 1) / KT;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;
  const int l16 = lane & 15;

  const uint16_t* kc_bh = a.kc + (size_t)bh * a.cap * DH;
  const uint16_t* vc_bh = a.vc + (size_t)bh * a.cap * DH;
  const uint16_t* kb_b = a.kb + ((size_t)b * a.n_blk * a.Hkv + kvh) * DH;
  const uint16_t* vb_b = a.vb + ((size_t)b * a.n_blk * a.Hkv + kvh) * DH;
  const size_t blk_stride = (size_t)a.Hkv * DH;

  // ---- this wave's query tiles, Q fragments kept in registers
  bool tact[QPW];
  int qblk[QPW];
  uint4 qf[QPW][KS];
  float m_run[QPW], l_run[QPW];
  bd_f32x4 oacc[QPW][DH / 16];
#pragma unroll
  for (int j = 0; j < QPW; ++j) {
    const int t = (qg * 4 + wave) * QPW + j;
    tact[j] = t < a.QT;
    const int r = t * 16 + l16;
    const bool rok = tact[j] && r < a.R;
    const int i = rok ? r / a.G : 0;
    const int hg = rok ? r % a.G : 0;
    qblk[j] = rok ? (a.q_off + i) / a.D : INT_MAX;
    const uint16_t* qp = a.q + (((size_t)b * a.n_q + i) * a.Hq + kvh * a.G + hg) * DH;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[j][ks] = rok ? *reinterpret_cast<const uint4*>(qp + 8 * g + 32 * ks) : make_uint4(0, 0, 0, 0);
    m_run[j] = BD_NEG_INF;
    l_run[j] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DH / 16; ++dt) oacc[j][dt] = bd_f32x4{0.f, 0.f, 0.f, 0.f};
  }
  bool any_active = false;
#pragma unroll
  for (int j = 0; j < QPW; ++j) any_active |= tact[j];

  // ---- tile loads (registers) and stores (LDS)
  uint4 kreg[NKL];
  uint4 vreg[4];
  auto key_ptr = [&](const uint16_t* cache_bh, const uint16_t* blk_b, int key) -> const uint16_t* {
    return key < L ? cache_bh + (size_t)key * DH : blk_b + (size_t)(key - L) * blk_stride;
  };
  auto load_tile = [&](int t) {
    const int kbase = kbeg + t * KT;
#pragma unroll
    for (int u = 0; u < NKL; ++u) {
      const int e = tid + kThreads * u;
      const int key = kbase + e / KCH;
      kreg[u] = key < kend ? *reinterpret_cast<const uint4*>(key_ptr(kc_bh, kb_b, key) + (e % KCH) * 8)
                           : make_uint4(0, 0, 0, 0);
    }
    if (tid < NVT) {
      const int kg = tid / KCH, dc = tid % KCH;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int key = kbase + 4 * kg + jj;
        vreg[jj] = key < kend ? *reinterpret_cast<const uint4*>(key_ptr(vc_bh, vb_b, key) + dc * 8)
                              : make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store_tile = [&](int sb) {
#pragma unroll
    for (int u = 0; u < NKL; ++u) {
      const int e = tid + kThreads * u;
      const int kk = e / KCH, ch = e % KCH;
      sK[sb][kk * KCH + (ch ^ (kk & (KCH - 1)))] = kreg[u];
    }
    if (tid < NVT) {
      const int kg = tid / KCH, dc = tid % KCH;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint2 pk;
        pk.x = half16(vreg[0], e) | (half16(vreg[1], e) << 16);
        pk.y = half16(vreg[2], e) | (half16(vreg[3], e) << 16);
        *reinterpret_cast<uint2*>(&sV[sb][(dc * 8 + e) * VP + 4 * kg]) = pk;
      }
    }
  };

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int sb = t & 1;
    if (t + 1 < ntiles) load_tile(t + 1);
    if (any_active) {
      const int kbase = kbeg + t * KT;
      // S^T = K Q^T: lane holds keys 16*kt + 4g + r of query column l16
      bd_f32x4 s[QPW][NKT];
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) {
#pragma unroll
        for (int j = 0; j < QPW; ++j) s[j][kt] = bd_f32x4{0.f, 0.f, 0.f, 0.f};
        const int kk = kt * 16 + l16;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const uint4 kf = sK[sb][kk * KCH + ((g + 4 * ks) ^ (kk & (KCH - 1)))];
#pragma unroll
          for (int j = 0; j < QPW; ++j)
            if (tact[j]) s[j][kt] = bd_mfma16(kf, qf[j][ks], s[j][kt]);
        }
      }
      // online softmax (base 2), probabilities packed as the B operand of P.V
      uint4 pf[QPW][KT / 32];
#pragma unroll
      for (int j = 0; j < QPW; ++j) {
        if (!tact[j]) continue;
        float mx = BD_NEG_INF;
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = kbase + kt * 16 + 4 * g + r;
            const bool vis = key < kend && (key < L || (key - L) / a.D <= qblk[j]);
            const float v = vis ? s[j][kt][r] * a.scale_log2 : BD_NEG_INF;
            s[j][kt][r] = v;
            mx = fmaxf(mx, v);
          }
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mnew = fmaxf(m_run[j], mx);
        const float muse = (mnew == BD_NEG_INF) ? 0.f : mnew;
        const float alpha = bd_exp2(m_run[j] - muse);
        m_run[j] = mnew;
        float ps = 0.f;
#pragma unroll
        for (int u = 0; u < KT / 32; ++u) {
          uint32_t w[4];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const bd_f32x4 sv = s[j][2 * u + h];
            const uint32_t b0 = bd_f2bf(bd_exp2(sv[0] - muse)), b1 = bd_f2bf(bd_exp2(sv[1] - muse));
            const uint32_t b2 = bd_f2bf(bd_exp2(sv[2] - muse)), b3 = bd_f2bf(bd_exp2(sv[3] - muse));
            ps += (bd_bf2f(b0) + bd_bf2f(b1)) + (bd_bf2f(b2) + bd_bf2f(b3));
            w[2 * h] = b0 | (b1 << 16);
            w[2 * h + 1] = b2 | (b3 << 16);
          }
          pf[j][u] = make_uint4(w[0], w[1], w[2], w[3]);
        }
        l_run[j] = l_run[j] * alpha + ps;
#pragma unroll
        for (int dt = 0; dt < DH / 16; ++dt) oacc[j][dt] *= alpha;
      }
      // O^T += V^T P^T: V^T fragment = two 4-key runs of one head-dim row
#pragma unroll
      for (int u = 0; u < KT / 32; ++u) {
#pragma unroll
        for (int dt = 0; dt < DH / 16; ++dt) {
          const uint16_t* vr = &sV[sb][(dt * 16 + l16) * VP + 32 * u + 4 * g];
          const uint2 lo = *reinterpret_cast<const uint2*>(vr);
          const uint2 hi = *reinterpret_cast<const uint2*>(vr + 16);
          const uint4 vf = make_uint4(lo.x, lo.y, hi.x, hi.y);
#pragma unroll
          for (int j = 0; j < QPW; ++j)
            if (tact[j]) oacc[j][dt] = bd_mfma16(vf, pf[j][u], oacc[j][dt]);
        }
      }
    }
    if (t + 1 < ntiles) store_tile(sb ^ 1);
    __syncthreads();
  }

  // ---- epilogue: normalised output (single chunk) or partials
#pragma unroll
  for (int j = 0; j < QPW; ++j) {
    if (!tact[j]) continue;
    float l = l_run[j];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const int r = ((qg * 4 + wave) * QPW + j) * 16 + l16;
    if (r >= a.R) continue;
    const int i = r / a.G, hg = r % a.G;
    if (single) {
      const float inv = l > 0.f ? 1.f / l : 0.f;
      uint16_t* op = a.o + (((size_t)b * a.n_q + i) * a.Hq + kvh * a.G + hg) * DH;
#pragma unroll
      for (int dt = 0; dt < DH / 16; ++dt) {
        const bd_f32x4 v = oacc[j][dt] * inv;
        *reinterpret_cast<uint2*>(op + dt * 16 + 4 * g) =
            make_uint2(bd_pack_bf2(v[0], v[1]), bd_pack_bf2(v[2], v[3]));
      }
      if (a.lse != nullptr && g == 0)
        a.lse[((size_t)b * a.Hq + kvh * a.G + hg) * a.n_q + i] = (m_run[j] + bd_log2(l)) * BD_LN2;
    } else {
      const size_t pi = (size_t)unit * (a.QT * 16) + r;
      float* po = a.part_o + pi * DH;
#pragma unroll
      for (int dt = 0; dt < DH / 16; ++dt)
        *reinterpret_cast<float4*>(po + dt * 16 + 4 * g) =
            make_float4(oacc[j][dt][0], oacc[j][dt][1], oacc[j][dt][2], oacc[j][dt][3]);
      if (g == 0) {
        a.part_ml[2 * pi] = m_run[j];
        a.part_ml[2 * pi + 1] = l;
      }
    }
  }
}

// Merge the key chunks of every (sequence, KV head) whose keys span more than
// one chunk: o = sum_c 2^(m_c - M) O_c / sum_c 2^(m_c - M) l_c.
template <int DH>
__global__ __launch_bounds__(kThreads) void attn_merge_kernel(AttnK a) {
  const size_t idx = (size_t)blockIdx.x * kThreads + threadIdx.x;
  const size_t total = (size_t)a.B * a.Hkv * a.R * (DH / 4);
  if (idx >= total) return;
  const int d4 = idx % (DH / 4);
  const int r = (idx / (DH / 4)) % a.R;
  const int bh = (int)(idx / (DH / 4) / a.R);
  const int b = bh / a.Hkv, kvh = bh % a.Hkv;
  int L = a.kv_len[b];
  L = L < 0 ? 0 : (L > a.cap ? a.cap : L);
  const int T = L + a.n_blk;
  const int nc = (T + a.chunk - 1) / a.chunk;
  if (nc <= 1) return;
  const size_t rp = (size_t)a.QT * 16;
  float M = BD_NEG_INF;
  for (int c = 0; c < nc; ++c) M = fmaxf(M, a.part_ml[2 * (((size_t)bh * a.nchunks + c) * rp + r)]);
  const float muse = (M == BD_NEG_INF) ? 0.f : M;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float lsum = 0.f;
  for (int c = 0; c < nc; ++c) {
    const size_t pi = ((size_t)bh * a.nchunks + c) * rp + r;
    const float w = bd_exp2(a.part_ml[2 * pi] - muse);
    lsum += w * a.part_ml[2 * pi + 1];
    const float4 v = *reinterpret_cast<const float4*>(a.part_o + pi * DH + 4 * d4);
    acc.x += w * v.x;
    acc.y += w * v.y;
    acc.z += w * v.z;
    acc.w += w * v.w;
  }
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  const int i = r / a.G, hg = r % a.G;
  uint16_t* op = a.o + (((size_t)b * a.n_q + i) * a.Hq + kvh * a.G + hg) * DH + 4 * d4;
  *reinterpret_cast<uint2*>(op) = make_uint2(bd_pack_bf2(acc.x * inv, acc.y * inv),
                                             bd_pack_bf2(acc.z * inv, acc.w * inv));
  if (a.lse != nullptr && d4 == 0)
    a.lse[((size_t)b * a.Hq + kvh * a.G + hg) * a.n_q + i] = (M + bd_log2(lsum)) * BD_LN2;
}

// ---- fp32 path -------------------------------------------------------------
struct AttnF {
  const float* q;
  const float* kc;
  const float* vc;
  const int32_t* kv_len;
  const float* kb;
  const float* vb;
  float* o;
  float* lse;
  int Hq, Hkv, G, d, D, n_q, q_off, cap, n_blk;
  float scale;
};

__device__ float block_reduce(float v, bool is_max, float* red) {
  for (int off = 32; off > 0; off >>= 1) {
    const float w = __shfl_xor(v, off);
    v = is_max ? fmaxf(v, w) : v + w;
  }
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
  for (int w = 1; w < kThreads / 64; ++w) r = is_max ? fmaxf(r, red[w]) : r + red[w];
  return r;
}

__global__ __launch_bounds__(kThreads) void attn_f32_kernel(AttnF a) {
  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int kvh = h / a.G;
  int L = a.kv_len[b];
  L = L < 0 ? 0 : (L > a.cap ? a.cap : L);
  const int T = L + a.n_blk;
  const int qblk = (a.q_off + i) / a.D;
  __shared__ float sq[128];
  __shared__ float sp[kThreads];
  __shared__ float red[kThreads / 64];
  if (tid < a.d) sq[tid] = a.q[(((size_t)b * a.n_q + i) * a.Hq + h) * a.d + tid];
  __syncthreads();
  const size_t bh = (size_t)b * a.Hkv + kvh;
  auto kp = [&](const float* cache, const float* blk, int key) -> const float* {
    return key < L ? cache + (bh * a.cap + key) * a.d
                   : blk + (((size_t)b * a.n_blk + (key - L)) * a.Hkv + kvh) * a.d;
  };
  float m = -__builtin_inff(), l = 0.f, acc = 0.f;
  for (int base = 0; base < T; base += kThreads) {
    const int key = base + tid;
    float s = -__builtin_inff();
    if (key < T && (key < L || (key - L) / a.D <= qblk)) {
      const float* k = kp(a.kc, a.kb, key);
      float dot = 0.f;
      for (int e = 0; e < a.d; ++e) dot += sq[e] * k[e];
      s = dot * a.scale;
    }
    const float cm = block_reduce(s, true, red);
    const float mnew = fmaxf(m, cm);
    const float muse = (mnew == -__builtin_inff()) ? 0.f : mnew;
    const float p = (s == -__builtin_inff()) ? 0.f : expf(s - muse);
    sp[tid] = p;
    const float ps = block_reduce(p, false, red);
    const float alpha = (m == -__builtin_inff()) ? 0.f : expf(m - muse);
    l = l * alpha + ps;
    if (tid < a.d) {
      float a2 = 0.f;
      const int n = min(kThreads, T - base);
      for (int kk = 0; kk < n; ++kk)
        if (sp[kk] != 0.f) a2 += sp[kk] * kp(a.vc, a.vb, base + kk)[tid];
      acc = acc * alpha + a2;
    }
    m = mnew;
    __syncthreads();
  }
  if (tid < a.d) a.o[(((size_t)b * a.n_q + i) * a.Hq + h) * a.d + tid] = acc / l;
  if (a.lse != nullptr && tid == 0) a.lse[((size_t)b * a.Hq + h) * a.n_q + i] = m + logf(l);
}

}  // namespace

BdAttnPlan bd_attn_plan(bd_dtype dt, int B, int Hq, int Hkv, int d, int n_q, int cap, int n_blk) {
  BdAttnPlan p{};
  const int G = Hq / Hkv;
  p.R = n_q * G;
  p.QT = (p.R + 15) / 16;
  p.qpw = 1;
  p.nqg = (p.QT + 4 * p.qpw - 1) / (4 * p.qpw);
  const int tmax = cap + n_blk;
  if (dt == BD_F32) {
    p.chunk = tmax;
    p.nchunks = 1;
    return p;
  }
  const long base = (long)B * Hkv * p.nqg;
  int nch = (int)((kTargetWGs + base - 1) / base);
  const int max_ch = (tmax + kMinChunk - 1) / kMinChunk;
  nch = nch < 1 ? 1 : (nch > max_ch ? max_ch : nch);
  int chunk = (tmax + nch - 1) / nch;
  chunk = (chunk + kKT - 1) / kKT * kKT;
  p.chunk = chunk;
  p.nchunks = (tmax + chunk - 1) / chunk;
  if (p.nchunks > 1) {
    const size_t rows = (size_t)B * Hkv * p.nchunks * p.QT * 16;
    p.part_o = 0;
    p.part_ml = rows * d * sizeof(float);
    p.ws_bytes = p.part_ml + rows * 2 * sizeof(float);
  }
  return p;
}

hipError_t bd_attn_launch(bd_dtype dt, const BdAttnPlan& p, const BdAttnArgs& x, hipStream_t s) {
  if (dt == BD_F32) {
    AttnF a{static_cast<const float*>(x.q), static_cast<const float*>(x.k_cache),
            static_cast<const float*>(x.v_cache), x.kv_len, static_cast<const float*>(x.k_blk),
            static_cast<const float*>(x.v_blk), static_cast<float*>(x.o), x.lse,
            x.Hq, x.Hkv, x.G, x.d, x.D, x.n_q, x.q_off, x.cap, x.n_blk, x.scale};
    hipLaunchKernelGGL(attn_f32_kernel, dim3(x.n_q, x.Hq, x.B), dim3(kThreads), 0, s, a);
    return hipGetLastError();
  }
  AttnK a{};
  a.q = static_cast<const uint16_t*>(x.q);
  a.kc = static_cast<const uint16_t*>(x.k_cache);
  a.vc = static_cast<const uint16_t*>(x.v_cache);
  a.kv_len = x.kv_len;
  a.kb = static_cast<const uint16_t*>(x.k_blk);
  a.vb = static_cast<const uint16_t*>(x.v_blk);
  a.o = static_cast<uint16_t*>(x.o);
  a.lse = x.lse;
  a.part_o = x.part_o;
  a.part_ml = x.part_ml;
  a.B = x.B; a.Hq = x.Hq; a.Hkv = x.Hkv; a.G = x.G; a.D = x.D; a.n_q = x.n_q; a.q_off = x.q_off;
  a.cap = x.cap; a.n_blk = x.n_blk;
  a.R = p.R; a.QT = p.QT; a.nqg = p.nqg; a.chunk = p.chunk; a.nchunks = p.nchunks;
  a.n_units = x.B * x.Hkv * p.nchunks;
  a.scale_log2 = x.scale * BD_LOG2E;
  const int n_wg = kXcd * a.nqg * ((a.n_units + kXcd - 1) / kXcd);
  if (x.d == 128)
    hipLaunchKernelGGL((attn_bf16_kernel<128, kKT, 1>), dim3(n_wg), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((attn_bf16_kernel<64, kKT, 1>), dim3(n_wg), dim3(kThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.nchunks == 1) return e;
  const size_t total = (size_t)x.B * x.Hkv * p.R * (x.d / 4);
  const dim3 grid((unsigned)((total + kThreads - 1) / kThreads));
  if (x.d == 128)
    hipLaunchKernelGGL(attn_merge_kernel<128>, grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(attn_merge_kernel<64>, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}
