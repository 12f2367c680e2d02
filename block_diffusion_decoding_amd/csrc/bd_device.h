// Device-side helpers shared by the gfx950 kernels of libbd.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <climits>

#include "../../include/bd.h"

typedef __bf16 bd_bf16x8 __attribute__((ext_vector_type(8)));
typedef float bd_f32x4 __attribute__((ext_vector_type(4)));

#define BD_LOG2E 1.4426950408889634f
#define BD_LN2 0.6931471805599453f
#define BD_NEG_INF (-__builtin_inff())

// bf16 is stored as its 16 raw bits.
__device__ __forceinline__ float bd_bf2f(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// float -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t bd_f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t bd_pack_bf2(float lo, float hi) {
  return bd_f2bf(lo) | (bd_f2bf(hi) << 16);
}

// v_mfma_f32_16x16x32_bf16.  Lane l supplies A row (l % 16) and B column
// (l % 16), eight consecutive K slots 8*(l/16) .. 8*(l/16)+7 each; it receives
// C rows 4*(l/16) .. 4*(l/16)+3 of column (l % 16).  Any fixed permutation of
// the K slots applied to both A and B leaves the product unchanged, which the
// kernels use to pick load-friendly K orders.
__device__ __forceinline__ bd_f32x4 bd_mfma16(const uint4& a, const uint4& b, bd_f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bd_bf16x8, a),
                                                __builtin_bit_cast(bd_bf16x8, b), c, 0, 0, 0);
}

// Hardware base-2 exponential and logarithm (v_exp_f32 / v_log_f32).
__device__ __forceinline__ float bd_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float bd_log2(float x) { return __builtin_amdgcn_logf(x); }

// Row maps (see bd_rows in bd.h).
// The guard of a call (bd_guard): true when no bits[b], b < n, has a bit of
// mask set (the call then does nothing).  The words were written before the
// kernel started and do not change while it runs, so they are read through
// the constant address space: scalar loads, eight at a time, that leave the
// vector-memory counter to the kernel's own loads.
typedef const __attribute__((address_space(4))) uint64_t* bd_const_u64_ptr;
__device__ __forceinline__ bool bd_guard_dead(const uint64_t* bits, uint64_t mask, int n) {
  if (bits == nullptr) return false;
  const bd_const_u64_ptr p = (bd_const_u64_ptr)bits;
  uint64_t any = 0;
  for (int b0 = 0; b0 < n; b0 += 8) {
    uint64_t w[8];  // all eight loads in flight before the first is used
#pragma unroll
    for (int u = 0; u < 8; ++u) w[u] = p[b0 + u < n ? b0 + u : n - 1];
#pragma unroll
    for (int u = 0; u < 8; ++u) any |= w[u];
  }
  return (any & mask) == 0;
}

__device__ __forceinline__ int bd_map_row(const bd_rows& m, int r) {
  return (r / m.group) * m.stride + m.offset + (r % m.group);
}

// (max, argmax, sum of exp(x - max)) triples: the combine is associative and
// commutative up to the rounding of the sum; argmax ties go to the lower index.
struct BdArgStat {
  float m;
  int i;
  float s;
};

__device__ __forceinline__ BdArgStat bd_stat_combine(BdArgStat a, BdArgStat b) {
  BdArgStat r;
  r.m = fmaxf(a.m, b.m);
  r.i = (a.m > b.m) ? a.i : (b.m > a.m) ? b.i : min(a.i, b.i);
  float sa = (a.m == BD_NEG_INF) ? 0.f : a.s * bd_exp2((a.m - r.m) * BD_LOG2E);
  float sb = (b.m == BD_NEG_INF) ? 0.f : b.s * bd_exp2((b.m - r.m) * BD_LOG2E);
  r.s = sa + sb;
  return r;
}

__device__ __forceinline__ BdArgStat bd_stat_shfl_xor(BdArgStat a, int mask) {
  BdArgStat b;
  b.m = __shfl_xor(a.m, mask);
  b.i = __shfl_xor(a.i, mask);
  b.s = __shfl_xor(a.s, mask);
  return b;
}

// Reductions over the 16 lanes of a row group (lanes 16k .. 16k+15) with DPP
// row rotations: after rotating by 8, 4, 2 and 1 every lane holds the result
// (the operations are commutative, and the fixed order makes them
// deterministic).  VALU-speed, no LDS round trip.
template <int CTRL>
__device__ __forceinline__ int bd_dpp_i(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xf, 0xf, false);
}
template <int CTRL>
__device__ __forceinline__ float bd_dpp_f(float x) {
  return __int_as_float(bd_dpp_i<CTRL>(__float_as_int(x)));
}
__device__ __forceinline__ float bd_row16_max(float x) {
  x = fmaxf(x, bd_dpp_f<0x128>(x));  // row_ror:8
  x = fmaxf(x, bd_dpp_f<0x124>(x));  // row_ror:4
  x = fmaxf(x, bd_dpp_f<0x122>(x));  // row_ror:2
  return fmaxf(x, bd_dpp_f<0x121>(x));  // row_ror:1
}
__device__ __forceinline__ float bd_row16_sum(float x) {
  x += bd_dpp_f<0x128>(x);
  x += bd_dpp_f<0x124>(x);
  x += bd_dpp_f<0x122>(x);
  return x + bd_dpp_f<0x121>(x);
}
__device__ __forceinline__ int bd_row16_min(int x) {
  x = min(x, bd_dpp_i<0x128>(x));
  x = min(x, bd_dpp_i<0x124>(x));
  x = min(x, bd_dpp_i<0x122>(x));
  return min(x, bd_dpp_i<0x121>(x));
}

// (max, lowest argmax, sum of exp(v - max)) of the N values v[] held by each
// of the 16 lanes of a row group, at columns col[]; masked values are -inf.
// The row max is found first, so every exponential uses it directly.
template <int N>
__device__ __forceinline__ BdArgStat bd_row16_stat(const float (&v)[N], const int (&col)[N]) {
  float m = v[0];
#pragma unroll
  for (int j = 1; j < N; ++j) m = fmaxf(m, v[j]);
  m = bd_row16_max(m);
  const float mu = (m == BD_NEG_INF) ? 0.f : m;
  float s = 0.f;
  int idx = INT_MAX;
#pragma unroll
  for (int j = 0; j < N; ++j) {
    s += bd_exp2((v[j] - mu) * BD_LOG2E);
    if (v[j] == m && v[j] != BD_NEG_INF) idx = min(idx, col[j]);
  }
  return BdArgStat{m, bd_row16_min(idx), bd_row16_sum(s)};
}


// Confidence-threshold unmasking of one sequence's window by one wavefront
// ("Fast-dLLM v2: Efficient Block-Diffusion LLM" notes, Key design 3; the v1
// article, Core technique 2).  Lane r holds window entry r: its confidence c
// and argmax am (ignored past win_len).  Candidates are the masked window
// positions; every candidate with c > thr is unmasked, and when candidates
// exist but none passes, the most confident one (lowest position on ties).
// A NaN confidence never passes and ranks last.  Writes the picked tokens,
// the new mask bits (also to bits_out when given: a second copy, e.g. in
// host memory the device can write), the count and the ascending positions.
// Returns the window entries it unmasked (bit r: entry r; the same in every lane).
__device__ inline uint64_t bd_unmask_wave(int r, int b, int D, int win_lo, int win_len, uint64_t bits, float c, int32_t am,
                                      float thr, int32_t* tokens, uint64_t* mask_bits, int32_t* n_unmasked,
                                      int32_t* unmasked_pos, uint64_t* bits_out) {
  const int pos = win_lo + r;
  const bool cand = r < win_len && ((bits >> pos) & 1ull);
  c = cand ? c : BD_NEG_INF;
  if (c != c) c = BD_NEG_INF;
  uint64_t pick = __ballot(cand && c > thr);
  const uint64_t cands = __ballot(cand);
  if (pick == 0 && cands != 0) {
    float best = c;
    for (int off = 32; off > 0; off >>= 1) best = fmaxf(best, __shfl_xor(best, off));
    const uint64_t eq = __ballot(cand && c == best);
    pick = eq & (~eq + 1ull);  // lowest position among the most confident
  }
  const bool mine = (pick >> r) & 1ull;
  if (mine) tokens[(size_t)b * D + pos] = am;
  const int n = __popcll(pick);
  if (unmasked_pos != nullptr && r < win_len) {
    const int rank = __popcll(pick & ((1ull << r) - 1ull));
    if (mine) unmasked_pos[(size_t)b * win_len + rank] = pos;
    if (r >= n) unmasked_pos[(size_t)b * win_len + r] = -1;
  }
  if (r == 0) {
    const uint64_t left = bits & ~(pick << win_lo);
    mask_bits[b] = left;
    if (bits_out != nullptr) bits_out[b] = left;
    if (n_unmasked != nullptr) n_unmasked[b] = n;
  }
  return pick;
}
