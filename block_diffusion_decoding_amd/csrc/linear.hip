// Support kernels of the refinement step: input rows and projections.
//
// Input rows: "Fast-dLLM v2: Efficient Block-Diffusion LLM" notes, Key design 2
// -- a masked position takes the learnable [MASK] embedding.  Projections:
// the Q/K/V projections of the block rows (fresh rows write their K/V into
// the in-block buffer, Key design 3) and the attention output projection
// with its residual; for the multi-layer decoder also the gate/up projection
// with the SwiGLU gate and the Q/K projections with the rotary embedding.
//
// bf16 projections: a persistent streaming GEMM on the MFMA core of
// stream_gemm.h.  The 16-column tiles of all output segments (Q, K, V share
// one launch) are dealt out to work-groups in balanced contiguous ranges; a
// work-group walks its range in passes of up to NTW tiles while the
// global->LDS DMA pipeline runs on across pass boundaries, so every weight
// byte is read once from HBM with no per-tile pipeline fill and no tail of
// short work-groups.  When the tiles alone cannot occupy the GPU, K is split
// over slices that write fp32 partial sums, added by a second launch that
// also applies the residual or the rotary embedding.
#include <cmath>

#include "bd_device.h"
#include "bd_launch.h"
#include "stream_gemm.h"

namespace {

constexpr int kThreads = 256;
// Tiling and scheduling; defaults chosen by measurement, overridable at build
// time.
#ifndef BD_GEMM_NS
#define BD_GEMM_NS 3
#endif
#ifndef BD_GEMM_MAX_MT
#define BD_GEMM_MAX_MT 4
#endif
constexpr int kCUs = 256;
constexpr int kLdsPerCU = 160 * 1024;
#ifndef BD_GEMM_MIN_CHUNKS
#define BD_GEMM_MIN_CHUNKS 4
#endif
// Schedule cost model (ns, bytes per ns): a work-group's pipeline stage takes
// at least LAT_NS / (NS - 1) (NS - 1 stages in flight against the memory
// latency), or longer when the resident work-groups' stage bytes exceed what
// HBM (weight tiles) and L2 (row tiles, empty weight slots) deliver; a K
// split adds a reduction launch and its partial-sum traffic.
#ifndef BD_GEMM_LAT_NS
#define BD_GEMM_LAT_NS 1400
#endif
#ifndef BD_GEMM_HBM_BPNS
#define BD_GEMM_HBM_BPNS 5000
#endif
#ifndef BD_GEMM_L2_BPNS
#define BD_GEMM_L2_BPNS 15000
#endif
#ifndef BD_GEMM_RED_NS
#define BD_GEMM_RED_NS 2500
#endif
// 0: never split K over the waves of a work-group; 1: for projections whose
// streaming plan needs a K-split reduction; 2: wherever it fits
#ifndef BD_GEMM_KWAVE
#define BD_GEMM_KWAVE 1
#endif
// cost of a 256 x 256 tile of the large-M kernel relative to a 256 x 128 one, x10
#ifndef BD_GEMM_BIG16_COST
#define BD_GEMM_BIG16_COST 16
#endif
#ifndef BD_GEMM_PART_BPNS
#define BD_GEMM_PART_BPNS 4000
#endif
constexpr int kNS = BD_GEMM_NS;  // pipeline stages
constexpr int kXcdGemm = 8;      // work-groups are dispatched round-robin over 8 XCDs
constexpr int kSliceBatch = 8;   // K slices whose partial sums a reduction thread loads at once
constexpr int kMaxSeg = 3;

struct GemmS {
  const uint16_t* x;
  bd_rows xr;
  int M, K, nseg, mode;
  const uint16_t* w[kMaxSeg];
  uint16_t* y[kMaxSeg];
  const uint16_t* res[kMaxSeg];
  bd_rows yr[kMaxSeg];
  bd_rows rr[kMaxSeg];
  int N[kMaxSeg];       // output columns per segment (SwiGLU: the gate width)
  int tb[kMaxSeg + 1];  // first 16-column tile of each segment; T from nseg on
  int ksplit;
  int vec_out;          // every output width % 4 == 0, y/res 8-byte aligned: vector stores
  float* part;          // [ksplit][M][T*16] fp32 partial sums (ksplit > 1)
  const int32_t* pos_base;  // rotary embedding (BD_GEMM_ROPE)
  int n_rows, pos_off, d;
  double log2_theta;
  const uint64_t* g_bits;   // guard (bd_guard): the launch does nothing when no
  uint64_t g_mask;          // g_bits[b], b < g_n, has a bit of g_mask set
  int g_n;
  int norm_x;               // SwiGLU mode: the rows of x are RMS-normalised first
  float norm_eps;
};

// Input RMSNorm (unit gains) folded into a SwiGLU projection: the product of
// a normalised row is the product of the raw row times rsqrt(mean x^2 + eps),
// so the kernels multiply raw x (bf16 from memory) and scale the gate and up
// sums of each row.  The sum of squares comes from the A fragments the MFMAs
// read anyway: lane L holds 8 values of row L % 16 per k-step, and the four
// lanes L % 16 == c together cover every k once.
typedef __bf16 bd_bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float bf16x8_sumsq(uint4 v, float s) {  // s + sum of the 8 squares (4 dot2 steps)
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const bd_bf16x2 p = __builtin_bit_cast(bd_bf16x2, w[h]);
    s = __builtin_amdgcn_fdot2_f32_bf16(p, p, s, false);
  }
  return s;
}
// Row total of a fragment tile's squares: lanes L with L % 16 == c end up
// with the sum of row c (every lane of the wave calls it).
__device__ __forceinline__ float frag_row_total(float ss) {
  const float t = ss + __shfl_xor(ss, 16);
  return t + __shfl_xor(t, 32);
}

__device__ __forceinline__ int seg_of(const GemmS& a, int gt) {
  return gt >= a.tb[2] ? 2 : (gt >= a.tb[1] ? 1 : 0);
}

// Rotated segments in the K-split-over-waves kernel: tile tt of a q or k
// segment is a "pair tile" whose rows 0..7 are the output columns
// h*d + 8t .. +7 of head h = tt / (d/16), t = tt % (d/16), and whose rows
// 8..15 are their rotation partners h*d + d/2 + 8t .. +7.  The rotate-half
// pairs (j, j + d/2) then sit in lanes c and c ^ 8 of the same 16-lane group
// of an MFMA result, so the rotation needs no other work-group's columns.
// Needs d % 16 == 0.
__device__ __forceinline__ int pair_tile_col(int tt, int r, int d) {
  const int th = d >> 4, h = tt / th, t = tt - h * th;
  return h * d + (r < 8 ? 8 * t + r : (d >> 1) + 8 * t + r - 8);
}
__device__ __forceinline__ bool rotated_seg(const GemmS& a, int sg) {
  return a.mode == BD_GEMM_ROPE && sg < 2 && (a.d & 15) == 0;
}

// Work-group (blockIdx.x, row block blockIdx.y, K slice blockIdx.z) owns
// scheduling units [g0, g0 + ng) of the T/G units (G = 1: a 16-column tile;
// G = 2 in SwiGLU mode: a gate tile and the matching up tile, adjacent in the
// tile order so that one wave holds both) and walks them in P passes.
// Epilogue per pass: bf16 store (+ residual), SwiGLU, or fp32 partial sums.
template <int MT, int NTW>
__global__ __launch_bounds__(kThreads, 2) void gemm_stream_kernel(GemmS a, int P, int G) {
  using C = bd_stream::Cfg<MT, NTW, kNS>;
  static_assert(C::NTP % 2 == 0, "a wave holds whole gate/up tile pairs");
  __shared__ uint4 sbuf[C::NS * C::STAGE_U4];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, l16 = lane & 15;
  const int wm = wave % C::WM, wn = wave / C::WM;
  const int m0 = blockIdx.y * MT * 16;
  const int z = blockIdx.z;
  const int K = a.K, nchK = K / C::KC;
  const int c0 = (int)((long long)z * nchK / a.ksplit);
  const int nch = (int)((long long)(z + 1) * nchK / a.ksplit) - c0;
  const int T = a.tb[a.nseg];
  const int Tg = T / G;
  const int g0 = (int)((long long)blockIdx.x * Tg / gridDim.x);
  const int ng = (int)((long long)(blockIdx.x + 1) * Tg / gridDim.x) - g0;
  auto pass_begin = [&](int p) { return G * (g0 + p * ng / P); };  // first tile of pass p
  const int nst = P * nch;
  const size_t koff = (size_t)c0 * C::KC;

  // DMA instruction f = wave + 4i loads rows 8*(f%2)..+7 of stage tile f/2:
  // tiles 0..NTW-1 are W (per pass), the next MT are X (fixed).  Slots past
  // the data read a valid row whose products are discarded.
  const int lrow = lane >> 3, lkb = (lane & 7) ^ lrow;
  const uint16_t* const dummy = a.x + (size_t)bd_map_row(a.xr, 0) * K + koff + 8 * lkb;
  const uint16_t* src[C::LW];
#pragma unroll
  for (int i = 0; i < C::LW; ++i) {
    const int f = wave + 4 * i, t = f >> 1;
    const int m = m0 + (t - NTW) * 16 + 8 * (f & 1) + lrow;
    src[i] = (f < C::FR && t >= NTW && m < a.M) ? a.x + (size_t)bd_map_row(a.xr, m) * K + koff + 8 * lkb : dummy;
  }
  auto set_pass = [&](int p) {  // W sources of pass p
    const int b = pass_begin(p), n = pass_begin(p + 1) - b;
#pragma unroll
    for (int i = 0; i < C::LW; ++i) {
      const int f = wave + 4 * i, t = f >> 1;
      if (f < C::FR && t < NTW) {
        const int r = 8 * (f & 1) + lrow;
        const uint16_t* row = dummy;
        if (t < n) {
          const int gt = b + t;
          if (a.mode == BD_GEMM_SWIGLU) {
            int c = (gt >> 1) * 16 + r;
            c = c < a.N[0] ? c : a.N[0] - 1;
            row = a.w[0] + (size_t)((gt & 1) ? a.N[0] + c : c) * K + koff + 8 * lkb;
          } else {
            const int sg = seg_of(a, gt);
            int c = (gt - a.tb[sg]) * 16 + r;
            c = c < a.N[sg] ? c : a.N[sg] - 1;
            row = a.w[sg] + (size_t)c * K + koff + 8 * lkb;
          }
        }
        src[i] = row;
      }
    }
  };
  int ip = 0, ich = 0, iss = 0;  // issue cursor: pass, chunk, stages issued
  set_pass(0);
  auto issue_next = [&]() {
    uint4* st = sbuf + (iss % C::NS) * C::STAGE_U4;
#pragma unroll
    for (int i = 0; i < C::LW; ++i)
      if (C::FR % 4 == 0 || wave + 4 * i < C::FR)
        __builtin_amdgcn_global_load_lds((bd_stream::glb_void_t*)(src[i] + (size_t)ich * C::KC),
                                         (bd_stream::lds_void_t*)(st + (wave + 4 * i) * 64), 16, 0, 0);
    ++iss;
    if (++ich == nch) {
      ich = 0;
      if (++ip < P) set_pass(ip);
    }
  };
  const bool more = wave < C::FR % 4;  // this wave issues LW (else LW_LO) loads per stage
  const int fo0 = bd_stream::frag_offset(lane, 0) / 16, fo1 = bd_stream::frag_offset(lane, 1) / 16;

  bd_f32x4 acc[C::MTW][C::NTP];
#pragma unroll
  for (int i = 0; i < C::MTW; ++i)
#pragma unroll
    for (int j = 0; j < C::NTP; ++j) acc[i][j] = bd_f32x4{0.f, 0.f, 0.f, 0.f};
  // input RMSNorm: the sums of squares of the rows, from the first pass's
  // fragments; row tile i of a row group is summed by the wave wn == i % WN
  // of the group, the scales meet in LDS at the end of the first pass
  __shared__ float nscale[MT * 16];
  float ss[C::MTW], scl[C::MTW][4];
#pragma unroll
  for (int i = 0; i < C::MTW; ++i) {
    ss[i] = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) scl[i][r] = 1.f;
  }

#pragma unroll
  for (int c = 0; c < C::NS - 1; ++c)
    if (c < nst) issue_next();
  // the guard's words load while the first stages are in flight
  if (bd_guard_dead(a.g_bits, a.g_mask, a.g_n)) {
    __builtin_amdgcn_s_waitcnt(bd_stream::vmcnt_imm(0));  // no DMA into this LDS after the work-group ends
    return;
  }

  int cp = 0, cch = 0;  // compute cursor: pass, chunk
  for (int s = 0; s < nst; ++s) {
    const int later = min(nst - s - 1, C::NS - 2);
    if (later == 0) __builtin_amdgcn_s_waitcnt(bd_stream::vmcnt_imm(0));
    else if (later == 1) {
      if (more) __builtin_amdgcn_s_waitcnt(bd_stream::vmcnt_imm(C::LW));
      else __builtin_amdgcn_s_waitcnt(bd_stream::vmcnt_imm(C::LW_LO));
    } else if (later == 2) {
      if (more) __builtin_amdgcn_s_waitcnt(bd_stream::vmcnt_imm(2 * C::LW));
      else __builtin_amdgcn_s_waitcnt(bd_stream::vmcnt_imm(2 * C::LW_LO));
    } else {
      if (more) __builtin_amdgcn_s_waitcnt(bd_stream::vmcnt_imm(3 * C::LW));
      else __builtin_amdgcn_s_waitcnt(bd_stream::vmcnt_imm(3 * C::LW_LO));
    }
    bd_stream::pipe_barrier();  // stage s is in LDS for every wave; the slot of s - 1 is free
    if (s + C::NS - 1 < nst) issue_next();
    // fragment reads as asm that waits inside the block (a plain LDS read
    // would get a wait for every DMA in flight in front of it)
    const uint32_t sb = bd_stream::lds_addr(sbuf + (s % C::NS) * C::STAGE_U4);
#pragma unroll
    for (int ks = 0; ks < C::KSC; ++ks) {
      const uint32_t fo = (ks == 0 ? fo0 : fo1) * 16;
      uint4 xa[C::MTW], wb[C::NTP];
      bd_stream::lds_frags_kstep<C::MTW, C::NTP>(sb + (NTW + wm * C::MTW) * 2048 + fo,
                                                 sb + wn * C::NTP * 2048 + fo, xa, wb);
#pragma unroll
      for (int i = 0; i < C::MTW; ++i)
#pragma unroll
        for (int j = 0; j < C::NTP; ++j) acc[i][j] = bd_mfma16(xa[i], wb[j], acc[i][j]);
      if (a.norm_x && cp == 0)
#pragma unroll
        for (int i = 0; i < C::MTW; ++i)
          if (i % C::WN == wn) ss[i] = bf16x8_sumsq(xa[i], ss[i]);
    }
    if (++cch < nch) continue;

    // ---- end of pass cp: rows m0 + (wm*MTW + i)*16 + 4g + r, tile slots
    // wn*NTP + j of the pass, column l16 of each
    const int b = pass_begin(cp), n = pass_begin(cp + 1) - b;
    if (a.mode == BD_GEMM_SWIGLU) {
      if (a.norm_x && cp == 0) {
        const uint32_t ns = bd_stream::lds_addr(nscale);
#pragma unroll
        for (int i = 0; i < C::MTW; ++i)
          if (i % C::WN == wn) {
            const float t = frag_row_total(ss[i]);
            if (g == 0) bd_stream::lds_write_f32(ns + ((wm * C::MTW + i) * 16 + l16) * 4, rsqrtf(t / (float)K + a.norm_eps));
          }
        bd_stream::pipe_barrier();
#pragma unroll
        for (int i = 0; i < C::MTW; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) scl[i][r] = bd_stream::lds_read_f32(ns + ((wm * C::MTW + i) * 16 + 4 * g + r) * 4);
      }
#pragma unroll
      for (int j = 0; j < C::NTP; j += 2) {
        const int slot = wn * C::NTP + j;
        const int col = ((b + slot) >> 1) * 16 + l16;
        if (slot < n && col < a.N[0]) {
#pragma unroll
          for (int i = 0; i < C::MTW; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int m = m0 + (wm * C::MTW + i) * 16 + 4 * g + r;
              if (m < a.M) {
                const float zg = acc[i][j][r] * scl[i][r], u = acc[i][j + 1][r] * scl[i][r];
                a.y[0][(size_t)bd_map_row(a.yr[0], m) * a.N[0] + col] =
                    (uint16_t)bd_f2bf(zg / (1.f + __expf(-zg)) * u);
              }
            }
        }
      }
    } else if (a.ksplit > 1) {
      const size_t Nt = (size_t)T * 16;
#pragma unroll
      for (int j = 0; j < C::NTP; ++j) {
        const int slot = wn * C::NTP + j;
        if (slot < n) {
          float* pz = a.part + (size_t)z * a.M * Nt + (size_t)(b + slot) * 16 + l16;
#pragma unroll
          for (int i = 0; i < C::MTW; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int m = m0 + (wm * C::MTW + i) * 16 + 4 * g + r;
              if (m < a.M) pz[(size_t)m * Nt] = acc[i][j][r];
            }
        }
      }
    } else {
      int sgj[C::NTP], colj[C::NTP];
      bool okj[C::NTP];
#pragma unroll
      for (int j = 0; j < C::NTP; ++j) {
        const int slot = wn * C::NTP + j;
        const int gt = b + slot;
        sgj[j] = seg_of(a, gt);
        colj[j] = (gt - a.tb[sgj[j]]) * 16 + l16;
        okj[j] = slot < n && colj[j] < a.N[sgj[j]];
      }
      // residual values first, all loads in flight together, then the stores
      // (y may be res: a lane reads exactly the elements it writes)
      float rv[C::MTW][C::NTP][4];
#pragma unroll
      for (int i = 0; i < C::MTW; ++i)
#pragma unroll
        for (int j = 0; j < C::NTP; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int m = m0 + (wm * C::MTW + i) * 16 + 4 * g + r;
            const uint16_t* res = a.res[sgj[j]];
            rv[i][j][r] = (okj[j] && m < a.M && res)
                              ? bd_bf2f(res[(size_t)bd_map_row(a.rr[sgj[j]], m) * a.N[sgj[j]] + colj[j]])
                              : 0.f;
          }
#pragma unroll
      for (int i = 0; i < C::MTW; ++i)
#pragma unroll
        for (int j = 0; j < C::NTP; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int m = m0 + (wm * C::MTW + i) * 16 + 4 * g + r;
            if (okj[j] && m < a.M)
              a.y[sgj[j]][(size_t)bd_map_row(a.yr[sgj[j]], m) * a.N[sgj[j]] + colj[j]] =
                  (uint16_t)bd_f2bf(acc[i][j][r] + rv[i][j][r]);
          }
    }
#pragma unroll
    for (int i = 0; i < C::MTW; ++i)
#pragma unroll
      for (int j = 0; j < C::NTP; ++j) acc[i][j] = bd_f32x4{0.f, 0.f, 0.f, 0.f};
    cch = 0;
    ++cp;
  }
}

// Projections with few 16-column tiles (the fresh rows of a refinement step
// against a 3584-wide weight, say): split over work-groups by K, they would
// need a reduction launch after the GEMM.  Here the K range is split over the
// four waves of a work-group instead.  Work-group (tile group, row block)
// owns NT consecutive tiles (in SwiGLU mode NT = 2: a gate and its up tile)
// and 16*MT rows; wave w walks the 64-wide K chunks [w*nch/4, (w+1)*nch/4)
// through a ring of NS stages of its own (stage: the NT W tiles, then the MT
// X tiles, 2 KiB each, loaded by global->LDS DMA in whole 128-byte lines,
// XOR-swizzled, as in stream_gemm.h), with no work-group barrier in the loop.
// (W fragments loaded straight into registers, 16 rows x 64 bytes per
// instruction, measured slower from HBM than these whole-line DMA tiles.)
// The waves' accumulators then meet in LDS and are added in wave order, so
// results do not depend on timing.  Grid: 8 x ceil(groups / 8) x ny
// work-groups, the row blocks of one tile group consecutive on one XCD (they
// read the same W tiles, the second time from L2).  One work-group per CU
// (the rings take up to 144 KiB of LDS).
template <int MT, int NT, int NS>
__global__ __launch_bounds__(kThreads, 1) void gemm_kwave_kernel(GemmS a, int ny) {
  constexpr int FRW = 2 * (NT + MT);  // DMA instructions per stage (one wave's)
  constexpr int STAGE_U4 = FRW * 64;
  static_assert(NS >= 2 && (NS - 2) * FRW < 64 && NS <= 8, "stages");
  static_assert(4 * MT * NT * 64 <= 4 * NS * STAGE_U4, "reduction area");
  __shared__ uint4 sbuf[4 * NS * STAGE_U4];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, l16 = lane & 15;
  const int xcd = blockIdx.x % kXcdGemm, t8 = blockIdx.x / kXcdGemm;
  const int rb = t8 % ny;
  const int tg = (t8 / ny) * kXcdGemm + xcd;
  const int T = a.tb[a.nseg];
  const int t0 = tg * NT;
  if (t0 >= T) return;
  const int n = T - t0 < NT ? T - t0 : NT;  // real tiles of this group
  const int m0 = rb * MT * 16;
  const int K = a.K, nchK = K / 64;
  const int cb = wave * nchK / 4, nch = (wave + 1) * nchK / 4 - cb;
  const bool swiglu = a.mode == BD_GEMM_SWIGLU;

  // instruction f loads rows 8*(f%2)..+7 of stage tile f/2 (W tiles first);
  // past the data: a valid X row whose products are discarded
  const int lrow = lane >> 3, lkb = (lane & 7) ^ lrow;
  const size_t koff = (size_t)cb * 64 + 8 * lkb;
  const uint16_t* const dummy = a.x + (size_t)bd_map_row(a.xr, 0) * K + koff;
  const uint16_t* src[FRW];
#pragma unroll
  for (int f = 0; f < FRW; ++f) {
    const int t = f >> 1, r = 8 * (f & 1) + lrow;
    const uint16_t* row = dummy;
    if (t < NT) {
      if (t < n) {
        const int gt = t0 + t;
        if (swiglu) {
          int c = (gt >> 1) * 16 + r;
          c = c < a.N[0] ? c : a.N[0] - 1;
          row = a.w[0] + (size_t)((gt & 1) ? a.N[0] + c : c) * K + koff;
        } else {
          const int sg = seg_of(a, gt);
          int c = rotated_seg(a, sg) ? pair_tile_col(gt - a.tb[sg], r, a.d) : (gt - a.tb[sg]) * 16 + r;
          c = c < a.N[sg] ? c : a.N[sg] - 1;
          row = a.w[sg] + (size_t)c * K + koff;
        }
      }
    } else {
      const int m = m0 + (t - NT) * 16 + r;
      if (m < a.M) row = a.x + (size_t)bd_map_row(a.xr, m) * K + koff;
    }
    src[f] = row;
  }
  uint4* const ring = sbuf + wave * NS * STAGE_U4;
  auto issue = [&](int c) {
    uint4* st = ring + (c % NS) * STAGE_U4;
#pragma unroll
    for (int f = 0; f < FRW; ++f)
      __builtin_amdgcn_global_load_lds((bd_stream::glb_void_t*)(src[f] + (size_t)c * 64),
                                       (bd_stream::lds_void_t*)(st + f * 64), 16, 0, 0);
  };
  const int fo0 = bd_stream::frag_offset(lane, 0), fo1 = bd_stream::frag_offset(lane, 1);

  bd_f32x4 acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = bd_f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int c = 0; c < NS - 1; ++c)
    if (c < nch) issue(c);
  // the guard's words load while the first stages are in flight
  if (bd_guard_dead(a.g_bits, a.g_mask, a.g_n)) {
    __builtin_amdgcn_s_waitcnt(bd_stream::vmcnt_imm(0));  // no DMA into this LDS after the work-group ends
    return;
  }
  for (int s = 0; s < nch; ++s) {
    // stage s complete: at most `later` younger stages still in flight
    const int later = min(nch - s - 1, NS - 2);
    if (later <= 0) __builtin_amdgcn_s_waitcnt(bd_stream::vmcnt_imm(0));
    else if (later == 1) __builtin_amdgcn_s_waitcnt(bd_stream::vmcnt_imm(FRW));
    else if (later == 2) __builtin_amdgcn_s_waitcnt(bd_stream::vmcnt_imm(NS > 3 ? 2 * FRW : 0));
    else if (later == 3) __builtin_amdgcn_s_waitcnt(bd_stream::vmcnt_imm(NS > 4 ? 3 * FRW : 0));
    else if (later == 4) __builtin_amdgcn_s_waitcnt(bd_stream::vmcnt_imm(NS > 5 ? 4 * FRW : 0));
    else if (later == 5) __builtin_amdgcn_s_waitcnt(bd_stream::vmcnt_imm(NS > 6 ? 5 * FRW : 0));
    else __builtin_amdgcn_s_waitcnt(bd_stream::vmcnt_imm(NS > 7 ? 6 * FRW : 0));
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (s + NS - 1 < nch) issue(s + NS - 1);  // into the slot read at s - 1 (its reads have completed)
    const uint32_t sb = bd_stream::lds_addr(ring + (s % NS) * STAGE_U4);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const uint32_t fo = ks == 0 ? fo0 : fo1;
      uint4 xa[MT], wb[NT];
      bd_stream::lds_frags_kstep<MT, NT>(sb + NT * 2048 + fo, sb + fo, xa, wb);
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[i][j] = bd_mfma16(xa[i], wb[j], acc[i][j]);
    }
  }

  // ---- the waves' sums meet in LDS: red[w][i*NT + j][lane]
  __syncthreads();
  bd_f32x4* red = reinterpret_cast<bd_f32x4*>(sbuf);
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) red[(wave * MT * NT + i * NT + j) * 64 + lane] = acc[i][j];
  __syncthreads();
  auto total = [&](int p) {  // tile pair p summed over the waves, in wave order
    bd_f32x4 v = red[p * 64 + lane];
#pragma unroll
    for (int w = 1; w < 4; ++w) v += red[(w * MT * NT + p) * 64 + lane];
    return v;
  };
  if (swiglu) {
    // wave w: row tiles i = w, w + 4, ... of the (gate, up) pair
    for (int i = wave; i < MT; i += 4) {
      const int col = (t0 >> 1) * 16 + l16;
      if (n < 2 || col >= a.N[0]) continue;
      const bd_f32x4 zg = total(i * NT), u = total(i * NT + 1);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + i * 16 + 4 * g + r;
        if (m < a.M)
          a.y[0][(size_t)bd_map_row(a.yr[0], m) * a.N[0] + col] =
              (uint16_t)bd_f2bf(zg[r] / (1.f + __expf(-zg[r])) * u[r]);
      }
    }
    return;
  }
  for (int p = wave; p < MT * NT; p += 4) {
    const int i = p / NT, j = p % NT;
    if (j >= n) continue;
    const int gt = t0 + j, sg = seg_of(a, gt);
    if (rotated_seg(a, sg)) {
      // pair tile: lane c < 8 holds x1 = column j of the head's first half,
      // lane c ^ 8 its partner x2 = column j + d/2; angle pos * theta^(-2j/d)
      // in fp64, the rotation in fp32 (as the K-split reduction does)
      const bd_f32x4 v = total(p);
      const int tt = gt - a.tb[sg], th = a.d >> 4, hd = tt / th, jf = 8 * (tt - hd * th) + (l16 & 7);
      const bool first = l16 < 8;
      const int col = hd * a.d + (first ? jf : (a.d >> 1) + jf);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float other = __shfl_xor(v[r], 8);
        const int m = m0 + i * 16 + 4 * g + r;
        if (m >= a.M) continue;
        const double pos = (double)(a.pos_base[m / a.n_rows] + a.pos_off + m % a.n_rows);
        const double ang = pos * exp2(-(2.0 * jf / a.d) * a.log2_theta);
        double sn, cs;
        sincos(ang, &sn, &cs);
        const float c = (float)cs, sv = (float)sn;
        const float x1 = first ? v[r] : other, x2 = first ? other : v[r];
        const float y = first ? x1 * c - x2 * sv : x2 * c + x1 * sv;
        a.y[sg][(size_t)bd_map_row(a.yr[sg], m) * a.N[sg] + col] = (uint16_t)bd_f2bf(y);
      }
      continue;
    }
    const int col = (gt - a.tb[sg]) * 16 + l16;
    if (col >= a.N[sg]) continue;
    const bd_f32x4 v = total(p);
    const uint16_t* res = a.res[sg];
    float rv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + i * 16 + 4 * g + r;
      rv[r] = (m < a.M && res) ? bd_bf2f(res[(size_t)bd_map_row(a.rr[sg], m) * a.N[sg] + col]) : 0.f;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + i * 16 + 4 * g + r;
      if (m < a.M) a.y[sg][(size_t)bd_map_row(a.yr[sg], m) * a.N[sg] + col] = (uint16_t)bd_f2bf(v[r] + rv[r]);
    }
  }
}

// Large-M projections (prompt prefill, exact steps of big batches, the
// training form): 256-row x (CT*16)-column tiles with 8 waves, the tile
// machinery of the batched LM head.  CT = 16: 2 x 4 waves of 128 x 64, two
// 64 KiB stages; CT = 8: 4 x 2 waves of 64 x 64, three 48 KiB stages.  The
// CT column tiles of a block are consecutive tiles of the segment order (in
// SwiGLU mode gate and up tiles alternate, so a wave holds whole pairs).  No
// K split (there are enough tiles); rows past M are neither loaded nor
// multiplied.  Work order: the larger operand is fetched from HBM once per
// block and the smaller one re-read from L2: with more weight columns than
// rows, the row blocks of a column block are consecutive on one XCD; with
// more rows (row_major), the column blocks of a row block are.
constexpr int kBigRows = 256, kBigThreads = 512;
template <int CT>
struct GBig {
  static constexpr int WR = CT == 16 ? 2 : 4;       // waves along the rows
  static constexpr int WC = 8 / WR;                 // waves along the columns
  static constexpr int MW = kBigRows / 16 / WR;     // row tiles per wave
  static constexpr int NWT = CT / WC;               // column tiles per wave
  static constexpr int NS = CT == 16 ? 2 : 3;       // stages
  static constexpr int TILES = kBigRows / 16 + CT;  // 16-row tiles per stage
  static constexpr int FR = 2 * TILES;              // DMA instructions per stage
  static constexpr int LW = FR / 8;                 // per wave
  static constexpr int STAGE_U4 = FR * 64;
  static_assert(MW % 4 == 0 && NWT == 4 && FR % 8 == 0 && LW <= 8, "wave tiling");
};

template <int CT>
__global__ __launch_bounds__(kBigThreads, 1) void gemm_big_kernel(GemmS a, int rb_count, int cb_count,
                                                                   int row_major) {
  using P = GBig<CT>;
  __shared__ uint4 sbuf[P::NS * P::STAGE_U4];
  if (bd_guard_dead(a.g_bits, a.g_mask, a.g_n)) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, l16 = lane & 15;
  const int wr = wave % P::WR, wc = wave / P::WR;
  // work-group w runs on XCD w % 8; its (w / 8)-th work-group takes the next
  // inner block of that XCD's outer blocks
  const int xcd = blockIdx.x & 7, q = blockIdx.x >> 3;
  int rb, cb;
  if (row_major) {
    const int per_xcd = (rb_count + 7) >> 3;
    cb = q % cb_count;
    rb = xcd * per_xcd + q / cb_count;
    if (rb >= rb_count) return;
  } else {
    const int per_xcd = (cb_count + 7) >> 3;
    rb = q % rb_count;
    cb = xcd * per_xcd + q / rb_count;
    if (cb >= cb_count) return;
  }
  const int m0 = rb * kBigRows;
  const int K = a.K, nch = K / 64;
  const int T = a.tb[a.nseg];
  const bool swiglu = a.mode == BD_GEMM_SWIGLU;

  // DMA sources: instruction f covers rows 8*(f%2)..+7 of stage tile f/2;
  // tiles 0..15 are X row tiles, the next CT are W column tiles.
  const int lrow = lane >> 3, lkb = (lane & 7) ^ lrow;
  const uint16_t* src[P::LW];
  const int live_tiles = min(kBigRows / 16, (a.M - m0 + 15) / 16);
  bool ld[P::LW];
  int issued = 0;
#pragma unroll
  for (int i = 0; i < P::LW; ++i) {
    const int f = wave + 8 * i, t = f >> 1, r = 8 * (f & 1) + lrow;
    if (t < kBigRows / 16) {
      const int m = m0 + t * 16 + r;
      src[i] = a.x + (size_t)bd_map_row(a.xr, m < a.M ? m : a.M - 1) * K + 8 * lkb;
      ld[i] = t < live_tiles;
    } else {
      int gt = cb * CT + (t - kBigRows / 16);
      gt = gt < T ? gt : T - 1;  // past the last tile: a valid row, products unused
      size_t wrow;
      const uint16_t* w;
      if (swiglu) {
        int c = (gt >> 1) * 16 + r;
        c = c < a.N[0] ? c : a.N[0] - 1;
        w = a.w[0];
        wrow = (size_t)((gt & 1) ? a.N[0] + c : c);
      } else {
        const int sg = seg_of(a, gt);
        int c = (gt - a.tb[sg]) * 16 + r;
        c = c < a.N[sg] ? c : a.N[sg] - 1;
        w = a.w[sg];
        wrow = (size_t)c;
      }
      src[i] = w + wrow * K + 8 * lkb;
      ld[i] = true;
    }
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

  bd_f32x4 acc[P::MW][P::NWT];
#pragma unroll
  for (int i = 0; i < P::MW; ++i)
#pragma unroll
    for (int j = 0; j < P::NWT; ++j) acc[i][j] = bd_f32x4{0.f, 0.f, 0.f, 0.f};
  // input RMSNorm: the waves of a row group (wc = 0 .. WC-1) take turns over
  // the k-steps, each summing the squares of all its row tiles on its steps;
  // the partial sums meet in LDS after the loop
  __shared__ float nsq[P::WC][kBigRows];
  float ss[P::MW];
#pragma unroll
  for (int i = 0; i < P::MW; ++i) ss[i] = 0.f;
  const uint32_t sbase = bd_stream::lds_addr(sbuf);
  const uint32_t fo[2] = {(uint32_t)bd_stream::frag_offset(lane, 0), (uint32_t)bd_stream::frag_offset(lane, 1)};
  // row tile i of this wave is row tile i*WR + wr of the block
  const uint32_t xt0 = wr * 2048, wt0 = (kBigRows / 16 + wc * P::NWT) * 2048;
  constexpr int XS = P::WR * 2048;
  const int live = min(P::MW, max(0, (live_tiles - wr + P::WR - 1) / P::WR));

#pragma unroll
  for (int c = 0; c < P::NS - 1; ++c)
    if (c < nch) issue(c);
  for (int ch = 0; ch < nch; ++ch) {
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
      const bool sq = a.norm_x && (2 * ch + ks) % P::WC == wc;
      if (sq)
#pragma unroll
        for (int i = 0; i < 4; ++i) ss[i] = bf16x8_sumsq(xa[i], ss[i]);
#pragma unroll
      for (int i0 = 4; i0 < P::MW; i0 += 4) {
        if (i0 >= live) break;
        bd_stream::lds_frags_4<XS>(st + xt0 + i0 * XS + fo[ks], xa);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (i0 + i < live)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i0 + i][j] = bd_mfma16(xa[i], wb[j], acc[i0 + i][j]);
        if (sq)
#pragma unroll
          for (int i = 0; i < 4; ++i) ss[i0 + i] = bf16x8_sumsq(xa[i], ss[i0 + i]);
      }
    }
  }

  // acc[i][j][r]: row m0 + (i*WR + wr)*16 + 4g + r, tile cb*CT + wc*NWT + j, column l16
  const int gt0 = cb * CT + wc * P::NWT;
  // input RMSNorm: nsq[0][row] becomes the scale of the block's row (no DMA in flight any more)
  if (a.norm_x) {
#pragma unroll
    for (int i = 0; i < P::MW; ++i) {
      const float t = frag_row_total(ss[i]);
      if (g == 0) nsq[wc][(i * P::WR + wr) * 16 + l16] = t;
    }
    __syncthreads();
    if (tid < kBigRows) {
      float t = nsq[0][tid];
#pragma unroll
      for (int w = 1; w < P::WC; ++w) t += nsq[w][tid];
      nsq[0][tid] = rsqrtf(t / (float)a.K + a.norm_eps);
    }
    __syncthreads();
  }
  auto row_scale = [&](int i, int r) { return a.norm_x ? nsq[0][(i * P::WR + wr) * 16 + 4 * g + r] : 1.f; };
  if (a.vec_out) {
    // Stores through LDS: in rounds of 64 rows the fp32 results (after the
    // SwiGLU gate) are staged as rows, then written out as 4-column vectors
    // (the residual added in fp32 on the way), so a wave writes whole row
    // segments instead of 2-byte scattered elements.  Row pitch TW + 16
    // floats: the four 16-lane groups of a write land in distinct banks.
    constexpr int TW = CT * 16, PITCH = TW + 16, RR = 64;
    float* lt = reinterpret_cast<float*>(sbuf);
    const int ow = swiglu ? TW / 2 : TW;  // output columns of the block
    for (int h = 0; h < kBigRows / RR; ++h) {
      if (m0 + h * RR >= a.M) break;  // the same for the whole work-group
      __syncthreads();                // the stages (or the previous round) are free
#pragma unroll
      for (int i = 0; i < P::MW; ++i) {
        const int rt = (i * P::WR + wr) * 16;
        if (rt / RR != h) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float* lrow = lt + (rt - h * RR + 4 * g + r) * PITCH;
          if (swiglu) {
#pragma unroll
            for (int j = 0; j < P::NWT; j += 2) {
              const float sc = row_scale(i, r);
              const float zg = acc[i][j][r] * sc, u = acc[i][j + 1][r] * sc;
              lrow[((wc * P::NWT + j) >> 1) * 16 + l16] = zg / (1.f + __expf(-zg)) * u;
            }
          } else {
#pragma unroll
            for (int j = 0; j < P::NWT; ++j) lrow[(wc * P::NWT + j) * 16 + l16] = acc[i][j][r];
          }
        }
      }
      __syncthreads();
      for (int c = tid; c < RR * (ow / 4); c += kBigThreads) {
        const int row = c / (ow / 4), c4 = (c % (ow / 4)) * 4;
        const int m = m0 + h * RR + row;
        if (m >= a.M) continue;
        int sg = 0, col, N;
        if (swiglu) {
          col = cb * (TW / 2) + c4;
          N = a.N[0];
        } else {
          const int gt = cb * CT + c4 / 16;
          if (gt >= T) continue;
          sg = seg_of(a, gt);
          col = (gt - a.tb[sg]) * 16 + c4 % 16;
          N = a.N[sg];
        }
        if (col >= N) continue;  // N % 4 == 0: a vector is wholly inside or outside
        const float4 v = *reinterpret_cast<const float4*>(lt + row * PITCH + c4);
        float vv[4] = {v.x, v.y, v.z, v.w};
        if (!swiglu && a.res[sg]) {
          const uint2 rv = *reinterpret_cast<const uint2*>(a.res[sg] + (size_t)bd_map_row(a.rr[sg], m) * N + col);
          vv[0] += bd_bf2f(rv.x & 0xffffu);
          vv[1] += bd_bf2f(rv.x >> 16);
          vv[2] += bd_bf2f(rv.y & 0xffffu);
          vv[3] += bd_bf2f(rv.y >> 16);
        }
        *reinterpret_cast<uint2*>(a.y[sg] + (size_t)bd_map_row(a.yr[sg], m) * N + col) =
            make_uint2(bd_pack_bf2(vv[0], vv[1]), bd_pack_bf2(vv[2], vv[3]));
      }
    }
    return;
  }
  if (swiglu) {
#pragma unroll
    for (int j = 0; j < P::NWT; j += 2) {
      const int col = ((gt0 + j) >> 1) * 16 + l16;
      if (gt0 + j >= T || col >= a.N[0]) continue;
#pragma unroll
      for (int i = 0; i < P::MW; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = m0 + (i * P::WR + wr) * 16 + 4 * g + r;
          if (m < a.M) {
            const float sc = row_scale(i, r);
            const float zg = acc[i][j][r] * sc, u = acc[i][j + 1][r] * sc;
            a.y[0][(size_t)bd_map_row(a.yr[0], m) * a.N[0] + col] = (uint16_t)bd_f2bf(zg / (1.f + __expf(-zg)) * u);
          }
        }
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < P::NWT; ++j) {
    const int gt = gt0 + j;
    if (gt >= T) continue;
    const int sg = seg_of(a, gt);
    const int col = (gt - a.tb[sg]) * 16 + l16;
    if (col >= a.N[sg]) continue;
    const int N = a.N[sg];
    const uint16_t* res = a.res[sg];
#pragma unroll
    for (int i = 0; i < P::MW; ++i) {
      float rv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {  // residual values first, then the stores
        const int m = m0 + (i * P::WR + wr) * 16 + 4 * g + r;
        rv[r] = (res && m < a.M) ? bd_bf2f(res[(size_t)bd_map_row(a.rr[sg], m) * N + col]) : 0.f;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + (i * P::WR + wr) * 16 + 4 * g + r;
        if (m < a.M) a.y[sg][(size_t)bd_map_row(a.yr[sg], m) * N + col] = (uint16_t)bd_f2bf(acc[i][j][r] + rv[r]);
      }
    }
  }
}

// K-split reduction: y[m, col] = sum over slices of part[z][m][col] (+ res),
// the slices added in order.  One thread per (row, 4 columns).  In a rotated
// segment (BD_GEMM_ROPE, segments 0 and 1) the thread of columns j..j+3 in the
// first half of a head also adds the partner columns j + d/2 .. and rotates
// the pairs (position pos_base[m / n_rows] + pos_off + m % n_rows, angle
// pos * theta^(-2j/d) in fp64, the rotation in fp32); the threads of the
// second halves have nothing to do.
__global__ __launch_bounds__(kThreads) void gemm_stream_reduce(GemmS a) {
  if (bd_guard_dead(a.g_bits, a.g_mask, a.g_n)) return;
  const int T = a.tb[a.nseg];
  const size_t Nt = (size_t)T * 16;
  const size_t t = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (t >= (size_t)a.M * T * 4) return;
  const int m = (int)(t / ((size_t)T * 4));
  const int rem = (int)(t % ((size_t)T * 4));
  const int gt = rem >> 2;
  const int sg = seg_of(a, gt);
  const int col = (gt - a.tb[sg]) * 16 + 4 * (rem & 3);
  const int N = a.N[sg];
  if (col >= N) return;
  const bool rope = a.mode == BD_GEMM_ROPE && sg < 2;
  const int half = a.d >> 1;
  if (rope && col % a.d >= half) return;
  const size_t zs = (size_t)a.M * Nt;
  const float* p = a.part + (size_t)m * Nt + (size_t)gt * 16 + 4 * (rem & 3);
  // slices in order; up to kSliceBatch slices' loads in flight at a time
  float lo[4] = {0.f, 0.f, 0.f, 0.f}, hi[4] = {0.f, 0.f, 0.f, 0.f};
  for (int z0 = 0; z0 < a.ksplit; z0 += kSliceBatch) {
    float4 v[kSliceBatch], h[kSliceBatch];
#pragma unroll
    for (int u = 0; u < kSliceBatch; ++u)
      if (z0 + u < a.ksplit) {
        v[u] = *reinterpret_cast<const float4*>(p + (z0 + u) * zs);
        if (rope) h[u] = *reinterpret_cast<const float4*>(p + (z0 + u) * zs + half);
      }
#pragma unroll
    for (int u = 0; u < kSliceBatch; ++u)
      if (z0 + u < a.ksplit) {
        lo[0] += v[u].x, lo[1] += v[u].y, lo[2] += v[u].z, lo[3] += v[u].w;
        if (rope) hi[0] += h[u].x, hi[1] += h[u].y, hi[2] += h[u].z, hi[3] += h[u].w;
      }
  }
  uint16_t* yrow = a.y[sg] + (size_t)bd_map_row(a.yr[sg], m) * N;
  if (rope) {
    const int bq = m / a.n_rows, iq = m % a.n_rows;
    const double pos = (double)(a.pos_base[bq] + a.pos_off + iq);
    const int j0 = col % a.d;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const double ang = pos * exp2(-(2.0 * (j0 + e) / a.d) * a.log2_theta);
      double sn, cs;
      sincos(ang, &sn, &cs);
      const float c = (float)cs, s = (float)sn;
      const float x1 = lo[e], x2 = hi[e];
      yrow[col + e] = (uint16_t)bd_f2bf(x1 * c - x2 * s);
      yrow[col + half + e] = (uint16_t)bd_f2bf(x2 * c + x1 * s);
    }
    return;
  }
  if (a.res[sg]) {  // residual loads first, then the stores
    const uint16_t* rrow = a.res[sg] + (size_t)bd_map_row(a.rr[sg], m) * N;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (col + e < N) lo[e] += bd_bf2f(rrow[col + e]);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (col + e < N) yrow[col + e] = (uint16_t)bd_f2bf(lo[e]);
}

// K-split reduction of a one-segment projection fused with the residual and
// the RMSNorm that follows it in a pre-norm layer:
//   y[yr(m)] = sum over slices of part[z][m] + res[rr(m)]   (stored in bf16)
//   h[hr(m)] = y[yr(m)] / sqrt(mean y^2 + eps)             (of the stored y)
// One work-group per row; thread t holds the 4-column groups t, t + 256, ...
// (rows up to kNormGroups * 1024 columns).  The row's sum of squares is added
// in a fixed order (wave sums, then the waves in order).
constexpr int kNormGroups = 4;
__global__ __launch_bounds__(kThreads) void gemm_reduce_norm(GemmS a, float eps, uint16_t* h, bd_rows hr) {
  if (bd_guard_dead(a.g_bits, a.g_mask, a.g_n)) return;
  __shared__ float red[kThreads / 64];
  const int m = blockIdx.x;
  const int N = a.N[0];
  const size_t Nt = (size_t)a.tb[a.nseg] * 16;
  const size_t zs = (size_t)a.M * Nt;
  const float* prow = a.part + (size_t)m * Nt;
  const uint16_t* rrow = a.res[0] ? a.res[0] + (size_t)bd_map_row(a.rr[0], m) * N : nullptr;
  uint16_t* yrow = a.y[0] + (size_t)bd_map_row(a.yr[0], m) * N;
  float v[kNormGroups][4];
#pragma unroll
  for (int g = 0; g < kNormGroups; ++g) v[g][0] = v[g][1] = v[g][2] = v[g][3] = 0.f;
  // slices in order; the loads of every column group of a batch of slices
  // are in flight together
  constexpr int ZB = kSliceBatch / 2;
  for (int z0 = 0; z0 < a.ksplit; z0 += ZB) {
    float4 t[kNormGroups][ZB];
#pragma unroll
    for (int g = 0; g < kNormGroups; ++g) {
      const int col = (g * kThreads + (int)threadIdx.x) * 4;
#pragma unroll
      for (int u = 0; u < ZB; ++u)
        if (col < N && z0 + u < a.ksplit) t[g][u] = *reinterpret_cast<const float4*>(prow + col + (z0 + u) * zs);
    }
#pragma unroll
    for (int g = 0; g < kNormGroups; ++g) {
      const int col = (g * kThreads + (int)threadIdx.x) * 4;
#pragma unroll
      for (int u = 0; u < ZB; ++u)
        if (col < N && z0 + u < a.ksplit)
          v[g][0] += t[g][u].x, v[g][1] += t[g][u].y, v[g][2] += t[g][u].z, v[g][3] += t[g][u].w;
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int g = 0; g < kNormGroups; ++g) {
    const int col = (g * kThreads + (int)threadIdx.x) * 4;
    if (col >= N) continue;
    if (rrow) {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[g][e] += bd_bf2f(rrow[col + e]);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[g][e] = bd_bf2f(bd_f2bf(v[g][e]));  // the stored value is what gets normalised
      ss += v[g][e] * v[g][e];
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) tot += red[w];
  const float inv = 1.f / __builtin_sqrtf(tot / (float)N + eps);
  uint16_t* hrow = h + (size_t)bd_map_row(hr, m) * N;
#pragma unroll
  for (int g = 0; g < kNormGroups; ++g) {
    const int col = (g * kThreads + (int)threadIdx.x) * 4;
    if (col >= N) continue;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      yrow[col + e] = (uint16_t)bd_f2bf(v[g][e]);
      hrow[col + e] = (uint16_t)bd_f2bf(v[g][e] * inv);
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
  const uint64_t* g_bits;
  uint64_t g_mask;
  int g_n;
  int norm_x;
  float norm_eps;
};

// fp32 projections: one thread per output element (small test shapes); in
// SwiGLU mode the thread forms the gate and the up product of its column.
__global__ __launch_bounds__(kThreads) void gemm_f32_kernel(GemmF a, int swiglu) {
  if (bd_guard_dead(a.g_bits, a.g_mask, a.g_n)) return;
  const int n = blockIdx.x * kThreads + threadIdx.x;
  const int m = blockIdx.y;
  if (n >= a.N) return;
  const float* xr = a.x + (size_t)bd_map_row(a.xr, m) * a.K;
  const float* wr = a.w + (size_t)n * a.K;
  float acc = 0.f, ss = 0.f;
  for (int k = 0; k < a.K; ++k) {
    acc += xr[k] * wr[k];
    ss += xr[k] * xr[k];
  }
  if (swiglu) {
    const float* ur = a.w + (size_t)(a.N + n) * a.K;
    float up = 0.f;
    for (int k = 0; k < a.K; ++k) up += xr[k] * ur[k];
    if (a.norm_x) {  // input RMSNorm (unit gains): both sums scale with the row
      const float sc = rsqrtf(ss / (float)a.K + a.norm_eps);
      acc *= sc;
      up *= sc;
    }
    acc = acc / (1.f + __expf(-acc)) * up;
  }
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

BdGemmPlan bd_gemm_plan(bd_dtype dt, int M, int K, const int* N, int nseg, int mode) {
  BdGemmPlan best{};
  if (dt == BD_F32 || M <= 0) return best;
  const int mt = (M + 15) / 16;
  const int mt0 = mt <= 1 ? 1 : (mt == 2 ? 2 : 4);
  const int G = mode == BD_GEMM_SWIGLU ? 2 : 1;
  int T = 0;
  if (mode == BD_GEMM_SWIGLU)
    T = 2 * ((N[0] + 15) / 16);
  else
    for (int i = 0; i < nseg; ++i) T += (N[i] + 15) / 16;
  const int Tg = T / G;
  const int nch = K / 64;
  int maxks = nch / BD_GEMM_MIN_CHUNKS;
  if (maxks < 1 || mode == BD_GEMM_SWIGLU) maxks = 1;
  double best_ns = -1;
  // candidates: row tile (16 .. 64 rows, or 128 above 64 rows), K slices, and
  // the number of passes per work-group (work-groups = units / pass size)
  for (int MT = mt0; MT <= (mt > 4 && BD_GEMM_MAX_MT >= 8 ? 8 : mt0); MT *= 2) {
    const int NTW = MT <= 4 ? 8 : 4;
    // resident work-groups: at most two per CU, fewer when the stages fill the LDS
    const int lds = kNS * 2 * (NTW + MT) * 1024;
    const int per_cu = kLdsPerCU / lds >= 2 ? 2 : 1;
    const int SLOTS = kCUs * per_cu;
    const int ny = (M + MT * 16 - 1) / (MT * 16);
    const int upp = NTW / G;  // units per pass
    for (int ks = 1; ks <= maxks; ++ks) {
      const int chunks = (nch + ks - 1) / ks;
      for (int k = 1; k <= 64; ++k) {
        const int nwg = (Tg + k * upp - 1) / (k * upp);
        if (k > 1 && nwg == (Tg + (k - 1) * upp - 1) / ((k - 1) * upp)) continue;  // same split as k - 1
        const long total = (long)nwg * ny * ks;
        const int passes = ((Tg + nwg - 1) / nwg * G + NTW - 1) / NTW;
        const double real = (double)T / ((double)nwg * passes);  // weight tiles per stage, on average
        const double per_wg = real * 2048.0 / BD_GEMM_HBM_BPNS + (MT + NTW - real) * 2048.0 / BD_GEMM_L2_BPNS;
        const double resident = (double)(total < SLOTS ? total : SLOTS);
        double stage = resident * per_wg;
        const double floor_ns = (double)BD_GEMM_LAT_NS / (kNS - 1);
        stage = stage > floor_ns ? stage : floor_ns;
        const double waves = (double)((total + SLOTS - 1) / SLOTS);
        double est = waves * passes * chunks * stage;
        if (ks > 1)
          est += BD_GEMM_RED_NS + (double)ks * M * T * 16 * 8 / BD_GEMM_PART_BPNS;
        else if (mode == BD_GEMM_ROPE)
          est += BD_GEMM_RED_NS;
        if (best_ns < 0 || est < best_ns) {
          best_ns = est;
          best.MT = MT;
          best.NTW = NTW;
          best.ny = ny;
          best.T = T;
          best.G = G;
          best.nwg = nwg;
          best.passes = passes;
          best.ksplit = ks;
        }
        if (nwg == 1) break;
      }
    }
  }
  best.ws_bytes = best.ksplit > 1 ? (size_t)best.ksplit * M * T * 16 * sizeof(float) : 0;
  // few tiles: K split over the waves of a work-group (no reduction launch),
  // one work-group per CU.  Every work-group reads all K of its rows of X
  // from L2, so long K rows stay with the K split over work-groups: measured
  // (cold caches) faster up to 4096-wide rows for one row block, up to 2048
  // for several.
  const int kmt = mt <= 1 ? 1 : (mt == 2 ? 2 : 4);
  const long kny = (M + kmt * 16 - 1) / (kmt * 16);
  const bool kw_fit = K <= 2048 || (K <= 4096 && kny == 1);
  if (BD_GEMM_KWAVE > 0 && nch >= 4 && (BD_GEMM_KWAVE > 1 || (best.ksplit > 1 && kw_fit))) {
    for (int nt = G; nt <= 2; nt += G) {
      if ((long)(T + nt - 1) / nt * kny <= kCUs) {
        best.kw_nt = nt;
        best.kw_mt = kmt;
        best.ny = (int)kny;
        best.ksplit = 1;
        best.ws_bytes = 0;
        break;
      }
    }
  }
  // large M: 256-row tiles when their blocks fill the GPU; of the two tile
  // widths the one with the fewer rounds of work-groups (one per CU) weighted
  // by the cost of its tiles (a 256-column tile costs BD_GEMM_BIG16_COST/10 of
  // a 128-column one)
  const int rbk = (M + kBigRows - 1) / kBigRows;
  if (M >= kBigRows) {
    const long t16 = (long)rbk * ((T + 15) / 16), t8 = (long)rbk * ((T + 7) / 8);
    const long r16 = (t16 + kCUs - 1) / kCUs, r8 = (t8 + kCUs - 1) / kCUs;
    int ct = 0;
    if (t16 >= kCUs || (t8 >= kCUs && r16 * BD_GEMM_BIG16_COST < r8 * 10)) ct = 16;
    else if (t8 >= kCUs) ct = 8;
    if (ct != 0) {
      best.big_ct = ct;
      best.kw_nt = 0;
      best.ksplit = 1;
      best.ws_bytes = 0;
    }
  }
  return best;
}

hipError_t bd_gemm_launch(bd_dtype dt, const BdGemmPlan& p, int M, int K, const void* x, bd_rows xr,
                          const BdGemmSeg* segs, int nseg, int mode, const BdGemmRope* rope,
                          const BdGemmNorm* post_norm, void* workspace, hipStream_t s, const bd_guard* guard,
                          float in_norm_eps) {
  const int norm_x = mode == BD_GEMM_SWIGLU && in_norm_eps >= 0.f ? 1 : 0;
  if (norm_x && p.kw_nt != 0) return hipErrorInvalidValue;  // the K split over waves has no input norm
  const uint64_t* g_bits = guard ? guard->bits : nullptr;
  const uint64_t g_mask = guard ? guard->mask : 0;
  const int g_n = guard ? guard->n : 0;
  // the RMSNorm after a one-segment projection rides on its K-split reduction
  // when there is one and the row fits a work-group's registers
  const bool fused_norm = post_norm != nullptr && dt == BD_BF16 && nseg == 1 && p.ksplit > 1 &&
                          segs[0].N % 4 == 0 && segs[0].N <= kNormGroups * kThreads * 4;
  if (dt == BD_F32) {
    for (int i = 0; i < nseg; ++i) {
      GemmF a{static_cast<const float*>(x), xr, M, K, static_cast<const float*>(segs[i].w),
              static_cast<float*>(segs[i].y), static_cast<const float*>(segs[i].res), segs[i].yr, segs[i].rr,
              segs[i].N, g_bits, g_mask, g_n, norm_x, in_norm_eps};
      hipLaunchKernelGGL(gemm_f32_kernel, dim3((segs[i].N + kThreads - 1) / kThreads, M), dim3(kThreads), 0, s,
                         a, mode == BD_GEMM_SWIGLU ? 1 : 0);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  } else {
    GemmS a{};
    a.x = static_cast<const uint16_t*>(x);
    a.xr = xr;
    a.g_bits = g_bits;
    a.g_mask = g_mask;
    a.g_n = g_n;
    a.norm_x = norm_x;
    a.norm_eps = in_norm_eps;
    a.M = M;
    a.K = K;
    a.nseg = nseg;
    a.mode = mode;
    int t = 0;
    for (int i = 0; i < nseg; ++i) {
      a.w[i] = static_cast<const uint16_t*>(segs[i].w);
      a.y[i] = static_cast<uint16_t*>(segs[i].y);
      a.res[i] = static_cast<const uint16_t*>(segs[i].res);
      a.yr[i] = segs[i].yr;
      a.rr[i] = segs[i].rr;
      a.N[i] = segs[i].N;
      a.tb[i] = t;
      t += mode == BD_GEMM_SWIGLU ? 2 * ((segs[i].N + 15) / 16) : (segs[i].N + 15) / 16;
    }
    for (int i = nseg; i <= kMaxSeg; ++i) a.tb[i] = t;
    a.vec_out = 1;
    for (int i = 0; i < nseg; ++i)
      if (segs[i].N % 4 != 0 || (reinterpret_cast<uintptr_t>(segs[i].y) & 7) != 0 ||
          (segs[i].res != nullptr && (reinterpret_cast<uintptr_t>(segs[i].res) & 7) != 0))
        a.vec_out = 0;
    a.ksplit = p.ksplit;
    a.part = p.ksplit > 1 ? static_cast<float*>(workspace) : nullptr;
    if (mode == BD_GEMM_ROPE) {
      a.pos_base = rope->pos_base;
      a.n_rows = rope->n_rows;
      a.pos_off = rope->pos_off;
      a.d = rope->d;
      a.log2_theta = std::log2((double)rope->theta);
    }
    if (p.kw_nt != 0) {  // K split over the waves
      const int groups = (p.T + p.kw_nt - 1) / p.kw_nt;
      const dim3 kgrid((unsigned)(kXcdGemm * ((groups + kXcdGemm - 1) / kXcdGemm) * p.ny));
#define BD_KWAVE(MT, NT, NS) hipLaunchKernelGGL((gemm_kwave_kernel<MT, NT, NS>), kgrid, dim3(kThreads), 0, s, a, p.ny)
      const int key = p.kw_mt * 10 + p.kw_nt;
      switch (key) {  // stages: the four rings fill at most 144 KiB of LDS
        case 11: BD_KWAVE(1, 1, 8); break;
        case 12: BD_KWAVE(1, 2, 6); break;
        case 21: BD_KWAVE(2, 1, 6); break;
        case 22: BD_KWAVE(2, 2, 4); break;
        case 41: BD_KWAVE(4, 1, 3); break;
        default: BD_KWAVE(4, 2, 3); break;
      }
#undef BD_KWAVE
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    } else if (p.big_ct != 0) {  // 256-row tiles, no K split
      const int rbk = (M + kBigRows - 1) / kBigRows, cbk = (p.T + p.big_ct - 1) / p.big_ct;
      const int row_major = rbk * kBigRows > cbk * p.big_ct * 16 ? 1 : 0;  // more rows than weight columns
      const dim3 bgrid((unsigned)(row_major ? 8 * ((rbk + 7) / 8) * cbk : 8 * ((cbk + 7) / 8) * rbk));
      if (p.big_ct == 16)
        hipLaunchKernelGGL(gemm_big_kernel<16>, bgrid, dim3(kBigThreads), 0, s, a, rbk, cbk, row_major);
      else
        hipLaunchKernelGGL(gemm_big_kernel<8>, bgrid, dim3(kBigThreads), 0, s, a, rbk, cbk, row_major);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    } else {
      const dim3 grid(p.nwg, p.ny, p.ksplit);
      switch (p.MT) {
        case 1: hipLaunchKernelGGL((gemm_stream_kernel<1, 8>), grid, dim3(kThreads), 0, s, a, p.passes, p.G); break;
        case 2: hipLaunchKernelGGL((gemm_stream_kernel<2, 8>), grid, dim3(kThreads), 0, s, a, p.passes, p.G); break;
        case 4:
          if (p.NTW == 8)
            hipLaunchKernelGGL((gemm_stream_kernel<4, 8>), grid, dim3(kThreads), 0, s, a, p.passes, p.G);
          else
            hipLaunchKernelGGL((gemm_stream_kernel<4, 4>), grid, dim3(kThreads), 0, s, a, p.passes, p.G);
          break;
        default: hipLaunchKernelGGL((gemm_stream_kernel<8, 4>), grid, dim3(kThreads), 0, s, a, p.passes, p.G); break;
      }
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      if (fused_norm) {
        hipLaunchKernelGGL(gemm_reduce_norm, dim3(M), dim3(kThreads), 0, s, a, post_norm->eps,
                           static_cast<uint16_t*>(post_norm->h), post_norm->hr);
        return hipGetLastError();
      }
      if (p.ksplit > 1) {
        const size_t n = (size_t)M * p.T * 4;
        hipLaunchKernelGGL(gemm_stream_reduce, dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads), 0, s,
                           a);
        hipError_t e2 = hipGetLastError();
        if (e2 != hipSuccess || post_norm == nullptr) return e2;
      }
    }
  }
  if (post_norm != nullptr && !fused_norm)
    return bd_rmsnorm_launch(dt, M, segs[0].N, segs[0].y, segs[0].yr, post_norm->eps, post_norm->h, post_norm->hr, s);
  // rotary embedding as its own pass where the projection had no reduction
  // (the K-split-over-waves kernel rotates its pair tiles itself)
  const bool rotated_in_kernel = dt == BD_BF16 && p.kw_nt != 0 && mode == BD_GEMM_ROPE && rope->d % 16 == 0;
  if (mode == BD_GEMM_ROPE && (dt == BD_F32 || p.ksplit == 1) && !rotated_in_kernel) {
    for (int i = 0; i < 2 && i < nseg; ++i) {
      hipError_t e = bd_rope_launch(dt, M / rope->n_rows, rope->n_rows, segs[i].N / rope->d, rope->d, segs[i].y,
                                    segs[i].yr, rope->pos_base, rope->pos_off, rope->theta, s);
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
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
