// Streaming skinny bf16 GEMM core for gfx950: C[m, n] = sum_k X[m, k] W[n, k]
// for a handful of rows m (the fresh block rows of a refinement step) and a
// long weight matrix W [N, K] that is read exactly once from HBM.
//
// A work-group (4 waves) owns MT*16 rows (MT in {1, 2, 4}) and NTW*16
// columns.  K is walked in chunks of KSC*32.  Every chunk is one pipeline
// stage in LDS holding, in v_mfma_f32_16x16x32_bf16 fragment order, the W
// fragments of all NTW column tiles and the X fragments of all MT row tiles;
// one fragment is 1 KiB = one global_load_lds_dwordx4 per wave (lane l's 16
// bytes land at base + 16*l), so the loads go from HBM/L2 straight into LDS
// without passing through registers and NS stages are in flight at once.
// Waves split the rows first (wave -> row tile) and the columns second, so a
// W fragment in LDS is read by MT waves and an X fragment by 4/MT waves.
//
// K slots: in k-step ks of a chunk, lane group g = lane / 16 supplies
// k = chunk*KSC*32 + 32*ks + 8*g .. +7 for both operands (any common
// permutation of the K slots leaves the product unchanged).
#pragma once

#include "bd_device.h"

namespace bd_stream {

constexpr int kThreads = 256;

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// Work-group barrier without the release/acquire fences of __syncthreads():
// those make the compiler wait for every outstanding global load (vmcnt(0))
// and would drain the load pipeline.  The loop's own s_waitcnt makes the
// awaited stage complete in LDS; the signal fences keep the compiler from
// moving memory operations across the barrier.
__device__ __forceinline__ void pipe_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// s_waitcnt immediate (gfx9 encoding) waiting for vmcnt <= n only.
__host__ __device__ constexpr int vmcnt_imm(int n) {
  return (n & 15) | (7 << 4) | (15 << 8) | (((n >> 4) & 3) << 14);
}

template <int MT_, int NTW_, int KSC_, int NS_>
struct Cfg {
  static constexpr int MT = MT_;        // row tiles per work-group
  static constexpr int NTW = NTW_;      // column tiles per work-group
  static constexpr int KSC = KSC_;      // 32-wide k-steps per chunk
  static constexpr int NS = NS_;        // pipeline stages
  static constexpr int WM = MT;         // waves along the rows
  static constexpr int WN = 4 / MT;     // waves along the columns
  static constexpr int NTP = NTW / WN;  // column tiles per wave
  static constexpr int WFR = NTW * KSC; // W fragments per stage
  static constexpr int XFR = MT * KSC;  // X fragments per stage
  static constexpr int FR = WFR + XFR;
  static constexpr int LW = (FR + 3) / 4;  // fragments (load instructions) per wave per stage, at most
  static constexpr int LW_LO = FR / 4;      // waves >= FR % 4 issue one fewer
  static constexpr int KC = KSC * 32;
  static constexpr int STAGE_U4 = FR * 64;
  static constexpr int LDS_BYTES = NS * STAGE_U4 * 16;
  static_assert(MT == 1 || MT == 2 || MT == 4, "MT");
  static_assert(NTW % WN == 0, "split");
  static_assert(NS == 2 || NS == 3, "stages");
};

// Row pointers: xrow(m) gives row m of X (K elements) or nullptr for a row
// that does not exist; such rows read row `xdummy` instead and their outputs
// are never used.  Columns >= N read row 0 of W likewise.
// K range: elements [k0, k0 + nch*KC) of rows of length K.
template <class C, class XRowF>
__device__ __forceinline__ void mainloop(const XRowF& xrow, const uint16_t* xdummy, int m0,
                                         const uint16_t* __restrict__ W, int N, int K, int n0, uint4* sbuf,
                                         bd_f32x4 (&acc)[C::NTP], int k0 = 0, int nch = -1) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;
  const int l16 = lane & 15;
  const int wm = wave % C::WM;
  const int wn = wave / C::WM;
  if (nch < 0) nch = K / C::KC;

#pragma unroll
  for (int j = 0; j < C::NTP; ++j) acc[j] = bd_f32x4{0.f, 0.f, 0.f, 0.f};

  // per-lane source pointers of this wave's fragments (chunk 0)
  const uint16_t* src[C::LW];
#pragma unroll
  for (int i = 0; i < C::LW; ++i) {
    const int f = wave + 4 * i;
    if (f >= C::FR) {
      src[i] = nullptr;
    } else if (f < C::WFR) {
      const int nt = f / C::KSC, ks = f % C::KSC;
      const int col = n0 + nt * 16 + l16;
      src[i] = W + (size_t)(col < N ? col : 0) * K + k0 + 32 * ks + 8 * g;
    } else {
      const int mt = (f - C::WFR) / C::KSC, ks = (f - C::WFR) % C::KSC;
      const uint16_t* p = xrow(m0 + mt * 16 + l16);
      src[i] = (p ? p : xdummy) + k0 + 32 * ks + 8 * g;
    }
  }
  auto issue = [&](int ch) {
    uint4* st = sbuf + (ch % C::NS) * C::STAGE_U4;
#pragma unroll
    for (int i = 0; i < C::LW; ++i)
      if (wave + 4 * i < C::FR)
        __builtin_amdgcn_global_load_lds((glb_void_t*)(src[i] + (size_t)ch * C::KC),
                                         (lds_void_t*)(st + (wave + 4 * i) * 64), 16, 0, 0);
  };
  const bool more = wave < C::FR % 4;  // this wave issues LW (else LW_LO) loads per stage

#pragma unroll
  for (int c = 0; c < C::NS - 1; ++c)
    if (c < nch) issue(c);

  for (int ch = 0; ch < nch; ++ch) {
    // chunks issued so far: min(nch, ch + NS - 1); keep the later ones in flight
    const int later = min(nch - ch - 1, C::NS - 2);
    if (later == 0) __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    else if (more) __builtin_amdgcn_s_waitcnt(vmcnt_imm(C::LW));
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(C::LW_LO));
    pipe_barrier();  // chunk ch is in LDS for every wave; slot of ch - 1 is free
    if (ch + C::NS - 1 < nch) issue(ch + C::NS - 1);
    const uint4* st = sbuf + (ch % C::NS) * C::STAGE_U4;
#pragma unroll
    for (int ks = 0; ks < C::KSC; ++ks) {
      const uint4 a = st[(C::WFR + wm * C::KSC + ks) * 64 + lane];
#pragma unroll
      for (int j = 0; j < C::NTP; ++j) {
        const int nt = wn * C::NTP + j;
        acc[j] = bd_mfma16(a, st[(nt * C::KSC + ks) * 64 + lane], acc[j]);
      }
    }
  }
  __syncthreads();  // stages may be reused by the caller's epilogue
}

}  // namespace bd_stream
