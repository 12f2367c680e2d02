// Skinny bf16 GEMM core for gfx950: C[m, n] = sum_k X[m, k] * W[n, k] with a
// small number of rows m (the fresh block rows of a refinement step) and a
// long weight matrix W [N, K] streamed once from HBM.
//
// Work-group = 4 waves.  A work-group owns MT*16 rows of X and 4*NT*16
// columns; wave w owns columns [col0 + w*NT*16, +NT*16).  K is walked in
// chunks of KC.  Each X chunk is staged in LDS in MFMA fragment order (a
// wave reads one fragment as one contiguous 1 KiB) and shared by the 4
// waves; W is loaded straight into registers in the B-operand layout, one
// chunk ahead of the MFMAs (register double buffering), 64 contiguous bytes
// of one W row per lane per 128-wide K group.
//
// K slots of v_mfma_f32_16x16x32_bf16: in K group kg (128 wide) and step ks
// (0..3), lane group g = lane / 16 supplies k = kg*128 + 8*g + 32*ks + 0..7
// for both operands, so each lane's four W loads of a K group are 64
// contiguous bytes.
#pragma once

#include "bd_device.h"

namespace bd_skinny {

constexpr int kThreads = 256;

template <int MT, int KC>
struct XStage {
  static constexpr int KG = KC / 128;
  static constexpr int N16 = MT * 16 * KC / 8;           // 16-byte pieces per chunk
  static constexpr int PER_T = (N16 + kThreads - 1) / kThreads;
  static constexpr int LDS_U4 = MT * KG * 4 * 64;        // uint4 per buffer
};

// X rows are fetched through a row functor: xrow(m) -> pointer to row m (K
// elements) or nullptr for a zero row.
template <int MT, int NT, int KC, class XRowF>
__device__ __forceinline__ void mainloop(const XRowF& xrow, int m0, const uint16_t* __restrict__ W,
                                         int N, int K, int col0, uint4* sX /* 2 buffers */,
                                         bd_f32x4 (&acc)[MT][NT]) {
  using XS = XStage<MT, KC>;
  constexpr int KG = XS::KG;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int l16 = lane & 15;
  const int nch = K / KC;

#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = bd_f32x4{0.f, 0.f, 0.f, 0.f};

  const uint16_t* wrow[NT];
  bool wok[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int col = col0 + nt * 16 + l16;
    wok[nt] = col < N;
    wrow[nt] = W + (size_t)(wok[nt] ? col : 0) * K + 8 * g;
  }

  uint4 xr[XS::PER_T];
  auto load_x = [&](int ch) {
#pragma unroll
    for (int u = 0; u < XS::PER_T; ++u) {
      const int e = tid + kThreads * u;
      xr[u] = make_uint4(0, 0, 0, 0);
      if (e < XS::N16) {
        const int ml = e / (KC / 8), c8 = e % (KC / 8);
        const uint16_t* p = xrow(m0 + ml);
        if (p != nullptr) xr[u] = *reinterpret_cast<const uint4*>(p + ch * KC + c8 * 8);
      }
    }
  };
  auto store_x = [&](int sb) {
#pragma unroll
    for (int u = 0; u < XS::PER_T; ++u) {
      const int e = tid + kThreads * u;
      if (e < XS::N16) {
        const int ml = e / (KC / 8), c8 = e % (KC / 8);
        const int mt = ml >> 4, r = ml & 15;
        const int kk = c8 * 8;
        const int kg = kk >> 7, within = kk & 127;
        const int ks = within >> 5, gg = (within & 31) >> 3;
        sX[sb * XS::LDS_U4 + ((mt * KG + kg) * 4 + ks) * 64 + gg * 16 + r] = xr[u];
      }
    }
  };
  auto load_w = [&](uint4 (&wb)[NT][KG][4], int ch) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int kg = 0; kg < KG; ++kg)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          wb[nt][kg][ks] = wok[nt] ? *reinterpret_cast<const uint4*>(wrow[nt] + ch * KC + kg * 128 + 32 * ks)
                                   : make_uint4(0, 0, 0, 0);
  };
  auto compute = [&](const uint4 (&wb)[NT][KG][4], int sb) {
#pragma unroll
    for (int kg = 0; kg < KG; ++kg)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        uint4 af[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) af[mt] = sX[sb * XS::LDS_U4 + ((mt * KG + kg) * 4 + ks) * 64 + lane];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = bd_mfma16(af[mt], wb[nt][kg][ks], acc[mt][nt]);
      }
  };

  uint4 w0[NT][KG][4], w1[NT][KG][4];
  load_x(0);
  load_w(w0, 0);
  store_x(0);
  __syncthreads();
  int ch = 0;
  while (true) {
    if (ch + 1 < nch) {
      load_x(ch + 1);
      load_w(w1, ch + 1);
    }
    compute(w0, ch & 1);
    if (ch + 1 < nch) store_x((ch + 1) & 1);
    __syncthreads();
    if (++ch >= nch) break;
    if (ch + 1 < nch) {
      load_x(ch + 1);
      load_w(w0, ch + 1);
    }
    compute(w1, ch & 1);
    if (ch + 1 < nch) store_x((ch + 1) & 1);
    __syncthreads();
    if (++ch >= nch) break;
  }
}

}  // namespace bd_skinny
