// Streaming skinny bf16 GEMM core for gfx950: C[m, n] = sum_k X[m, k] W[n, k]
// for a handful of rows m (the fresh block rows of a refinement step) and a
// long weight matrix W [N, K] that is read exactly once from HBM.
//
// A work-group (4 waves) owns MT*16 rows (MT in {1, 2, 4, 8}) and NTW*16
// columns.  K is walked in chunks of 64; every chunk is one pipeline stage in
// LDS holding the NTW column tiles of W and the MT row tiles of X, each tile
// 16 rows x 64 k = 2 KiB.  The tiles arrive by global->LDS DMA
// (global_load_lds_dwordx4: lane l's 16 bytes land at base + 16*l), NS stages
// in flight, without passing through registers.
//
// Load shape: one DMA instruction covers 8 rows x 128 B, i.e. whole 128-byte
// lines; a 16-row tile is two instructions.  (Sixteen rows x 64 B per
// instruction, the MFMA fragment shape, touches twice as many lines and
// measured about 3x slower for L2-resident rows, which is what the shared X
// rows of every work-group are.)  Lane l of an instruction loads row l/8 and
// 16-byte k-block (l%8) ^ (l/8), so LDS slot 8r+p holds k-block p^r of row r:
// the XOR swizzle makes the fragment reads below conflict-free.
//
// MFMA v_mfma_f32_16x16x32_bf16: in k-step ks (0, 1) of a chunk, lane L
// supplies row L%16 and k-block 4*ks + L/16 of its tile, read with one
// ds_read_b128 at a per-lane offset.  A wave computes MTW row tiles x NTP
// column tiles (MTW = min(MT, 2)): at 64 rows a 32x64 sub-tile, reading
// 2 X + 4 W fragments per k-step.  All fragments of a chunk are read in one
// batch before its MFMAs, so the LDS latency is paid once per chunk.
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

template <int MT_, int NTW_, int NS_>
struct Cfg {
  static constexpr int MT = MT_;        // row tiles per work-group
  static constexpr int NTW = NTW_;      // column tiles per work-group
  static constexpr int NS = NS_;        // pipeline stages
  static constexpr int MTW = MT < 2 ? MT : 2;  // row tiles per wave
  static constexpr int WM = MT / MTW;   // waves along the rows
  static constexpr int WN = 4 / WM;     // waves along the columns
  static constexpr int NTP = NTW / WN;  // column tiles per wave
  static constexpr int KSC = 2;         // 32-wide k-steps per chunk
  static constexpr int KC = 64;         // k per chunk
  static constexpr int FR = 2 * (NTW + MT);  // DMA instructions per stage (1 KiB each)
  static constexpr int LW = (FR + 3) / 4;    // instructions per wave per stage, at most
  static constexpr int LW_LO = FR / 4;       // waves >= FR % 4 issue one fewer
  static constexpr int STAGE_U4 = FR * 64;
  static constexpr int LDS_BYTES = NS * STAGE_U4 * 16;
  static_assert(MT == 1 || MT == 2 || MT == 4 || MT == 8, "MT");
  static_assert(NTW % WN == 0, "split");
  static_assert(NS >= 2 && NS <= 5, "stages");
};

// LDS byte address of a shared-memory pointer.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// One 4-byte LDS write / read as asm that waits inside the block, for use
// while global->LDS DMA is in flight (plain accesses would get a wait for
// every outstanding DMA in front of them).
__device__ __forceinline__ void lds_write_f32(uint32_t addr, float v) {
  asm volatile("ds_write_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : : "v"(addr), "v"(v) : "memory");
}
__device__ __forceinline__ float lds_read_f32(uint32_t addr) {
  float v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
  return v;
}

// Fragment reads written as asm with the wait inside the block: the compiler
// then cannot guard them with a wait for every outstanding global->LDS DMA
// (it cannot tell which LDS bytes a DMA writes), which would serialise the
// next stage's loads with this stage's MFMAs.  Tiles are 2 KiB.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 as_uint4(u32x4_t r) { return make_uint4(r[0], r[1], r[2], r[3]); }

// x[i] from a + XS*i, w[j] from b + 2048*j (byte addresses and strides).
template <int XS = 2048>
__device__ __forceinline__ void lds_frags_4x4(uint32_t a, uint32_t b, uint4 (&x)[4], uint4 (&w)[4]) {
  u32x4_t r[8];
  asm volatile(
      "ds_read_b128 %0, %8\n\t"
      "ds_read_b128 %1, %8 offset:%10\n\t"
      "ds_read_b128 %2, %8 offset:%11\n\t"
      "ds_read_b128 %3, %8 offset:%12\n\t"
      "ds_read_b128 %4, %9\n\t"
      "ds_read_b128 %5, %9 offset:2048\n\t"
      "ds_read_b128 %6, %9 offset:4096\n\t"
      "ds_read_b128 %7, %9 offset:6144\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
      : "v"(a), "v"(b), "i"(XS), "i"(2 * XS), "i"(3 * XS)
      : "memory");
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = as_uint4(r[i]);
    w[i] = as_uint4(r[4 + i]);
  }
}

// x[i] from a + XS*i.
template <int XS = 2048>
__device__ __forceinline__ void lds_frags_4(uint32_t a, uint4 (&x)[4]) {
  u32x4_t r[4];
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %4 offset:%5\n\t"
      "ds_read_b128 %2, %4 offset:%6\n\t"
      "ds_read_b128 %3, %4 offset:%7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
      : "v"(a), "i"(XS), "i"(2 * XS), "i"(3 * XS)
      : "memory");
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = as_uint4(r[i]);
}

// One k-step's fragments of a wave: NX X fragments from xa + 2048*i and NW W
// fragments from wa + 2048*j (byte addresses; tiles are 2 KiB apart).
template <int NX, int NW>
__device__ __forceinline__ void lds_frags_kstep(uint32_t xa, uint32_t wa, uint4 (&x)[NX], uint4 (&w)[NW]);

template <>
__device__ __forceinline__ void lds_frags_kstep<2, 4>(uint32_t xa, uint32_t wa, uint4 (&x)[2], uint4 (&w)[4]) {
  u32x4_t r[6];
  asm volatile(
      "ds_read_b128 %0, %6\n\t"
      "ds_read_b128 %1, %6 offset:2048\n\t"
      "ds_read_b128 %2, %7\n\t"
      "ds_read_b128 %3, %7 offset:2048\n\t"
      "ds_read_b128 %4, %7 offset:4096\n\t"
      "ds_read_b128 %5, %7 offset:6144\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5])
      : "v"(xa), "v"(wa)
      : "memory");
  x[0] = as_uint4(r[0]);
  x[1] = as_uint4(r[1]);
#pragma unroll
  for (int j = 0; j < 4; ++j) w[j] = as_uint4(r[2 + j]);
}

template <>
__device__ __forceinline__ void lds_frags_kstep<2, 2>(uint32_t xa, uint32_t wa, uint4 (&x)[2], uint4 (&w)[2]) {
  u32x4_t r[4];
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %4 offset:2048\n\t"
      "ds_read_b128 %2, %5\n\t"
      "ds_read_b128 %3, %5 offset:2048\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
      : "v"(xa), "v"(wa)
      : "memory");
  x[0] = as_uint4(r[0]);
  x[1] = as_uint4(r[1]);
  w[0] = as_uint4(r[2]);
  w[1] = as_uint4(r[3]);
}

template <>
__device__ __forceinline__ void lds_frags_kstep<1, 2>(uint32_t xa, uint32_t wa, uint4 (&x)[1], uint4 (&w)[2]) {
  u32x4_t r[3];
  asm volatile(
      "ds_read_b128 %0, %3\n\t"
      "ds_read_b128 %1, %4\n\t"
      "ds_read_b128 %2, %4 offset:2048\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2])
      : "v"(xa), "v"(wa)
      : "memory");
  x[0] = as_uint4(r[0]);
  w[0] = as_uint4(r[1]);
  w[1] = as_uint4(r[2]);
}

template <>
__device__ __forceinline__ void lds_frags_kstep<1, 1>(uint32_t xa, uint32_t wa, uint4 (&x)[1], uint4 (&w)[1]) {
  u32x4_t r[2];
  asm volatile(
      "ds_read_b128 %0, %2\n\t"
      "ds_read_b128 %1, %3\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1])
      : "v"(xa), "v"(wa)
      : "memory");
  x[0] = as_uint4(r[0]);
  w[0] = as_uint4(r[1]);
}

template <>
__device__ __forceinline__ void lds_frags_kstep<2, 1>(uint32_t xa, uint32_t wa, uint4 (&x)[2], uint4 (&w)[1]) {
  u32x4_t r[3];
  asm volatile(
      "ds_read_b128 %0, %3\n\t"
      "ds_read_b128 %1, %3 offset:2048\n\t"
      "ds_read_b128 %2, %4\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2])
      : "v"(xa), "v"(wa)
      : "memory");
  x[0] = as_uint4(r[0]);
  x[1] = as_uint4(r[1]);
  w[0] = as_uint4(r[2]);
}

template <>
__device__ __forceinline__ void lds_frags_kstep<4, 1>(uint32_t xa, uint32_t wa, uint4 (&x)[4], uint4 (&w)[1]) {
  u32x4_t r[5];
  asm volatile(
      "ds_read_b128 %0, %5\n\t"
      "ds_read_b128 %1, %5 offset:2048\n\t"
      "ds_read_b128 %2, %5 offset:4096\n\t"
      "ds_read_b128 %3, %5 offset:6144\n\t"
      "ds_read_b128 %4, %6\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4])
      : "v"(xa), "v"(wa)
      : "memory");
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = as_uint4(r[i]);
  w[0] = as_uint4(r[4]);
}

template <>
__device__ __forceinline__ void lds_frags_kstep<4, 2>(uint32_t xa, uint32_t wa, uint4 (&x)[4], uint4 (&w)[2]) {
  u32x4_t r[6];
  asm volatile(
      "ds_read_b128 %0, %6\n\t"
      "ds_read_b128 %1, %6 offset:2048\n\t"
      "ds_read_b128 %2, %6 offset:4096\n\t"
      "ds_read_b128 %3, %6 offset:6144\n\t"
      "ds_read_b128 %4, %7\n\t"
      "ds_read_b128 %5, %7 offset:2048\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5])
      : "v"(xa), "v"(wa)
      : "memory");
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = as_uint4(r[i]);
  w[0] = as_uint4(r[4]);
  w[1] = as_uint4(r[5]);
}

// N fragments from a + 2048*i (consecutive 2 KiB tiles).
template <int N>
__device__ __forceinline__ void lds_frags(uint32_t a, uint4 (&x)[N]);

template <>
__device__ __forceinline__ void lds_frags<1>(uint32_t a, uint4 (&x)[1]) {
  u32x4_t r;
  asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(r) : "v"(a) : "memory");
  x[0] = as_uint4(r);
}

template <>
__device__ __forceinline__ void lds_frags<2>(uint32_t a, uint4 (&x)[2]) {
  u32x4_t r[2];
  asm volatile(
      "ds_read_b128 %0, %2\n\t"
      "ds_read_b128 %1, %2 offset:2048\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1])
      : "v"(a)
      : "memory");
  x[0] = as_uint4(r[0]);
  x[1] = as_uint4(r[1]);
}

template <>
__device__ __forceinline__ void lds_frags<4>(uint32_t a, uint4 (&x)[4]) {
  lds_frags_4<2048>(a, x);
}

// Byte offset, inside a 2 KiB tile, of lane `lane`'s fragment for k-step ks.
__device__ __forceinline__ int frag_offset(int lane, int ks) {
  const int r = lane & 15, r7 = r & 7;
  return (r >> 3) * 1024 + (r7 * 8 + ((4 * ks + (lane >> 4)) ^ r7)) * 16;
}

}  // namespace bd_stream
