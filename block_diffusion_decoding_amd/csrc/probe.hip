// Measurement support, not a step of the method: the streaming LM head's
// global->LDS load pattern with no arithmetic.  Work-group w takes an equal
// range of 16-row tiles of a row-major [rows, row_bytes] matrix and walks it
// in passes of 8 tiles, one 128-byte piece of every row of the pass per
// stage (two whole-line DMA instructions of 8 rows x 128 B per tile, the
// weight tiles with the non-temporal hint), through a 3-stage LDS ring with a
// barrier per stage; with x_tiles = 4 each stage also loads the matching
// 128-byte piece of 64 rows of x, as the LM head loads its rows.  Timed next
// to the LM head on the same matrix, it separates the cost of the load
// pattern from that of the rest of the kernel.
#include "bd_launch.h"
#include "stream_gemm.h"

namespace {

template <int XT>
__global__ __launch_bounds__(256, 2) void probe_stream_kernel(const uint8_t* w, int tiles, int row_bytes,
                                                              const uint8_t* x) {
  constexpr int NS = 3;
  __shared__ uint4 ring[NS][1024 + XT * 128];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wg = blockIdx.x, nwg = gridDim.x;
  const int t0 = (int)((long)wg * tiles / nwg), t1 = (int)((long)(wg + 1) * tiles / nwg);
  const int chunks = row_bytes / 128;
  const int nst = (t1 - t0 + 7) / 8 * chunks;  // stages: passes x 128-byte pieces
  for (int s = 0; s < nst; ++s) {
    if (s >= NS - 1) __builtin_amdgcn_s_waitcnt(bd_stream::vmcnt_imm((4 + XT / 2) * (NS - 2)));
    __builtin_amdgcn_s_barrier();
    uint4* slot = ring[s % NS];
    const int p = s / chunks, c = s - p * chunks;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int f = wave + 4 * i;  // rows 8*(f%2)..+7 of the pass's tile f/2
      int t = t0 + p * 8 + (f >> 1);
      t = t < t1 ? t : t1 - 1;     // a short last pass re-reads its last tile
      const size_t row = (size_t)t * 16 + 8 * (f & 1) + (lane >> 3);
      __builtin_amdgcn_global_load_lds((bd_stream::glb_void_t*)(w + row * row_bytes + c * 128 + (lane & 7) * 16),
                                       (bd_stream::lds_void_t*)(slot + f * 64), 16, 0, 2);
    }
#pragma unroll
    for (int i = 0; i < XT / 2; ++i) {
      const int f = wave + 4 * i;  // rows 8f .. 8f+7 of x
      const size_t row = (size_t)8 * f + (lane >> 3);
      __builtin_amdgcn_global_load_lds((bd_stream::glb_void_t*)(x + row * row_bytes + c * 128 + (lane & 7) * 16),
                                       (bd_stream::lds_void_t*)(slot + 1024 + f * 64), 16, 0, 0);
    }
  }
  __builtin_amdgcn_s_waitcnt(bd_stream::vmcnt_imm(0));  // no DMA into this LDS after the work-group ends
  __syncthreads();
}

}  // namespace

extern "C" bd_status bd_probe_weight_stream(const void* w, int rows, int row_bytes, const void* x, int x_tiles,
                                            int work_groups, void* stream) {
  if (!w || rows < 16 || rows % 16 != 0 || row_bytes < 128 || row_bytes % 128 != 0) return BD_EINVAL;
  if ((x_tiles != 0 && x_tiles != 4) || (x_tiles != 0 && !x)) return BD_EINVAL;
  if ((reinterpret_cast<uintptr_t>(w) & 15u) != 0 || (x && (reinterpret_cast<uintptr_t>(x) & 15u) != 0))
    return BD_EINVAL;
  const int tiles = rows / 16;
  if (work_groups < 1 || work_groups > 4096 || work_groups > tiles) return BD_EINVAL;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const uint8_t* wp = static_cast<const uint8_t*>(w);
  const uint8_t* xp = static_cast<const uint8_t*>(x);
  if (x_tiles == 4)
    hipLaunchKernelGGL(probe_stream_kernel<4>, dim3(work_groups), dim3(256), 0, s, wp, tiles, row_bytes, xp);
  else
    hipLaunchKernelGGL(probe_stream_kernel<0>, dim3(work_groups), dim3(256), 0, s, wp, tiles, row_bytes, xp);
  return bd_hip_status(hipGetLastError());
}
