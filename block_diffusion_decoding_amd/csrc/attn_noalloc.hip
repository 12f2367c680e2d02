// bd_block_attn_noalloc: the hybrid-mask block attention with its split-key
// partials in a static device buffer instead of a caller workspace, for
// callers that cannot allocate device memory (see include/bd.h).
//
// The buffer is a file-scope device array.  Its name is only a host-side
// stand-in in host code, so the device address is looked up once per device
// with hipGetSymbolAddress (that device current) and kept; the kernels get
// that address as their workspace argument, exactly as they get a caller's
// workspace from bd_block_attn.
#include <mutex>

#include "bd_launch.h"

namespace {

constexpr size_t kScratchBytes = size_t(32) << 20;  // 32 MiB per GPU
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's copy of `scratch` (looked up on first use).
bd_status scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return bd_hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return BD_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return bd_hip_status(e);
    if (p == nullptr) return BD_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return BD_OK;
}

}  // namespace

extern "C" {

size_t bd_block_attn_noalloc_scratch_bytes(void) { return kScratchBytes; }

bd_status bd_block_attn_noalloc(bd_dtype dt, int B, int Hq, int Hkv, int d, int D, const void* q, int n_q,
                                int q_off, const void* k_cache, const void* v_cache, const int32_t* kv_len,
                                int cap, const void* k_blk, const void* v_blk, int n_blk, float scale, void* o,
                                float* lse, void* stream) {
  // every argument error is reported before the scratch lookup touches HIP
  const bd_status chk = bd_block_attn_check(dt, B, Hq, Hkv, d, D, q, n_q, q_off, k_cache, v_cache, kv_len, cap,
                                            k_blk, v_blk, n_blk, scale, o);
  if (chk != BD_OK || B == 0 || n_q == 0) return chk;
  const size_t need = bd_attn_plan(dt, B, Hq, Hkv, d, n_q, cap, n_blk).ws_bytes;
  if (need > kScratchBytes) return BD_ESCRATCH;
  void* ws = nullptr;
  if (need > 0) {
    const bd_status st = scratch_ptr(&ws);
    if (st != BD_OK) return st;
  }
  return bd_block_attn(dt, B, Hq, Hkv, d, D, q, n_q, q_off, k_cache, v_cache, kv_len, cap, k_blk, v_blk, n_blk,
                       scale, o, lse, ws, need > 0 ? kScratchBytes : 0, stream);
}

}  // extern "C"
