// Confidence-threshold unmasking and the block-level cache append.
//
// Unmask: "Fast-dLLM v2: Efficient Block-Diffusion LLM" notes, Key design 3
// (masked positions whose confidence exceeds the threshold are decoded in
// parallel, the rest wait; threshold 1.0 reduces to one token per step) and
// the "Fast-dLLM" v1 article, Core technique 2.  One wavefront per sequence:
// a ballot over the window's lanes gives the passing set, a wave max gives
// the fallback pick, and mbcnt-style prefix counts compact the positions.
//
// Append: Key design 3 and the v2 news article's hierarchical-cache
// paragraph -- a finished block's K/V become read-only context.
//
// Candidate rows: Key design 3 (only masked positions of the active window
// are predicted) and Key design 2 (candidate j reads the output row of
// position j-1): the masked window positions of the whole batch are listed
// in (sequence, position) order so that the LM head computes only them.
#include "bd_device.h"
#include "bd_launch.h"

namespace {

__global__ __launch_bounds__(64) void unmask_kernel(int D, int win_lo, int win_len, const float* conf,
                                                    const int32_t* argmax, float thr, const float* thr_dev,
                                                    const int32_t* win_lo_dev, int32_t* tokens, uint64_t* mask_bits,
                                                    int32_t* n_unmasked, int32_t* unmasked_pos) {
  const int b = blockIdx.x;
  const int r = threadIdx.x;
  if (thr_dev != nullptr) thr = thr_dev[b];  // per-sequence threshold from device memory
  if (win_lo_dev != nullptr) {               // per-sequence window; one outside the block changes nothing
    win_lo = win_lo_dev[b];
    if (win_lo < 0 || win_lo + win_len > D) {
      if (r == 0 && n_unmasked != nullptr) n_unmasked[b] = 0;
      if (unmasked_pos != nullptr && r < win_len) unmasked_pos[(size_t)b * win_len + r] = -1;
      return;
    }
  }
  const uint64_t bits = mask_bits[b];
  const bool in = r < win_len;
  const float c = in ? conf[(size_t)b * win_len + r] : BD_NEG_INF;
  const int32_t am = in ? argmax[(size_t)b * win_len + r] : -1;
  bd_unmask_wave(r, b, D, win_lo, win_len, bits, c, am, thr, tokens, mask_bits, n_unmasked, unmasked_pos, nullptr);
}

// One work-group per (sequence b, row r < n_rows): copies the row when bit r
// of row_mask[b] is set, from src to dst (and from src1 to dst1 when given),
// in 16-byte pieces; layouts [B, n_rows, row_bytes].
__global__ __launch_bounds__(256) void copy_rows_kernel(int n_rows, int row_bytes, const uint64_t* row_mask,
                                                        const uint8_t* src0, uint8_t* dst0, const uint8_t* src1,
                                                        uint8_t* dst1) {
  const int b = blockIdx.x, r = blockIdx.y;
  if (!((row_mask[b] >> r) & 1ull)) return;
  const size_t row = ((size_t)b * n_rows + r) * row_bytes;
  for (int e = threadIdx.x * 16; e < row_bytes; e += blockDim.x * 16) {
    *reinterpret_cast<uint4*>(dst0 + row + e) = *reinterpret_cast<const uint4*>(src0 + row + e);
    if (src1 != nullptr) *reinterpret_cast<uint4*>(dst1 + row + e) = *reinterpret_cast<const uint4*>(src1 + row + e);
  }
}

// Per-sequence window schedule (one work-group; thread t takes sequences t,
// t + blockDim.x, ...): the host's bookkeeping of per-sequence window
// progression done on the device before each batched step, so that steps can
// be queued without a host round trip.  A sequence that took part in the
// previous step has opened its window; it then moves past every window with
// no masked position left (opening the next one), and the step's inputs
// follow from its window and whether the step opens it.  Rows of the LM
// head's source buffer [2, B, 1 + D, hidden]: buffer 0 this step's output
// rows, buffer 1 the snapshot rows (row 0 the carry); window position p reads
// the output row of position p - 1, i.e. row p.
__global__ __launch_bounds__(256) void persequence_schedule_kernel(int B, int D, int S, const uint64_t* mask_bits,
                                                                   int32_t* win, int32_t* opening, int32_t* ran,
                                                                   uint64_t* restore, uint64_t* save,
                                                                   uint64_t* save_h, int32_t* row_idx,
                                                                   int32_t* win_lo, int32_t* kinds, int32_t* live) {
  __shared__ int any;
  if (threadIdx.x == 0) any = 0;
  __syncthreads();
  const int nw = D / S;
  const uint64_t full = (1ull << D) - 1ull, wmask = (1ull << S) - 1ull;
  for (int b = threadIdx.x; b < B; b += blockDim.x) {
    const uint64_t bits = mask_bits[b];
    int w = win[b], op = opening[b];
    if (ran[b]) op = 0;
    while (w < nw && ((bits >> (w * S)) & wmask) == 0) {
      ++w;
      op = 1;
    }
    const bool active = w < nw;
    win[b] = w;
    opening[b] = op;
    ran[b] = active ? 1 : 0;
    const int w0 = active ? w * S : 0;
    const uint64_t wb = wmask << w0;
    restore[b] = active && !op ? (full & ~wb) : 0ull;
    save[b] = active && op ? full : 0ull;
    save_h[b] = active && op ? (((full << 1) | 1ull) ^ 1ull) : 0ull;  // output rows 1 .. D
    win_lo[b] = active ? w0 : D;
    for (int j = 0; j < S; ++j) {
      const int q = w0 + j - 1;  // the token shift: position w0 + j reads the output of position q
      const bool fresh = op || q >= w0;
      int r;
      if (q < 0 || !active) r = (B + b) * (1 + D);
      else r = (fresh ? b : B + b) * (1 + D) + q + 1;
      row_idx[(size_t)b * S + j] = r;
    }
    if (kinds != nullptr) kinds[b] = active ? 2 * w + (op ? 0 : 1) : -1;
    if (active) any = 1;
  }
  __syncthreads();
  if (threadIdx.x == 0 && live != nullptr && any) live[0] += 1;
}

// One work-group per sequence: copy n_rows in-block rows behind the committed
// rows of every KV head, then advance the committed length.
__global__ __launch_bounds__(256) void append_kernel(int Hkv, int row_bytes, int cap, uint8_t* k_cache,
                                                     uint8_t* v_cache, int32_t* kv_len, const uint8_t* k_blk,
                                                     const uint8_t* v_blk, int n_blk, int n_rows) {
  const int b = blockIdx.x;
  int L = kv_len[b];
  L = L < 0 ? 0 : L;
  const int pieces = row_bytes / 16;
  const int total = Hkv * n_rows * pieces;
  for (int e = threadIdx.x; e < total; e += blockDim.x) {
    const int p = e % pieces;
    const int row = (e / pieces) % n_rows;
    const int h = e / pieces / n_rows;
    if (L + row >= cap) continue;
    const size_t src = (((size_t)b * n_blk + row) * Hkv + h) * row_bytes + p * 16;
    const size_t dst = (((size_t)b * Hkv + h) * cap + L + row) * row_bytes + p * 16;
    *reinterpret_cast<uint4*>(k_cache + dst) = *reinterpret_cast<const uint4*>(k_blk + src);
    *reinterpret_cast<uint4*>(v_cache + dst) = *reinterpret_cast<const uint4*>(v_blk + src);
  }
  __syncthreads();
  if (threadIdx.x == 0) kv_len[b] = L + n_rows;
}

// One work-group of 256 threads walks the B*win_len window entries in
// rounds of 256: a ballot per wave and the wave totals give each candidate
// its slot; entries past the count are set to -1.
__global__ __launch_bounds__(256) void candidates_kernel(int B, int win_lo, int win_len, const uint64_t* mask_bits,
                                                        int rows_per_seq, int32_t* row_idx, int32_t* out_pos,
                                                        int32_t* count) {
  __shared__ int wsum[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = B * win_len;
  int base = 0;
  for (int e0 = 0; e0 < n; e0 += 256) {
    const int e = e0 + tid;
    const int b = e / win_len, r = e - b * win_len;
    const int pos = win_lo + r;
    const bool cand = e < n && ((mask_bits[b < B ? b : 0] >> pos) & 1ull);
    const uint64_t bal = __ballot(cand);
    const int before = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) wsum[wave] = __popcll(bal);
    __syncthreads();
    int off = base;
    for (int w = 0; w < wave; ++w) off += wsum[w];
    if (cand) {
      row_idx[off + before] = b * rows_per_seq + pos;
      out_pos[off + before] = e;
    }
    base += wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();
  }
  for (int e = base + tid; e < n; e += 256) {
    row_idx[e] = -1;
    out_pos[e] = -1;
  }
  if (tid == 0) *count = base;
}

}  // namespace

hipError_t bd_candidates_launch(int B, int win_lo, int win_len, const uint64_t* mask_bits, int rows_per_seq,
                                int32_t* row_idx, int32_t* out_pos, int32_t* count, hipStream_t s) {
  hipLaunchKernelGGL(candidates_kernel, dim3(1), dim3(256), 0, s, B, win_lo, win_len, mask_bits, rows_per_seq,
                     row_idx, out_pos, count);
  return hipGetLastError();
}

hipError_t bd_unmask_launch(int B, int D, int win_lo, int win_len, const float* conf, const int32_t* argmax,
                            float threshold, const float* threshold_dev, int32_t* tokens, uint64_t* mask_bits,
                            int32_t* n_unmasked, int32_t* unmasked_pos, hipStream_t s, const int32_t* win_lo_dev) {
  hipLaunchKernelGGL(unmask_kernel, dim3(B), dim3(64), 0, s, D, win_lo, win_len, conf, argmax, threshold,
                     threshold_dev, win_lo_dev, tokens, mask_bits, n_unmasked, unmasked_pos);
  return hipGetLastError();
}

hipError_t bd_persequence_schedule_launch(int B, int D, int S, const uint64_t* mask_bits, int32_t* win,
                                         int32_t* opening, int32_t* ran, uint64_t* restore, uint64_t* save,
                                         uint64_t* save_h, int32_t* row_idx, int32_t* win_lo, int32_t* kinds,
                                         int32_t* live, hipStream_t s) {
  hipLaunchKernelGGL(persequence_schedule_kernel, dim3(1), dim3(256), 0, s, B, D, S, mask_bits, win, opening, ran,
                     restore, save, save_h, row_idx, win_lo, kinds, live);
  return hipGetLastError();
}

hipError_t bd_copy_rows_launch(int B, int n_rows, int row_bytes, const uint64_t* row_mask, const void* src0,
                               void* dst0, const void* src1, void* dst1, hipStream_t s) {
  hipLaunchKernelGGL(copy_rows_kernel, dim3(B, n_rows), dim3(256), 0, s, n_rows, row_bytes, row_mask,
                     static_cast<const uint8_t*>(src0), static_cast<uint8_t*>(dst0),
                     static_cast<const uint8_t*>(src1), static_cast<uint8_t*>(dst1));
  return hipGetLastError();
}

hipError_t bd_append_launch(bd_dtype dt, int B, int Hkv, int d, int cap, void* k_cache, void* v_cache,
                            int32_t* kv_len, const void* k_blk, const void* v_blk, int n_blk, int n_rows,
                            hipStream_t s) {
  const int row_bytes = d * (dt == BD_F32 ? 4 : 2);
  hipLaunchKernelGGL(append_kernel, dim3(B), dim3(256), 0, s, Hkv, row_bytes, cap,
                     static_cast<uint8_t*>(k_cache), static_cast<uint8_t*>(v_cache), kv_len,
                     static_cast<const uint8_t*>(k_blk), static_cast<const uint8_t*>(v_blk), n_blk, n_rows);
  return hipGetLastError();
}
