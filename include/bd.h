/*
 * bd.h -- C ABI of libbd: one block-diffusion refinement step on MI355X (gfx950).
 *
 * The method (Fast-dLLM v2) decodes a sequence block by block.  Inside the
 * current block of D positions the model refines masked positions in
 * parallel; finished blocks become read-only context in a block-level KV
 * cache.  One refinement step is:
 *
 *   input rows + Q/K/V projections     bd_embed_rows, bd_qkv_proj   (support)
 *   hybrid-mask GQA attention           bd_block_attn
 *   output projection + residual        bd_linear                    (support)
 *   LM head with token shift + softmax
 *     confidence / argmax               bd_lmhead_confidence
 *     (only the masked candidates)      bd_candidate_rows + bd_lmhead_confidence_rows
 *   confidence-threshold unmasking      bd_threshold_unmask
 *     (LM head + unmask, one call)      bd_lmhead_unmask
 *     (per-sequence windows)            bd_threshold_unmask_windows, bd_copy_rows,
 *                                       bd_persequence_schedule
 *   (block finished) cache append       bd_kv_append
 *
 * Sources, by page title and section:
 *   [v2 notes]   "Fast-dLLM v2: Efficient Block-Diffusion LLM" (ICLR 2026 paper
 *                notes): Framework, flowchart, Key designs 1-4.
 *   [v1 article] "Fast-dLLM: Training-free Acceleration of Diffusion LLM by
 *                Enabling KV Cache and Parallel Decoding" (article), Core
 *                technique 1 (block-wise KV cache, DualCache) and 2
 *                (confidence-aware parallel decoding).
 *   [v2 news]    Fast-dLLM v2 news article: block structure and hierarchical
 *                cache paragraphs.
 *
 * Conventions (every call):
 *   - Tensor pointers are DEVICE pointers owned by the caller, dense row-major
 *     in the layouts given below.  The library never allocates or frees them.
 *   - Scratch memory, where a call needs it, is a caller-owned device
 *     `workspace` of at least the size the matching *_workspace_size()
 *     returns.  It must be zero-filled before its first use and may then be
 *     reused by later calls on the same stream; it must not be shared by
 *     calls that can run concurrently.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream) and return at once.  Argument errors are detected on the host
 *     before anything is launched and return BD_EINVAL (or BD_ECAPACITY /
 *     BD_EUNSUPPORTED); nothing is written in that case.  A launch failure
 *     returns BD_EHIP and bd_last_hip_error() gives the hipError_t.
 *   - Empty work (B == 0, n_q == 0, M == 0, n_rows == 0) is a no-op returning
 *     BD_OK.
 *   - dtype selects the storage type of the floating-point tensors (fp32 or
 *     bf16).  Accumulation is always fp32; conf, max, lse are fp32; token
 *     ids and indices are int32.
 *   - No exceptions cross the ABI; the only global state is the last HIP error
 *     (thread-local).
 */
#ifndef BD_H
#define BD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum bd_status {
  BD_OK = 0,
  BD_EINVAL = 1,        /* bad argument (null pointer, shape, small workspace) */
  BD_EUNSUPPORTED = 2,  /* valid but not implemented (e.g. head dim) */
  BD_ECAPACITY = 3,     /* a cache append would exceed its capacity */
  BD_EHIP = 4,          /* a HIP runtime call failed */
  BD_ESCRATCH = 5       /* needs more scratch than the static buffer of
                           bd_block_attn_noalloc holds */
} bd_status;

typedef enum bd_dtype { BD_F32 = 0, BD_BF16 = 1 } bd_dtype;

/* Row map of a 2-D operand: logical row r lives at buffer row
 *   (r / group) * stride + offset + (r % group).
 * {n, n, 0} is the dense identity for an operand of n rows.  It lets one call
 * read or write a window of rows of every sequence of a [B, R, cols] buffer:
 * {rows_per_seq, R, first_row}.  group >= 1, stride >= 0, offset >= 0. */
typedef struct bd_rows {
  int32_t group;
  int32_t stride;
  int32_t offset;
} bd_rows;

/* An optional condition on a call, tested on the device when its kernels run:
 * the call does nothing (its outputs keep their contents) when no bits[b],
 * 0 <= b < n, has a bit of mask set.  In a refinement step: bits = the
 * batch's mask bits, mask = the window's positions, so that a step slot past
 * the end of its window (queued before the host knows the window is done)
 * skips its work.  The struct is read on the host during the call; bits is a
 * device pointer (8-byte aligned), 1 <= n <= 4096.  Calls that take a guard
 * pointer accept NULL (always run). */
typedef struct bd_guard {
  const uint64_t* bits;
  uint64_t mask;
  int32_t n;
} bd_guard;

const char* bd_version(void);
const char* bd_status_string(bd_status s);
/* hipError_t of the last failed HIP call on this thread (0 if none). */
int bd_last_hip_error(void);

/* ------------------------------------------------------------------------
 * bd_block_attn -- hybrid-mask grouped-query attention of the fresh rows of
 * the current block ([v2 notes] Framework and Key design 2: attention is
 * bidirectional inside a block and causal across blocks; the own block is
 * seen whole, masked positions included; [v2 news] block structure).
 *
 *   q       [B, n_q, Hq, d]     queries of in-block rows q_off .. q_off+n_q-1
 *   k_cache [B, Hkv, cap, d]    block-level cache: committed rows [0, kv_len[b])
 *   v_cache [B, Hkv, cap, d]    ([v2 notes] Key design 3: finished blocks are
 *                                read-only context)
 *   kv_len  [B] int32 (device)  committed length per sequence (ragged); values
 *                               are clamped to [0, cap]
 *   k_blk   [B, n_blk, Hkv, d]  K/V of the in-block rows: the fresh rows of this
 *   v_blk   [B, n_blk, Hkv, d]  step plus, in a DualCache step, the snapshot rows
 *                               of the rest of the block ([v2 notes] Key design 3;
 *                               [v1 article] Core technique 1).  n_blk = D for a
 *                               refinement step, a multiple of D for a multi-block
 *                               prefill.
 *   o       [B, n_q, Hq, d]     output (dtype of q)
 *   lse     [B, Hq, n_q] fp32   natural log-sum-exp of the scaled scores, or NULL
 *
 * Query row i (in-block row r = q_off + i, block index r / D) sees every cache
 * row and the in-block rows c with c / D <= r / D.  Query head h reads KV head
 * h / (Hq / Hkv).  Scores are scale * q.k.  Supported: d in {64, 128}; bf16
 * uses MFMA, fp32 a plain VALU kernel.  Requires Hq % Hkv == 0, D >= 1,
 * q_off + n_q <= n_blk, n_blk % D == 0.
 * ---------------------------------------------------------------------- */
size_t bd_block_attn_workspace_size(bd_dtype dt, int B, int Hq, int Hkv, int d, int n_q,
                                    int cap, int n_blk);
bd_status bd_block_attn(bd_dtype dt, int B, int Hq, int Hkv, int d, int D,
                        const void* q, int n_q, int q_off,
                        const void* k_cache, const void* v_cache, const int32_t* kv_len, int cap,
                        const void* k_blk, const void* v_blk, int n_blk,
                        float scale, void* o, float* lse,
                        void* workspace, size_t ws_bytes, void* stream);
/* bd_block_attn with a guard (see bd_guard): nothing is computed or written
 * when the guard's condition fails on the device. */
bd_status bd_block_attn_guarded(bd_dtype dt, int B, int Hq, int Hkv, int d, int D,
                                const void* q, int n_q, int q_off,
                                const void* k_cache, const void* v_cache, const int32_t* kv_len, int cap,
                                const void* k_blk, const void* v_blk, int n_blk,
                                float scale, void* o, float* lse,
                                void* workspace, size_t ws_bytes, const bd_guard* guard, void* stream);

/* bd_block_attn_noalloc -- bd_block_attn without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  Same arguments,
 * layouts, mask, results and error checks as bd_block_attn; the split-key
 * partials live in a static device buffer of the library instead
 * (bd_block_attn_noalloc_scratch_bytes() bytes, 32 MiB, one per GPU the
 * library runs on, held until the process ends).  The call allocates and frees
 * nothing: the buffer's address is looked up once per device (with that device
 * current) on the first call there.
 *   Returns BD_ESCRATCH, before any launch, when the problem needs more than
 *   the buffer holds (bd_block_attn_workspace_size() of the same arguments;
 *   every refinement step of the 7B workloads up to 32 sequences x 16384
 *   committed rows fits; a multi-block prefill may not).
 *   The stream must belong to the current device.  Every call on a GPU shares
 *   that GPU's buffer: calls that can overlap on one GPU (different streams,
 *   threads or processes sharing a context) race and must be serialised by
 *   the caller.  Nothing in the buffer needs clearing between calls. */
bd_status bd_block_attn_noalloc(bd_dtype dt, int B, int Hq, int Hkv, int d, int D, const void* q, int n_q,
                                int q_off, const void* k_cache, const void* v_cache, const int32_t* kv_len,
                                int cap, const void* k_blk, const void* v_blk, int n_blk, float scale, void* o,
                                float* lse, void* stream);
size_t bd_block_attn_noalloc_scratch_bytes(void);

/* ------------------------------------------------------------------------
 * bd_lmhead_confidence -- LM head with token shift and fused softmax
 * statistics ([v2 notes] Key design 2: the prediction for a masked position i
 * is read from the output row of position i-1; [v1 article] Core technique 2:
 * the confidence of a position is the probability the model gives its
 * predicted token).
 *
 *   h_src   [n_src, hidden]     output rows (dtype)
 *   row_idx [M] int32 (device)  output row m uses h_src[row_idx[m]]; NULL =
 *                               identity (M <= n_src).  The token shift is
 *                               expressed here.  An index outside [0, n_src)
 *                               yields argmax -1 and NaN statistics for that row.
 *   w       [V, hidden]         LM-head weights, row-major (dtype)
 *   argmax  [M] int32           lowest vocabulary id among the maximal logits
 *   conf    [M] fp32            max softmax probability = exp(max - lse)
 *   max_logit, lse [M] fp32     max logit and natural log-sum-exp (may be NULL)
 *   logits  [M, V] fp32         debug dump of the logits, or NULL
 *
 * The logits are never materialised unless `logits` is given.
 * ---------------------------------------------------------------------- */
size_t bd_lmhead_workspace_size(bd_dtype dt, int M, int hidden, int V);
bd_status bd_lmhead_confidence(bd_dtype dt, int M, int hidden, int V,
                               const void* h_src, int n_src, const int32_t* row_idx,
                               const void* w,
                               int32_t* argmax, float* conf, float* max_logit, float* lse,
                               float* logits,
                               void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * bd_candidate_rows -- the LM-head rows a refinement step needs: only masked
 * positions of the active window are candidates ([v2 notes] Key design 3),
 * and candidate j reads the output row of position j-1 ([v2 notes] Key
 * design 2).  Lists them batch-wide in (sequence, position) order.
 *
 *   mask_bits [B] uint64 (device)  bit j set <=> position j still [MASK]
 *   win_lo, win_len                window [win_lo, win_lo + win_len), win_len <= 64
 *   rows_per_seq                   rows of the output-row buffer per sequence:
 *                                  row b*rows_per_seq + j holds the output of
 *                                  position j-1 (row 0 = the carry), so the
 *                                  source row of candidate (b, j) is
 *                                  b*rows_per_seq + j; needs rows_per_seq > win_lo + win_len - 1
 *   row_idx  [B*win_len] int32     out: source row of the k-th candidate
 *   out_pos  [B*win_len] int32     out: b*win_len + (j - win_lo) of the k-th candidate
 *   count    [1] int32             out: number of candidates
 * Entries k >= count are set to -1.  B*win_len <= 4096.
 * ---------------------------------------------------------------------- */
bd_status bd_candidate_rows(int B, int win_lo, int win_len, const uint64_t* mask_bits, int rows_per_seq,
                            int32_t* row_idx, int32_t* out_pos, int32_t* count, void* stream);

/* ------------------------------------------------------------------------
 * bd_lmhead_confidence_rows -- bd_lmhead_confidence over a row list whose
 * length is known only on the device (the candidates of bd_candidate_rows):
 * only rows m < min(*m_dev, M) are computed, and row m's results are written
 * at out_pos[m] of the output arrays, which hold n_out entries (an out_pos
 * outside [0, n_out) drops that row's results).  M is the capacity of
 * row_idx/out_pos and sizes the workspace (bd_lmhead_workspace_size(dt, M,
 * ...)); the launch covers M rows, work beyond the count exits early.  Same
 * statistics and argument rules as bd_lmhead_confidence otherwise; the
 * debug dump, if given, is [M, V] in list order.
 * ---------------------------------------------------------------------- */
bd_status bd_lmhead_confidence_rows(bd_dtype dt, int M, int hidden, int V,
                                    const void* h_src, int n_src, const int32_t* row_idx,
                                    const int32_t* out_pos, const int32_t* m_dev, int n_out,
                                    const void* w,
                                    int32_t* argmax, float* conf, float* max_logit, float* lse,
                                    float* logits,
                                    void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * bd_threshold_unmask -- confidence-aware parallel unmasking in the active
 * window ([v2 notes] Key design 3; [v1 article] Core technique 2).
 *
 * Window = positions [win_lo, win_lo + win_len) of each sequence's block.
 *   conf, argmax [B, win_len]   entry r predicts position win_lo + r
 *   tokens       [B, D] int32   in/out: unmasked positions receive argmax
 *   mask_bits    [B] uint64     in/out: bit j set <=> position j is [MASK]
 *   n_unmasked   [B] int32      out: number unmasked in this step (may be NULL)
 *   unmasked_pos [B, win_len]   out: unmasked positions ascending, -1 padded
 *                               (may be NULL)
 * Candidates are masked window positions.  Every candidate with
 * conf > threshold is unmasked; if candidates exist and none passes, the single
 * most confident candidate is (lowest position on ties).  threshold = 1.0 thus
 * decodes one token per step.  Requires 1 <= D <= 64,
 * 0 <= win_lo, win_lo + win_len <= D, win_len <= 64.
 * ---------------------------------------------------------------------- */
bd_status bd_threshold_unmask(int B, int D, int win_lo, int win_len,
                              const float* conf, const int32_t* argmax, float threshold,
                              int32_t* tokens, uint64_t* mask_bits,
                              int32_t* n_unmasked, int32_t* unmasked_pos, void* stream);

/* The same rule with a per-sequence threshold read from device memory
 * (threshold [B] fp32) when the kernel runs: a captured step graph can then
 * follow a threshold schedule (the pages leave adaptive thresholds to future
 * work; the value is the caller's).  A NaN threshold passes no candidate
 * (the fallback still unmasks one). */
bd_status bd_threshold_unmask_tau(int B, int D, int win_lo, int win_len,
                                  const float* conf, const int32_t* argmax, const float* threshold,
                                  int32_t* tokens, uint64_t* mask_bits,
                                  int32_t* n_unmasked, int32_t* unmasked_pos, void* stream);

/* The same rule with each sequence's own window (per-sequence window
 * progression, where every sequence advances through its block on its own
 * schedule; the tokens are those of the lockstep schedule, since a sequence
 * with no candidate changes no state):
 *   win_lo [B] int32 (device)   window of sequence b = [win_lo[b], win_lo[b] + win_len);
 *                               a window outside [0, D) leaves the sequence as
 *                               it is (n_unmasked 0, unmasked_pos -1)
 * Requires 1 <= win_len <= D <= 64. */
bd_status bd_threshold_unmask_windows(int B, int D, int win_len, const int32_t* win_lo,
                                      const float* conf, const int32_t* argmax, float threshold,
                                      int32_t* tokens, uint64_t* mask_bits,
                                      int32_t* n_unmasked, int32_t* unmasked_pos, void* stream);

/* Measurement support, not a step of the method: the streaming LM head's
 * load pattern with no arithmetic, so that timing it next to the LM head on
 * the same matrix separates the cost of the loads from the rest of the
 * kernel.  Work-group w of work_groups takes an equal range of the 16-row
 * tiles of w [rows, row_bytes] (row-major, device) and reads it into LDS in
 * passes of 8 tiles, one 128-byte piece of each row of the pass per stage;
 * with x_tiles = 4 every stage also reads the matching piece of 64 rows of
 * x [64, row_bytes] (device), as the LM head reads its rows.  Nothing is
 * written to memory.  Requires rows % 16 == 0, row_bytes % 128 == 0,
 * x_tiles in {0, 4} (x may be NULL when 0), 16-byte aligned pointers and
 * 1 <= work_groups <= min(4096, rows / 16); BD_EINVAL otherwise.
 * Asynchronous on `stream`. */
bd_status bd_probe_weight_stream(const void* w, int rows, int row_bytes, const void* x, int x_tiles,
                                 int work_groups, void* stream);

/* Per-sequence window schedule on the device, so that the batched steps of
 * per-sequence window progression can be queued without a host round trip
 * ([v2 notes] Key designs 3 and 4: windows of S positions decoded left to
 * right, each opened by an exact step that refreshes the DualCache snapshot).
 * Before each step every sequence b updates its state and writes the step's
 * inputs:
 *   state, device int32 [B] each, kept between steps (a block starts with
 *   win = 0, opening = 1, ran = 0):
 *     win[b]      current window (D / S: the sequence has finished the block)
 *     opening[b]  1 when this step opens window win[b] (an exact step)
 *     ran[b]      1 when the sequence took part in the previous step
 *   update: if ran[b], opening[b] = 0; then while win[b] < D / S and
 *     positions [S win[b], S win[b] + S) of mask_bits[b] are all clear:
 *     win[b] += 1, opening[b] = 1; finally ran[b] = (win[b] < D / S).
 *   outputs, device (written for every b):
 *     restore[b], save[b], save_h[b] uint64   bd_copy_rows masks: a DualCache
 *         sequence restores its snapshot K/V rows outside its window
 *         (restore); an opening sequence saves its K/V rows 0 .. D-1 (save)
 *         and output rows 1 .. D (save_h) as its new snapshot; 0 otherwise
 *     row_idx [B * S] int32   LM-head source rows in a row buffer
 *         [2, B, 1 + D, hidden] (buffer 0: this step's output rows; buffer 1:
 *         the snapshot rows, row 0 the carry): window position p reads row p
 *         of its sequence (the output of position p - 1), from buffer 0 when
 *         the step opens the window or p - 1 lies in it, else from buffer 1;
 *         a finished sequence and position 0 read the carry
 *     win_lo [B] int32        S win[b], or D for a finished sequence (for
 *                             bd_threshold_unmask_windows)
 *     kinds [B] int32 or NULL 2 win[b] + 1 for a DualCache step, 2 win[b]
 *                             for an opening step, -1 when finished
 *     live [1] int32 or NULL  incremented when some sequence takes part
 * mask_bits [B] (the batch's bits before the step) is read only.  One
 * work-group; the call is asynchronous on `stream`.  Requires
 * 1 <= S <= D <= 63 and D % S == 0 (BD_EINVAL otherwise or for a NULL
 * required pointer). */
bd_status bd_persequence_schedule(int B, int D, int S, const uint64_t* mask_bits, int32_t* win,
                                  int32_t* opening, int32_t* ran, uint64_t* restore, uint64_t* save,
                                  uint64_t* save_h, int32_t* row_idx, int32_t* win_lo, int32_t* kinds,
                                  int32_t* live, void* stream);

/* Per-sequence masked row copy (support for per-sequence window progression:
 * restoring a sequence's DualCache snapshot rows outside its window, saving
 * the rows of an exact step as the new snapshot):
 *   for every sequence b and row r < n_rows with bit r of row_mask[b] set:
 *     dst0[b, r, :] = src0[b, r, :]   (and dst1 from src1 when both are given)
 *   layouts [B, n_rows, row_bytes], row_mask [B] uint64 (device)
 * Requires n_rows <= 64, row_bytes % 16 == 0 and 16-byte aligned pointers. */
bd_status bd_copy_rows(int B, int n_rows, int row_bytes, const uint64_t* row_mask,
                       const void* src0, void* dst0, const void* src1, void* dst1, void* stream);

/* ------------------------------------------------------------------------
 * bd_lmhead_unmask -- bd_lmhead_confidence followed by bd_threshold_unmask
 * in one call, for a lockstep window of at most 64 rows ([v2 notes] Key
 * designs 2 and 3: the confidences of the window's rows decide which of its
 * masked positions are decoded).  The LM head's final reduction and the
 * threshold rule share one kernel (one work-group per sequence), which saves
 * a launch per refinement step.
 *
 *   row m = b * win_len + r predicts position win_lo + r of sequence b; its
 *   source row is h_src[row_idx[m]] (row_idx may be NULL = m)
 *   argmax, conf, max_logit, lse [B, win_len]: as bd_lmhead_confidence
 *   (max_logit and lse may be NULL); the fold order of the per-tile partials
 *   differs from bd_lmhead_confidence, so conf and lse may differ from it in
 *   the last bits
 *   threshold / threshold_dev: a fixed threshold, or (threshold_dev != NULL)
 *   a per-sequence [B] fp32 threshold read from device memory
 *   tokens, mask_bits, n_unmasked, unmasked_pos: as bd_threshold_unmask
 *   mask_bits_host [B] or NULL: the new mask bits are also written here.
 *     It must be pinned host memory from hipHostMalloc (the device writes it
 *     directly; no copy is enqueued); the values are valid on the host once
 *     the stream has passed this call (e.g. after an event recorded behind
 *     it has completed).
 *   workspace: bd_lmhead_workspace_size(dt, B * win_len, hidden, V) bytes.
 * When no sequence has a masked position in the window the LM head does no
 * work: tokens, bits and the statistics are left as they were and only
 * mask_bits_host is written.  A captured step can thus be replayed past the
 * end of its window at the cost of its other kernels.
 * Requires B * win_len <= 64 and the rules of both calls.
 * ---------------------------------------------------------------------- */
bd_status bd_lmhead_unmask(bd_dtype dt, int B, int D, int win_lo, int win_len, int hidden, int V,
                           const void* h_src, int n_src, const int32_t* row_idx, const void* w,
                           float threshold, const float* threshold_dev,
                           int32_t* argmax, float* conf, float* max_logit, float* lse,
                           int32_t* tokens, uint64_t* mask_bits, int32_t* n_unmasked,
                           int32_t* unmasked_pos, uint64_t* mask_bits_host,
                           void* workspace, size_t ws_bytes, void* stream);

/* The next step's input rows, kept current by bd_lmhead_unmask_next: after
 * the unmask, the row of every position it decoded becomes that token's
 * embedding plus the position's plant, bit for bit as bd_embed_rows writes
 * it (an invalid token: a NaN row); positions still masked keep the [MASK]
 * row they hold.  A DualCache step that follows on the same window then
 * needs no bd_embed_rows call ([v2 notes] Key design 2: a masked position
 * is embedded as [MASK], a decoded one as its token).
 *   embedding [V + 1, hidden] (the call's dtype and V)
 *   plant     [B, D, hidden] or NULL
 *   x         [B, D, hidden] the block's input rows (device; written)
 * 16-byte aligned; hidden % 8 (bf16) or % 4 (fp32) == 0, else
 * BD_EUNSUPPORTED. */
typedef struct bd_next_rows {
  const void* embedding;
  const void* plant;
  void* x;
} bd_next_rows;

/* bd_lmhead_unmask that also writes the next step's input rows (next may be
 * NULL: then it is bd_lmhead_unmask). */
bd_status bd_lmhead_unmask_next(bd_dtype dt, int B, int D, int win_lo, int win_len, int hidden, int V,
                                const void* h_src, int n_src, const int32_t* row_idx, const void* w,
                                float threshold, const float* threshold_dev,
                                int32_t* argmax, float* conf, float* max_logit, float* lse,
                                int32_t* tokens, uint64_t* mask_bits, int32_t* n_unmasked,
                                int32_t* unmasked_pos, uint64_t* mask_bits_host, const bd_next_rows* next,
                                void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * bd_kv_append -- commit a finished block to the block-level cache ([v2
 * notes] Key design 3: a decoded block's K/V become read-only context; [v2
 * news] hierarchical cache: reused like an autoregressive KV cache).
 *
 *   k_blk, v_blk [B, n_blk, Hkv, d]   rows [0, n_rows) are appended
 *   k_cache, v_cache [B, Hkv, cap, d] rows [kv_len[b], kv_len[b] + n_rows) written
 *   kv_len [B] int32 (device)         in/out: kv_len[b] += n_rows
 *   kv_len_host [B] int32 or NULL     host mirror of kv_len before the call; when
 *                                     given, overflow of cap returns BD_ECAPACITY
 *                                     before any launch.  Without it, rows that
 *                                     would land at or past cap are dropped.
 * ---------------------------------------------------------------------- */
bd_status bd_kv_append(bd_dtype dt, int B, int Hkv, int d, int cap,
                       void* k_cache, void* v_cache, int32_t* kv_len, const int32_t* kv_len_host,
                       const void* k_blk, const void* v_blk, int n_blk, int n_rows, void* stream);

/* ------------------------------------------------------------------------
 * Support calls (not one of the four steps above; they complete the step).
 * ---------------------------------------------------------------------- */

/* Input rows of the block ([v2 notes] Key design 2: a masked position takes
 * the learnable [MASK] embedding, row V of E).
 *   E [V+1, hidden]; tokens [B, D] int32; mask_bits [B] uint64, or NULL when no
 *   position is masked (then D may exceed 64, e.g. a multi-block prompt);
 *   plant [B, D, hidden] or NULL: an additive offset per block row;
 *   x [B, n_rows, hidden] out: row i of sequence b is block position row_off + i.
 * A token id outside [0, V) on an unmasked position yields a NaN row.
 * hidden must be a multiple of 8 (bf16) or 4 (fp32). */
bd_status bd_embed_rows(bd_dtype dt, int B, int D, int row_off, int n_rows, int hidden, int V,
                        const void* E, const int32_t* tokens, const uint64_t* mask_bits,
                        const void* plant, void* x, void* stream);

/* y[yr(m), n] = sum_k x[xr(m), k] * w[n, k]  (+ res[rr(m), n] when res != NULL)
 * for m < M, n < N.  x rows hold K elements, y/res rows hold N elements;
 * w is [N, K] row-major.  bf16 uses MFMA with fp32 accumulation and needs
 * K % 256 == 0; when the column tiles alone cannot fill the GPU, K is split
 * over work-groups and the slices are added in a fixed order through the
 * workspace (bd_linear_workspace_size; 0 means none is needed) by a second
 * kernel of the same call.  y may be res (same rows): each element is read
 * before it is written. */
size_t bd_linear_workspace_size(bd_dtype dt, int M, int N, int K);
bd_status bd_linear(bd_dtype dt, int M, int N, int K,
                    const void* x, bd_rows xr, const void* w,
                    const void* res, bd_rows rr, void* y, bd_rows yr,
                    void* workspace, size_t ws_bytes, void* stream);
/* bd_linear with a guard (see bd_guard). */
bd_status bd_linear_guarded(bd_dtype dt, int M, int N, int K,
                            const void* x, bd_rows xr, const void* w,
                            const void* res, bd_rows rr, void* y, bd_rows yr,
                            void* workspace, size_t ws_bytes, const bd_guard* guard, void* stream);

/* A projection into the residual stream followed by the RMSNorm of the
 * result (a pre-norm layer's output projection or down projection and the
 * norm in front of the next sublayer):
 *   y[yr(m)] += x[xr(m)] W^T                     (y: residual stream, in place)
 *   h[hr(m)]  = y[yr(m)] / sqrt(mean_k y^2 + eps)  (unit gains, of the stored y)
 * Where K is split, the norm is taken by the reduction kernel (one
 * work-group per row, bf16, N % 4 == 0 and N <= 4096); otherwise a RMSNorm
 * pass follows.  h must not overlap y.  Workspace: bd_linear_workspace_size. */
bd_status bd_linear_residual_rmsnorm(bd_dtype dt, int M, int N, int K,
                                     const void* x, bd_rows xr, const void* w,
                                     void* y, bd_rows yr, float eps, void* h, bd_rows hr,
                                     void* workspace, size_t ws_bytes, void* stream);

/* The three input projections of one attention layer in one launch:
 *   q[qr(m)] = x[xr(m)] Wq^T  (Nq columns), k[kr(m)] = x[xr(m)] Wk^T and
 *   v[vr(m)] = x[xr(m)] Wv^T  (Nkv columns each).  Workspace as bd_linear. */
size_t bd_qkv_proj_workspace_size(bd_dtype dt, int M, int K, int Nq, int Nkv);
bd_status bd_qkv_proj(bd_dtype dt, int M, int K, const void* x, bd_rows xr,
                      const void* wq, int Nq, void* q, bd_rows qr,
                      const void* wk, const void* wv, int Nkv,
                      void* k, bd_rows kr, void* v, bd_rows vr,
                      void* workspace, size_t ws_bytes, void* stream);
/* bd_qkv_proj with a guard (see bd_guard). */
bd_status bd_qkv_proj_guarded(bd_dtype dt, int M, int K, const void* x, bd_rows xr,
                              const void* wq, int Nq, void* q, bd_rows qr,
                              const void* wk, const void* wv, int Nkv,
                              void* k, bd_rows kr, void* v, bd_rows vr,
                              void* workspace, size_t ws_bytes, const bd_guard* guard, void* stream);

/* bd_qkv_proj followed by the rotary embedding of q and k (as bd_rope, with
 * H = Nq/d resp. Nkv/d heads; logical row m = b*n_rows + i sits at position
 * pos_base[b] + pos_off + i), in the same call: where K is split the rotation
 * is applied by the reduction kernel to the fp32 sums, otherwise by a rotary
 * pass over q and k.  d % 8 == 0, Nq and Nkv multiples of d, M a multiple of
 * n_rows, theta > 1.  Workspace: bd_qkv_proj_rope_workspace_size. */
size_t bd_qkv_proj_rope_workspace_size(bd_dtype dt, int M, int K, int Nq, int Nkv);
bd_status bd_qkv_proj_rope(bd_dtype dt, int M, int K, const void* x, bd_rows xr,
                           const void* wq, int Nq, void* q, bd_rows qr,
                           const void* wk, const void* wv, int Nkv,
                           void* k, bd_rows kr, void* v, bd_rows vr,
                           int d, const int32_t* pos_base, int n_rows, int pos_off, float theta,
                           void* workspace, size_t ws_bytes, void* stream);

/* Gate/up projection of a SwiGLU MLP with the gate applied in the epilogue:
 *   a[ar(m), n] = silu(x[xr(m)] . w_gu[n]) * (x[xr(m)] . w_gu[inter + n])
 * for m < M, n < inter; w_gu [2*inter, K] holds the gate rows, then the up
 * rows; silu(z) = z / (1 + exp(-z)) in fp32 on the fp32 sums.  The gate and
 * up tile of the same columns are computed by one wave, so the [M, 2*inter]
 * projection is never stored.  No workspace. */
bd_status bd_gate_up_swiglu(bd_dtype dt, int M, int K, const void* x, bd_rows xr, const void* w_gu, int inter,
                            void* a, bd_rows ar, void* stream);

/* bd_gate_up_swiglu on RMS-normalised rows (unit gains), the pre-MLP norm of
 * a pre-norm layer folded into the projection:
 *   a[ar(m), n] = silu(h_m . w_gu[n]) * (h_m . w_gu[inter + n]),
 *   h_m = x[xr(m)] / sqrt(mean_k x[xr(m)][k]^2 + eps)
 * The kernels multiply the raw rows and scale each row's gate and up sums by
 * 1/sqrt(mean x^2 + eps), its sum of squares taken from the same loads (bf16:
 * of the bf16 values, in fp32).  eps >= 0.  No workspace. */
bd_status bd_gate_up_swiglu_rmsnorm(bd_dtype dt, int M, int K, const void* x, bd_rows xr, float eps,
                                    const void* w_gu, int inter, void* a, bd_rows ar, void* stream);

/* ------------------------------------------------------------------------
 * Layer pieces of the multi-layer decode (support calls).  The pages name the
 * model family ([v2 notes] main results: Qwen2.5-style decoders adapted to
 * block diffusion) but not its layer equations; these are that family's
 * usual pieces, applied in pre-norm layers.  bf16 or fp32 storage (dt),
 * fp32 arithmetic; in place is allowed for bd_rmsnorm (x == y, same rows).
 * Rows that the row maps send to the same buffer row are undefined.
 * ---------------------------------------------------------------------- */

/* RMSNorm with unit gains: y[yr(m)] = x[xr(m)] / sqrt(mean_k x[xr(m), k]^2 + eps)
 * for m < M; rows hold `hidden` elements.  eps >= 0. */
bd_status bd_rmsnorm(bd_dtype dt, int M, int hidden, const void* x, bd_rows xr, float eps, void* y,
                     bd_rows yr, void* stream);

/* Rotary position embedding (rotate-half form), in place.  Logical row
 * m = b*n_rows + i (b < B, i < n_rows) is buffer row xr(m) of x, holding H
 * heads of d elements; it sits at position pos_base[b] + pos_off + i
 * (pos_base [B] int32 on the device, e.g. the committed lengths).  For each
 * head and j < d/2 the pair (x_j, x_{j+d/2}) is rotated by the angle
 * pos * theta^(-2j/d): (x_j cos - x_{j+d/2} sin, x_{j+d/2} cos + x_j sin).
 * d even, theta > 1. */
bd_status bd_rope(bd_dtype dt, int B, int n_rows, int H, int d, void* x, bd_rows xr, const int32_t* pos_base,
                  int pos_off, float theta, void* stream);

/* SwiGLU gate: a[ar(m), n] = silu(gu[gr(m), n]) * gu[gr(m), inter + n] for m < M,
 * n < inter, silu(z) = z / (1 + exp(-z)); rows of gu hold the gate projection
 * then the up projection (2*inter elements), rows of a hold inter; a must
 * not overlap gu. */
bd_status bd_swiglu(bd_dtype dt, int M, int inter, const void* gu, bd_rows gr, void* a, bd_rows ar,
                    void* stream);

/* ------------------------------------------------------------------------
 * Training form (forward pass and loss value only).  [v2 notes] Key design 2:
 * the noisy sequence x_t (masked positions -> [MASK]) and the clean x_0 of a
 * sample are concatenated into 2L positions and attended under one hybrid
 * mask; each sample appears twice, with a mask m and its complement; the
 * loss is the cross-entropy of the masked tokens, each predicted from the
 * logits of the position before it.
 * ---------------------------------------------------------------------- */

/* Attention over the 2L layout of S sequences (S counts every view):
 *   q [S, 2L, Hq, d], k/v [S, 2L, Hkv, d]; within a sequence rows 0..L-1 are
 *   x_t, rows L..2L-1 are x_0; block of row p = (p mod L) / D.
 *   A noisy row of block b sees the noisy rows of block b and the clean rows
 *   of blocks < b; a clean row of block b sees the clean rows of blocks <= b;
 *   clean rows never see noisy rows.  o [S, 2L, Hq, d]; scale usually 1/sqrt(d).
 * Each (sequence, half, block) is run as a block over a prefix cache (the
 * clean rows of earlier blocks), with the block's own rows as in-block keys:
 * the workspace (bd_train_attn_workspace_size, always > 0) receives the
 * clean K/V in cache layout and the per-block lengths.  L % D == 0,
 * d in {64, 128}; Hq % Hkv == 0. */
size_t bd_train_attn_workspace_size(bd_dtype dt, int S, int L, int D, int Hq, int Hkv, int d);
bd_status bd_train_attn(bd_dtype dt, int S, int L, int D, int Hq, int Hkv, int d,
                        const void* q, const void* k, const void* v, float scale, void* o,
                        void* workspace, size_t ws_bytes, void* stream);

/* Cross-entropy terms of the supervised positions:
 *   nll[m] = lse[m] - h_src[row_idx[m]] . w[target[m]]      (m < M)
 * with lse from bd_lmhead_confidence on the same rows (row_idx = the
 * token-shift source rows; NULL = identity) and w the LM head [V, hidden];
 * the dot product in fp32.  loss_sum (optional) [1] = sum_m nll[m], added in
 * a fixed order in fp64.  A row index outside [0, n_src) or a target
 * outside [0, V) gives a NaN term.  hidden % 8 == 0 (bf16) or % 4 (fp32). */
bd_status bd_masked_nll(bd_dtype dt, int M, int hidden, int V, const void* h_src, int n_src,
                        const int32_t* row_idx, const void* w, const int32_t* target, const float* lse,
                        float* nll, float* loss_sum, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BD_H */
