// LM head with token shift and fused softmax statistics.
//
// Method: "Fast-dLLM v2: Efficient Block-Diffusion LLM" notes, Key design 2
// (token shift: the prediction for masked position i is read from the output
// row of position i-1, expressed here by a row index per output row) and Key
// design 3 (confidence-threshold unmasking needs, per candidate, the predicted
// token and its probability); "Fast-dLLM" v1 article, Core technique 2 (the
// confidence of a position is the probability the model gives its token).
//
// The logits h W^T are never written to memory (unless a debug dump is
// requested).  Each work-group reduces its tile of logits to, per row,
// (max, lowest argmax, sum of exp(l - max)); a second kernel folds the tiles
// of a row in a fixed order into argmax, max, log-sum-exp and
// confidence = exp(max - lse).
//
// bf16, up to 64 rows: streaming MFMA GEMM, persistent over the vocabulary
// (lm_stream_kernel): weights streamed once from HBM through a 3-stage
// asynchronous global->LDS pipeline, every work-group an equal share; each
// lane keeps running statistics of its own columns across the passes, and
// the lanes and waves of a row meet once at the end.
// bf16, more rows (a whole batch's window or block, where the product is
// MFMA-bound): 256-row work-group tiles, see lm_big_kernel.
// fp32: plain VALU kernel.
//
// With a device-side row count (bd_lmhead_confidence_rows: the masked
// candidates listed first by bd_candidate_rows) rows past the count are
// skipped -- whole row blocks exit, and the 256-row kernel skips the loads
// and MFMAs of its row tiles past the count -- and the merge writes each
// row's statistics to its output slot.
#include <climits>

#include "bd_device.h"
#include "bd_launch.h"
#include "stream_gemm.h"

namespace {

constexpr int kThreads = 256;
// bf16 tiling; defaults chosen by measurement, overridable at build time.
#ifndef BD_LM_NTW
#define BD_LM_NTW 8
#endif
#ifndef BD_LM_NS
#define BD_LM_NS 3
#endif
// Work-groups of the streaming kernel.  For rows of 2048 and more columns
// one per CU: the weight stream runs faster with one stream per CU (a
// global->LDS read probe of the 7B head's 1.09 GB in this kernel's order:
// 158 us with 256 work-groups, 173 us with 512); narrower rows (fewer chunks
// per pass) keep two per CU.
#ifndef BD_LM_STREAM_WGS
#define BD_LM_STREAM_WGS 256
#endif
#ifndef BD_LM_STREAM_WGS_NARROW
#define BD_LM_STREAM_WGS_NARROW 512
#endif
// Cache policy of the streaming kernel's W loads: 2 = non-temporal.  The
// LM-head weights are read once per step and are far larger than the caches;
// streamed with the non-temporal hint they run faster and leave the smaller
// tensors of the step (projection weights, committed K/V) in the
// memory-side cache for the next step.
#ifndef BD_LM_AUX
#define BD_LM_AUX 2
#endif
// waves per work-group of the streaming kernel
#ifndef BD_LM_WAVES
#define BD_LM_WAVES 4
#endif
constexpr int kNTW = BD_LM_NTW;  // 16-column tiles per pass (bf16, up to 64 rows)
constexpr int kNS = BD_LM_NS;    // pipeline stages (bf16)
constexpr int kStreamWGs = BD_LM_STREAM_WGS;         // rows of >= 2048 columns
constexpr int kStreamWGsNarrow = BD_LM_STREAM_WGS_NARROW;
constexpr int kLmWaves = BD_LM_WAVES;
constexpr int kF32Rows = 16;  // rows per work-group (fp32)

struct LmK {
  const uint16_t* h;
  int n_src;
  const int32_t* row_idx;
  const uint16_t* w;
  float* logits;
  int M, hidden, V, nvt;
  float* pmax;
  int32_t* pidx;
  float* psum;
  const int32_t* m_dev;  // device row count, or NULL
  // optional skip test (the LM head fused with the unmask): the launch does
  // nothing when no sequence b < skip_B has a bit of skip_mask set in
  // skip_bits[b], i.e. no masked position is left in the window
  const uint64_t* skip_bits;
  uint64_t skip_mask;
  int skip_B;
  int32_t* ran;  // with the skip test: 1 when the launch computed, else 0
};

// Rows taken: min(M, *m_dev) when a device count is given (the row list of
// the masked candidates), else M.
__device__ __forceinline__ int lm_rows(const int32_t* m_dev, int M) {
  if (m_dev == nullptr) return M;
  const int c = *m_dev;
  return c < 0 ? 0 : (c < M ? c : M);
}

// Source row of row m, in two steps so that a wave's row-index loads can all
// be in flight before any is used: lm_row_index clamps m into [0, M) (M >= 1)
// so its load is always in bounds, lm_row_ptr rejects rows past the count
// and out-of-range indices (their outputs are never used).
__device__ __forceinline__ int lm_row_index(const LmK& a, int m) {
  const int mc = m < a.M ? m : a.M - 1;
  return a.row_idx ? a.row_idx[mc] : mc;
}

__device__ __forceinline__ const uint16_t* lm_row_ptr(const LmK& a, int m, int r, int Meff) {
  return (m < Meff && r >= 0 && r < a.n_src) ? a.h + (size_t)r * a.hidden : nullptr;
}

// Running statistics of one lane's logits of one row over the passes: the
// exponentials use a lazy offset (raised only when a logit exceeds it by more
// than kLmLazy, so every term stays below 2^(kLmLazy*log2 e) and most passes
// need no rescale), next to the exact maximum and its lowest column.  The
// lanes' statistics meet once, at the end of the work-group's range.
constexpr float kLmLazy = 5.5f;
struct LmLane {
  float off;  // offset of the sum (-inf until a finite logit is seen)
  float s;    // sum of exp(v - off)
  float bv;   // largest logit
  int idx;    // its lowest column
};
template <int N>
__device__ __forceinline__ void lm_lane_update(LmLane& st, const float (&v)[N], const int (&col)[N]) {
  float mt = v[0];
#pragma unroll
  for (int j = 1; j < N; ++j) mt = fmaxf(mt, v[j]);
  if (mt > st.off + kLmLazy) {  // -inf + kLmLazy is -inf: the first finite logit sets the offset
    st.s *= bd_exp2((st.off - mt) * BD_LOG2E);
    st.off = mt;
  }
  const float mu = st.off == BD_NEG_INF ? 0.f : st.off;
#pragma unroll
  for (int j = 0; j < N; ++j) {
    st.s += bd_exp2((v[j] - mu) * BD_LOG2E);
    if (v[j] > st.bv) {  // columns arrive in increasing order: the first maximum is the lowest
      st.bv = v[j];
      st.idx = col[j];
    }
  }
}
// (max, lowest argmax, sum of exp(v - max)) of a row over the 16 lanes of its group
__device__ __forceinline__ BdArgStat lm_lane_row(const LmLane& st) {
  const float m = bd_row16_max(st.bv);
  const float mu = m == BD_NEG_INF ? 0.f : m;
  const float sl = st.off == BD_NEG_INF ? 0.f : st.s * bd_exp2((st.off - mu) * BD_LOG2E);
  const int il = (st.bv == m && m != BD_NEG_INF) ? st.idx : INT_MAX;
  return BdArgStat{m, bd_row16_min(il), bd_row16_sum(sl)};
}

template <int MT, int NWV>
struct LmCfg {  // the stage layout of stream_gemm.h over NWV waves
  static constexpr int NS = kNS;
  static constexpr int MTW = MT < 2 ? MT : 2;  // row tiles per wave
  static constexpr int WM = MT / MTW;          // waves along the rows
  static constexpr int WN = NWV / WM;          // waves along the columns
  static constexpr int NTP = kNTW / WN;        // column tiles per wave
  static constexpr int KSC = 2;                // 32-wide k-steps per chunk
  static constexpr int KC = 64;                // k per chunk
  static constexpr int FR = 2 * (kNTW + MT);   // DMA instructions per stage (1 KiB each)
  static constexpr int LW = (FR + NWV - 1) / NWV, LW_LO = FR / NWV;  // per wave (waves >= FR % NWV: LW_LO)
  static constexpr int WI = 2 * kNTW / NWV;    // W instructions per wave
  static constexpr int STAGE_U4 = FR * 64;
  static_assert(kNTW % WN == 0 && (2 * kNTW) % NWV == 0, "split");
  static_assert(NS >= 2 && NS <= 5, "stages");
};

// Streaming LM head for up to 64 rows, persistent over the vocabulary.
// Work-group w of nwg owns the 16-column tiles [w*T/nwg, (w+1)*T/nwg),
// T = ceil(V/16), and walks them in P passes of at most kNTW tiles (equal
// splits of its range), so every work-group streams the same share of W and
// all of them finish together.  The 64-wide K chunks of all its passes form
// one stream of pipeline stages (stage s: pass s / nch, chunk s % nch): the
// first stages of a pass are in flight while the previous pass finishes its
// MFMAs and folds its logits into each lane's running statistics (LmLane: no
// cross-lane work and no barrier between passes); the lanes and waves of a
// row meet once at the end, and one (max, argmax, sum) per row is stored.
// Stage layout as in stream_gemm.h: kNTW W tiles then MT X tiles, each 16
// rows x 64 k (2 KiB, two whole-line DMA instructions, XOR-swizzled).  A pass
// with fewer than kNTW tiles fills its unused W slots from row 0 of h (an L2
// hit), so every stage issues the same loads per wave and the waits count
// exactly; the epilogue ignores the logits of those slots.
template <int MT, int NWV>
__global__ __launch_bounds__(64 * NWV, NWV == 4 ? 2 : 1) void lm_stream_kernel(LmK a, int P) {
  using C = LmCfg<MT, NWV>;
  __shared__ uint4 sbuf[C::NS * C::STAGE_U4];
  __shared__ BdArgStat red[C::WN * MT * 16];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, l16 = lane & 15;
  const int wm = wave % C::WM, wn = wave / C::WM;
  const int m0 = blockIdx.y * MT * 16;
  const int Meff = lm_rows(a.m_dev, a.M);
  if (m0 >= Meff) return;  // the whole row block is past the row count
  const int K = a.hidden, nch = K / C::KC, nst = P * nch;
  const int T = (a.V + 15) >> 4;
  const int t0 = (int)((long long)blockIdx.x * T / gridDim.x);
  const int nt = (int)((long long)(blockIdx.x + 1) * T / gridDim.x) - t0;
  auto pass_begin = [&](int p) { return t0 + p * nt / P; };  // first tile of pass p

  // DMA instruction f = wave + 4i loads rows 8*(f%2)..+7 of stage tile f/2:
  // tiles 0..kNTW-1 are W (per pass), the next MT are X (fixed).
  const int lrow = lane >> 3, lkb = (lane & 7) ^ lrow;
  int xm[C::LW], xi[C::LW];
#pragma unroll
  for (int i = 0; i < C::LW; ++i) {  // row indices first: their loads are in flight together
    const int f = wave + NWV * i, t = f >> 1;
    xm[i] = m0 + (t - kNTW) * 16 + 8 * (f & 1) + lrow;
    xi[i] = (f < C::FR && t >= kNTW) ? lm_row_index(a, xm[i]) : 0;
  }
  const uint16_t* const hdummy = a.h + 8 * lkb;
  const uint16_t* src[C::LW];
#pragma unroll
  for (int i = 0; i < C::LW; ++i) {
    const uint16_t* p = lm_row_ptr(a, xm[i], xi[i], Meff);
    src[i] = p ? p + 8 * lkb : hdummy;  // X rows; W rows are set per pass
  }
  auto set_pass = [&](int p) {  // W sources of pass p
    const int b = pass_begin(p), n = pass_begin(p + 1) - b;
#pragma unroll
    for (int i = 0; i < C::LW; ++i) {
      const int f = wave + NWV * i, t = f >> 1;
      if (f < C::FR && t < kNTW) {
        const int col = (b + t) * 16 + 8 * (f & 1) + lrow;
        src[i] = t >= n ? hdummy : a.w + (size_t)(col < a.V ? col : 0) * K + 8 * lkb;
      }
    }
  };
  int ip = 0, ich = 0, iss = 0;  // issue cursor: pass, chunk, stages issued
  set_pass(0);
  auto issue_next = [&]() {
    uint4* st = sbuf + (iss % C::NS) * C::STAGE_U4;
    // instructions i < WI load W tiles (for every wave), the rest X rows
#pragma unroll
    for (int i = 0; i < C::WI; ++i)
      __builtin_amdgcn_global_load_lds((bd_stream::glb_void_t*)(src[i] + (size_t)ich * C::KC),
                                       (bd_stream::lds_void_t*)(st + (wave + NWV * i) * 64), 16, 0, BD_LM_AUX);
#pragma unroll
    for (int i = C::WI; i < C::LW; ++i)
      if (C::FR % NWV == 0 || wave + NWV * i < C::FR)
        __builtin_amdgcn_global_load_lds((bd_stream::glb_void_t*)(src[i] + (size_t)ich * C::KC),
                                         (bd_stream::lds_void_t*)(st + (wave + NWV * i) * 64), 16, 0, 0);
    ++iss;
    if (++ich == nch) {
      ich = 0;
      if (++ip < P) set_pass(ip);
    }
  };
  const bool more = wave < C::FR % NWV;  // this wave issues LW (else LW_LO) loads per stage
  const int fo0 = bd_stream::frag_offset(lane, 0) / 16, fo1 = bd_stream::frag_offset(lane, 1) / 16;

  bd_f32x4 acc[C::MTW][C::NTP];
#pragma unroll
  for (int i = 0; i < C::MTW; ++i)
#pragma unroll
    for (int j = 0; j < C::NTP; ++j) acc[i][j] = bd_f32x4{0.f, 0.f, 0.f, 0.f};
  LmLane ls[C::MTW][4];  // this lane's columns of rows m0 + (wm*MTW + i)*16 + 4g + r, over the passes
#pragma unroll
  for (int i = 0; i < C::MTW; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) ls[i][r] = LmLane{BD_NEG_INF, 0.f, BD_NEG_INF, INT_MAX};

  // the skip test's bits load with the row indices (at most 64 sequences)
  uint64_t skip_word = 0;
  if (a.skip_bits != nullptr && lane < a.skip_B) skip_word = a.skip_bits[lane];
  // the row-index loads (and every other global load so far) complete before
  // the pipeline starts, so no register wait is left for the loop
  __builtin_amdgcn_s_waitcnt(bd_stream::vmcnt_imm(0));
  if (a.skip_bits != nullptr) {
    const bool go = __ballot((skip_word & a.skip_mask) != 0) != 0;
    if (blockIdx.x == 0 && blockIdx.y == 0 && tid == 0) *a.ran = go ? 1 : 0;  // for the merge
    if (!go) return;  // no masked position left in the window: nothing to predict
  }
#pragma unroll
  for (int c = 0; c < C::NS - 1; ++c)
    if (c < nst) issue_next();

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
    // fragment reads: asm that waits inside the block (otherwise the compiler,
    // unable to tell which LDS bytes the DMA in flight writes, puts a
    // vmcnt(0) in front of them and drains the pipeline every stage)
    const uint32_t sb = bd_stream::lds_addr(sbuf + (s % C::NS) * C::STAGE_U4);
#pragma unroll
    for (int ks = 0; ks < C::KSC; ++ks) {
      const uint32_t fo = (ks == 0 ? fo0 : fo1) * 16;
      uint4 xa[C::MTW], wb[C::NTP];
      bd_stream::lds_frags_kstep<C::MTW, C::NTP>(sb + (kNTW + wm * C::MTW) * 2048 + fo,
                                                 sb + wn * C::NTP * 2048 + fo, xa, wb);
#pragma unroll
      for (int i = 0; i < C::MTW; ++i)
#pragma unroll
        for (int j = 0; j < C::NTP; ++j) acc[i][j] = bd_mfma16(xa[i], wb[j], acc[i][j]);
    }
    if (++cch < nch) continue;

    // ---- end of pass cp: rows m0 + (wm*MTW + i)*16 + 4g + r, columns
    // (b + wn*NTP + j)*16 + l16; slots past the pass and columns past V are out
    const int b = pass_begin(cp), n = pass_begin(cp + 1) - b;
    int col[C::NTP];
    bool cok[C::NTP];
#pragma unroll
    for (int j = 0; j < C::NTP; ++j) {
      col[j] = (b + wn * C::NTP + j) * 16 + l16;
      cok[j] = wn * C::NTP + j < n && col[j] < a.V;
    }
    if (a.logits != nullptr) {  // debug dump of the raw logits (tests only)
#pragma unroll
      for (int i = 0; i < C::MTW; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = m0 + (wm * C::MTW + i) * 16 + 4 * g + r;
#pragma unroll
          for (int j = 0; j < C::NTP; ++j)
            if (m < Meff && cok[j]) a.logits[(size_t)m * a.V + col[j]] = acc[i][j][r];
        }
    }
    // no cross-lane work here: each lane folds its logits into its own
    // running statistics, so the next pass's stages keep streaming
#pragma unroll
    for (int i = 0; i < C::MTW; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v[C::NTP];
#pragma unroll
        for (int j = 0; j < C::NTP; ++j) v[j] = cok[j] ? acc[i][j][r] : BD_NEG_INF;
        lm_lane_update(ls[i][r], v, col);
      }
    }
#pragma unroll
    for (int i = 0; i < C::MTW; ++i)
#pragma unroll
      for (int j = 0; j < C::NTP; ++j) acc[i][j] = bd_f32x4{0.f, 0.f, 0.f, 0.f};
    cch = 0;
    ++cp;
  }
  // the rows' statistics: over the 16 lanes of each row group, then over the
  // WN waves that hold the row's columns (in wave order)
#pragma unroll
  for (int i = 0; i < C::MTW; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const BdArgStat rs = lm_lane_row(ls[i][r]);
      if (l16 == 0) red[wn * (MT * 16) + (wm * C::MTW + i) * 16 + 4 * g + r] = rs;
    }
  __syncthreads();
  BdArgStat run{BD_NEG_INF, INT_MAX, 0.f};
  if (tid < MT * 16) {
#pragma unroll
    for (int w = 0; w < C::WN; ++w) run = bd_stat_combine(run, red[w * (MT * 16) + tid]);
  }
  if (tid < MT * 16 && m0 + tid < Meff) {
    const size_t pi = (size_t)blockIdx.x * a.M + m0 + tid;  // [work-group][row]: whole cache lines
    a.pmax[pi] = run.m;
    a.pidx[pi] = run.i;
    a.psum[pi] = run.s;
  }
}

// ---------------------------------------------------------------------------
// Large-M bf16 LM head: each work-group computes a 256-row x (CT*16)-column
// tile of the logits with 8 waves and reduces it to per-row partials.
//   CT = 16 (more than 256 rows, MFMA-bound): 2 x 4 waves of 128 x 64, two
//            64 KiB stages;
//   CT = 8  (up to 256 rows, HBM-bound): 4 x 2 waves of 64 x 64, three
//            48 KiB stages (two in flight) and twice the work-groups, so the
//            weight stream has more bytes in flight and a shorter tail.
// K is walked in 64-wide chunks filled by whole-line DMA (the tile layout of
// stream_gemm.h: a 16-row x 64-k tile is 2 KiB, two instructions of 8 rows x
// 128 B, XOR-swizzled k-blocks).  Work order: the row blocks of one column
// block are consecutive on one XCD, so a W column block is fetched from HBM
// once and re-read from that XCD's L2.
constexpr int kBigRows = 256, kBigThreads = 512;
#ifndef BD_LM_NARROW_MAX_ROWS
#define BD_LM_NARROW_MAX_ROWS 256
#endif
constexpr int kNarrowMaxRows = BD_LM_NARROW_MAX_ROWS;  // up to this many rows: 256 x 128 tiles

template <int CT>
struct Big {
  static constexpr int WR = CT == 16 ? 2 : 4;       // waves along the rows
  static constexpr int WC = 8 / WR;                 // waves along the columns
  static constexpr int MW = kBigRows / 16 / WR;     // row tiles per wave
  static constexpr int NWT = CT / WC;               // column tiles per wave
  static constexpr int NS = CT == 16 ? 2 : 3;       // stages
  static constexpr int TILES = kBigRows / 16 + CT;  // 16-row tiles per stage
  static constexpr int FR = 2 * TILES;              // DMA instructions per stage
  static constexpr int LW = FR / 8;                 // per wave
  static constexpr int STAGE_U4 = FR * 64;
  static_assert(MW % 4 == 0 && NWT == 4 && FR % 8 == 0, "wave tiling");
};

template <int CT>
__global__ __launch_bounds__(kBigThreads, 1) void lm_big_kernel(LmK a, int rb_count, int cb_count) {
  using P = Big<CT>;
  __shared__ uint4 sbuf[P::NS * P::STAGE_U4];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, l16 = lane & 15;
  const int wr = wave % P::WR, wc = wave / P::WR;
  // XCD-aware order: work-group w runs on XCD w % 8; the (w / 8)-th work-group
  // of an XCD takes row block q % rb_count of column block
  // xcd * per_xcd + q / rb_count, so the row blocks of a column block share
  // one L2 (W is fetched from HBM once).
  const int xcd = blockIdx.x & 7, q = blockIdx.x >> 3;
  const int per_xcd = (cb_count + 7) >> 3;
  const int rb = q % rb_count, cb = xcd * per_xcd + q / rb_count;
  if (cb >= cb_count) return;
  const int m0 = rb * kBigRows, n0 = cb * CT * 16;
  const int nch = a.hidden / 64;
  const int Meff = lm_rows(a.m_dev, a.M);
  if (m0 >= Meff) return;  // the whole row block is past the row count

  // DMA sources: instruction f covers rows 8*(f%2)..+7 of stage tile f/2;
  // tiles 0..15 are X row tiles, the next CT are W column tiles.
  const int lrow = lane >> 3, lkb = (lane & 7) ^ lrow;
  int xi[P::LW];  // row indices first: their loads are in flight together
#pragma unroll
  for (int i = 0; i < P::LW; ++i) {
    const int f = wave + 8 * i, t = f >> 1, r = 8 * (f & 1) + lrow;
    xi[i] = t < kBigRows / 16 ? lm_row_index(a, m0 + t * 16 + r) : 0;
  }
  const uint16_t* src[P::LW];
#pragma unroll
  for (int i = 0; i < P::LW; ++i) {
    const int f = wave + 8 * i, t = f >> 1, r = 8 * (f & 1) + lrow;
    if (t < kBigRows / 16) {
      const uint16_t* p = lm_row_ptr(a, m0 + t * 16 + r, xi[i], Meff);
      src[i] = (p ? p : a.h) + 8 * lkb;
    } else {
      const int col = n0 + (t - kBigRows / 16) * 16 + r;
      src[i] = a.w + (size_t)(col < a.V ? col : 0) * a.hidden + 8 * lkb;
    }
  }
  // X tiles past the row count are not loaded (their MFMAs are skipped);
  // the number of loads this wave issues per stage is then a wave-uniform
  // value and the pipeline waits select the matching immediate.
  const int live_tiles = (Meff - m0 + 15) / 16;
  bool ld[P::LW];
  int issued = 0;
#pragma unroll
  for (int i = 0; i < P::LW; ++i) {
    const int t = (wave + 8 * i) >> 1;
    ld[i] = t >= kBigRows / 16 || t < live_tiles;
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
  static_assert(P::LW <= 8, "wait immediates");

  bd_f32x4 acc[P::MW][P::NWT];
#pragma unroll
  for (int i = 0; i < P::MW; ++i)
#pragma unroll
    for (int j = 0; j < P::NWT; ++j) acc[i][j] = bd_f32x4{0.f, 0.f, 0.f, 0.f};
  const uint32_t sbase = bd_stream::lds_addr(sbuf);
  const uint32_t fo[2] = {(uint32_t)bd_stream::frag_offset(lane, 0), (uint32_t)bd_stream::frag_offset(lane, 1)};
  // Row tiles are dealt to the row waves in turn (tile i of this wave is row
  // tile i*WR + wr), so that the waves sharing a SIMD get equal shares when
  // rows past the count are skipped.  First X / W tile as a byte offset.
  const uint32_t xt0 = wr * 2048, wt0 = (kBigRows / 16 + wc * P::NWT) * 2048;
  constexpr int XS = P::WR * 2048;  // byte stride between this wave's X tiles
  // this wave's 16-row tiles that hold rows below the count (MFMAs of the
  // others are skipped: the candidate rows are listed first)
  const int live = min(P::MW, max(0, (live_tiles - wr + P::WR - 1) / P::WR));

#pragma unroll
  for (int c = 0; c < P::NS - 1; ++c)
    if (c < nch) issue(c);
  for (int ch = 0; ch < nch; ++ch) {
    // chunks issued so far: min(nch, ch + NS - 1); keep the later ones in flight
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
#pragma unroll
      for (int i0 = 4; i0 < P::MW; i0 += 4) {
        if (i0 >= live) break;
        bd_stream::lds_frags_4<XS>(st + xt0 + i0 * XS + fo[ks], xa);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (i0 + i < live)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i0 + i][j] = bd_mfma16(xa[i], wb[j], acc[i0 + i][j]);
      }
    }
  }
  __syncthreads();  // the stages become the reduction buffer

  // acc[i][j][r]: row m0 + (i*WR + wr)*16 + 4g + r, column n0 + wc*NWT*16 + 16j + l16
  if (a.logits != nullptr) {  // debug dump of the raw logits (tests only)
#pragma unroll
    for (int i = 0; i < P::MW; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + (i * P::WR + wr) * 16 + 4 * g + r;
#pragma unroll
        for (int j = 0; j < P::NWT; ++j) {
          const int col = n0 + (wc * P::NWT + j) * 16 + l16;
          if (m < Meff && col < a.V) a.logits[(size_t)m * a.V + col] = acc[i][j][r];
        }
      }
  }
  const bool ragged = n0 + CT * 16 > a.V;  // only the last column block
  int col[P::NWT];
#pragma unroll
  for (int j = 0; j < P::NWT; ++j) col[j] = n0 + (wc * P::NWT + j) * 16 + l16;
  BdArgStat* red = reinterpret_cast<BdArgStat*>(sbuf);  // [WC column waves][256 rows]
#pragma unroll
  for (int i = 0; i < P::MW; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float v[P::NWT];
#pragma unroll
      for (int j = 0; j < P::NWT; ++j) v[j] = (ragged && col[j] >= a.V) ? BD_NEG_INF : acc[i][j][r];
      const BdArgStat st = bd_row16_stat(v, col);
      if (l16 == 0) red[wc * kBigRows + (i * P::WR + wr) * 16 + 4 * g + r] = st;
    }
  }
  __syncthreads();
  if (tid < kBigRows && m0 + tid < Meff) {
    BdArgStat st = red[tid];
#pragma unroll
    for (int w = 1; w < P::WC; ++w) st = bd_stat_combine(st, red[w * kBigRows + tid]);
    const size_t pi = (size_t)(m0 + tid) * a.nvt + cb;  // [row][tile]: few, wide work-groups
    a.pmax[pi] = st.m;
    a.pidx[pi] = st.i;
    a.psum[pi] = st.s;
  }
}

struct LmF {
  const float* h;
  int n_src;
  const int32_t* row_idx;
  const float* w;
  float* logits;
  int M, hidden, V, nvt;
  float* pmax;
  int32_t* pidx;
  float* psum;
  const int32_t* m_dev;
};

__global__ __launch_bounds__(kThreads) void lm_f32_kernel(LmF a) {
  __shared__ float sh[kF32Rows][kThreads];
  __shared__ BdArgStat red[kThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = blockIdx.x * kThreads + tid;
  const int m0 = blockIdx.y * kF32Rows;
  const int Meff = lm_rows(a.m_dev, a.M);
  if (m0 >= Meff) return;
  const float* hrow[kF32Rows];
#pragma unroll
  for (int r = 0; r < kF32Rows; ++r) {
    const int m = m0 + r;
    const int src = (m < Meff) ? (a.row_idx ? a.row_idx[m] : m) : -1;
    hrow[r] = (src >= 0 && src < a.n_src) ? a.h + (size_t)src * a.hidden : nullptr;
  }
  float acc[kF32Rows];
#pragma unroll
  for (int r = 0; r < kF32Rows; ++r) acc[r] = 0.f;
  for (int k0 = 0; k0 < a.hidden; k0 += kThreads) {
    const int kn = min(kThreads, a.hidden - k0);
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kF32Rows; ++r) sh[r][tid] = (hrow[r] != nullptr && tid < kn) ? hrow[r][k0 + tid] : 0.f;
    __syncthreads();
    if (col < a.V) {
      const float* wr = a.w + (size_t)col * a.hidden + k0;
      for (int kk = 0; kk < kn; ++kk) {
        const float wv = wr[kk];
#pragma unroll
        for (int r = 0; r < kF32Rows; ++r) acc[r] += sh[r][kk] * wv;
      }
    }
  }
#pragma unroll
  for (int r = 0; r < kF32Rows; ++r) {
    const int m = m0 + r;
    if (a.logits != nullptr && m < Meff && col < a.V) a.logits[(size_t)m * a.V + col] = acc[r];
    BdArgStat st = (col < a.V) ? BdArgStat{acc[r], col, 1.f} : BdArgStat{BD_NEG_INF, INT_MAX, 0.f};
    for (int off = 1; off < 64; off <<= 1) st = bd_stat_combine(st, bd_stat_shfl_xor(st, off));
    __syncthreads();
    if (lane == 0) red[wave] = st;
    __syncthreads();
    if (tid == 0 && m < Meff) {
      BdArgStat t = red[0];
      for (int w = 1; w < kThreads / 64; ++w) t = bd_stat_combine(t, red[w]);
      const size_t pi = (size_t)blockIdx.x * a.M + m;
      a.pmax[pi] = t.m;
      a.pidx[pi] = t.i;
      a.psum[pi] = t.s;
    }
  }
}

// Fold the tiles of each row; one work-group per row.  Each thread keeps up to
// kMergePer of the row's tile statistics in registers: the row max is found
// first, then every tile's sum is scaled with one exp2 and the argmax is the
// lowest column among the tiles that reach the max.  The order of the sums
// is fixed, so the result is deterministic.
constexpr int kMergePer = 8;
constexpr int kFuseThreads = 512;  // merge fused with the unmask: 8 waves, one row each at a time
constexpr int kFusePer = 8;        // partials per lane held in registers (up to 512 per row)

__device__ __forceinline__ float block_max(float v, float* sh) {
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  v = sh[0];
  for (int w = 1; w < kThreads / 64; ++w) v = fmaxf(v, sh[w]);
  return v;
}

__global__ __launch_bounds__(kThreads) void lm_merge_kernel(const int32_t* row_idx, int n_src, int M,
                                                            int nvt, size_t ts, size_t rs, const float* pmax,
                                                            const int32_t* pidx,
                                                            const float* psum, int32_t* argmax, float* conf,
                                                            float* max_logit, float* lse, const int32_t* m_dev,
                                                            const int32_t* out_pos, int n_out) {
  __shared__ float shm[kThreads / 64];
  __shared__ float shs[kThreads / 64];
  __shared__ int shi[kThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = blockIdx.x;
  if (m >= lm_rows(m_dev, M)) return;
  const int om = out_pos ? out_pos[m] : m;  // output slot of this row
  if (out_pos != nullptr && (om < 0 || om >= n_out)) return;
  // partial (row m, tile t) is at t * ts + m * rs: [tile][row] from the
  // streaming kernels (whose work-groups then store whole cache lines),
  // [row][tile] from the 256-row kernel (whose merge rows read contiguously)
  const float* pmr = pmax + (size_t)m * rs;
  const float* psr = psum + (size_t)m * rs;
  const int32_t* pir = pidx + (size_t)m * rs;
  float mx = BD_NEG_INF, s = 0.f;
  int idx = INT_MAX;
  if (nvt <= kMergePer * kThreads) {
    float pm[kMergePer], ps[kMergePer];
    int pi[kMergePer];
#pragma unroll
    for (int u = 0; u < kMergePer; ++u) {
      const int t = tid + u * kThreads;
      const bool ok = t < nvt;
      pm[u] = ok ? pmr[t * ts] : BD_NEG_INF;
      ps[u] = ok ? psr[t * ts] : 0.f;
      pi[u] = ok ? pir[t * ts] : INT_MAX;
    }
#pragma unroll
    for (int u = 0; u < kMergePer; ++u) mx = fmaxf(mx, pm[u]);
    mx = block_max(mx, shm);
    const float mu = (mx == BD_NEG_INF) ? 0.f : mx;
#pragma unroll
    for (int u = 0; u < kMergePer; ++u) {
      s += ps[u] * bd_exp2((pm[u] - mu) * BD_LOG2E);
      if (pm[u] == mx && pm[u] != BD_NEG_INF) idx = min(idx, pi[u]);
    }
  } else {  // very large vocabularies: pairwise combines over a strided loop
    BdArgStat st{BD_NEG_INF, INT_MAX, 0.f};
    for (int t = tid; t < nvt; t += kThreads)
      st = bd_stat_combine(st, BdArgStat{pmr[t * ts], pir[t * ts], psr[t * ts]});
    mx = block_max(st.m, shm);
    const float mu = (mx == BD_NEG_INF) ? 0.f : mx;
    s = (st.m == BD_NEG_INF) ? 0.f : st.s * bd_exp2((st.m - mu) * BD_LOG2E);
    if (st.m == mx && st.m != BD_NEG_INF) idx = st.i;
  }
  for (int off = 32; off > 0; off >>= 1) {
    s += __shfl_xor(s, off);
    idx = min(idx, __shfl_xor(idx, off));
  }
  if (lane == 0) {
    shs[wave] = s;
    shi[wave] = idx;
  }
  __syncthreads();
  if (tid != 0) return;
  for (int w = 1; w < kThreads / 64; ++w) {
    s += shs[w];
    idx = min(idx, shi[w]);
  }
  const int src = row_idx ? row_idx[m] : m;
  const bool ok = src >= 0 && src < n_src && s > 0.f;
  const float nan = __builtin_nanf("");
  argmax[om] = ok ? idx : -1;
  conf[om] = ok ? 1.f / s : nan;
  if (max_logit != nullptr) max_logit[om] = ok ? mx : nan;
  if (lse != nullptr) lse[om] = ok ? mx + bd_log2(s) * BD_LN2 : nan;
}

// The fused call's skip flag: 16 bytes after the partials.
int32_t* lm_ran_flag(const BdLmPlan& p, const BdLmArgs& x) {
  return reinterpret_cast<int32_t*>(reinterpret_cast<char*>(x.pmax) + p.ws_bytes - 16);
}

// Merge fused with the threshold unmask: one work-group per sequence.  The
// sequence's win_len rows are padded to RP (a power of two) lanes, so one
// load instruction of a wave covers 64 / RP tiles x RP consecutive rows
// (short runs of whole partial rows instead of 64 scattered words; the
// partials are [tile][row]).  Lane (q, r) folds tiles q + (64 / RP) * (wave
// + 8 u) of row r in batches held in registers; lanes of one row, then the 8
// waves (through LDS), combine their (max, argmax, sum) in a fixed order.
// Wave 0 lane r then holds row r: it writes the statistics (unless the LM
// head skipped its work: no masked position in the window of any sequence)
// and the wave applies the threshold rule.
// Saves the unmask launch of the step.
__global__ __launch_bounds__(kFuseThreads) void lm_merge_unmask_kernel(const int32_t* row_idx, int n_src, int nvt,
                                                                      const float* pmax, const int32_t* pidx,
                                                                      const float* psum, int32_t* argmax, float* conf,
                                                                      float* max_logit, float* lse, int M, int RP,
                                                                      const int32_t* ran, BdLmUnmask u) {
  constexpr int NW = kFuseThreads / 64;
  __shared__ BdArgStat sh[NW][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.x;
  // this sequence's bits before the unmask below (only this work-group writes
  // them) and whether the LM head computed (it skips a window with no masked
  // position in any sequence: then the statistics are left as they were)
  const uint64_t bits0 = u.mask_bits[b];
  const bool computed = ran == nullptr || *ran != 0;
  const int r = lane & (RP - 1);
  const int q = lane / RP;
  const int tpi = 64 / RP;                // tiles per wave instruction
  const bool live = r < u.win_len;
  const int m = b * u.win_len + (live ? r : 0);
  BdArgStat st{BD_NEG_INF, INT_MAX, 0.f};
  for (int t0 = q + tpi * wave; t0 < nvt; t0 += tpi * NW * kFusePer) {
    float pm[kFusePer], ps[kFusePer];
    int pi[kFusePer];
#pragma unroll
    for (int k = 0; k < kFusePer; ++k) {
      const int t = t0 + tpi * NW * k;
      const bool ok = live && t < nvt;
      const size_t at = (size_t)t * M + m;
      pm[k] = ok ? pmax[at] : BD_NEG_INF;
      ps[k] = ok ? psum[at] : 0.f;
      pi[k] = ok ? pidx[at] : INT_MAX;
    }
    float bm = pm[0];
#pragma unroll
    for (int k = 1; k < kFusePer; ++k) bm = fmaxf(bm, pm[k]);
    const float mu = (bm == BD_NEG_INF) ? 0.f : bm;
    float bs = 0.f;
    int bi = INT_MAX;
#pragma unroll
    for (int k = 0; k < kFusePer; ++k) {
      bs += ps[k] * bd_exp2((pm[k] - mu) * BD_LOG2E);
      if (pm[k] == bm && pm[k] != BD_NEG_INF) bi = min(bi, pi[k]);
    }
    st = bd_stat_combine(st, BdArgStat{bm, bi, bs});
  }
  for (int off = RP; off < 64; off <<= 1) st = bd_stat_combine(st, bd_stat_shfl_xor(st, off));
  if (q == 0) sh[wave][r] = st;
  __syncthreads();
  __shared__ uint64_t sh_pick;  // entries unmasked here, their tokens and their list (next rows)
  __shared__ int32_t sh_tok[64], sh_pos[64];
  if (wave == 0) {
  if (q == 0)
    for (int w = 1; w < NW; ++w) st = bd_stat_combine(st, sh[w][r]);
  float c = BD_NEG_INF;
  int32_t am = -1;
  if (live && q == 0 && computed) {
    const int src = row_idx ? row_idx[m] : m;
    const bool ok = src >= 0 && src < n_src && st.s > 0.f;
    const float nan = __builtin_nanf("");
    c = ok ? 1.f / st.s : nan;
    am = ok ? st.i : -1;
    argmax[m] = am;
    conf[m] = c;
    if (max_logit != nullptr) max_logit[m] = ok ? st.m : nan;
    if (lse != nullptr) lse[m] = ok ? st.m + bd_log2(st.s) * BD_LN2 : nan;
  }
  // lane r (< RP, so q == 0) holds window entry r
  const float thr = u.threshold_dev != nullptr ? u.threshold_dev[b] : u.threshold;
  const uint64_t pick = bd_unmask_wave(lane, b, u.D, u.win_lo, u.win_len, bits0, lane < RP ? c : BD_NEG_INF,
                                       lane < RP ? am : -1, thr, u.tokens, u.mask_bits, u.n_unmasked,
                                       u.unmasked_pos, u.bits_out);
  if (u.x != nullptr) {
    if (lane == 0) sh_pick = pick;
    if (lane < RP) sh_tok[lane] = am;
    if ((pick >> lane) & 1ull) sh_pos[__popcll(pick & ((1ull << lane) - 1ull))] = lane;
  }
  }
  if (u.x == nullptr) return;
  // Next step's input rows: the row of every position decoded here becomes
  // its token's embedding (+ the plant), as bd_embed_rows would write it; the
  // rows of positions still masked keep the [MASK] embedding they hold.
  __syncthreads();
  const uint64_t pk = sh_pick;
  const int np = __popcll(pk);
  const int per = u.f32 ? 4 : 8;  // elements per 16-byte vector
  const int nv = u.hidden / per;
  for (int t = tid; t < np * nv; t += kFuseThreads) {
    const int k = t / nv, e = (t - k * nv) * per;
    const int ent = sh_pos[k], tok = sh_tok[ent];
    const bool ok = tok >= 0 && tok < u.V;
    const size_t row = (size_t)b * u.D + u.win_lo + ent;
    const size_t eoff = (size_t)(ok ? tok : 0) * u.hidden + e, roff = row * u.hidden + e;
    if (u.f32) {
      float4 f = *(reinterpret_cast<const float4*>(static_cast<const float*>(u.emb) + eoff));
      if (u.plant) {
        const float4 p = *(reinterpret_cast<const float4*>(static_cast<const float*>(u.plant) + roff));
        f.x += p.x; f.y += p.y; f.z += p.z; f.w += p.w;
      }
      if (!ok) f = make_float4(__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""));
      *reinterpret_cast<float4*>(static_cast<float*>(u.x) + roff) = f;
    } else {
      const uint4 ev = *(reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(u.emb) + eoff));
      const uint4 pv = u.plant ? *(reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(u.plant) + roff))
                               : make_uint4(0, 0, 0, 0);
      const uint32_t ew[4] = {ev.x, ev.y, ev.z, ev.w}, pw[4] = {pv.x, pv.y, pv.z, pv.w};
      uint32_t ow[4];
#pragma unroll
      for (int h = 0; h < 4; ++h)
        ow[h] = !ok ? 0x7fc07fc0u
                    : (u.plant ? bd_pack_bf2(bd_bf2f(ew[h] & 0xffffu) + bd_bf2f(pw[h] & 0xffffu),
                                             bd_bf2f(ew[h] >> 16) + bd_bf2f(pw[h] >> 16))
                               : ew[h]);
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(u.x) + roff) = make_uint4(ow[0], ow[1], ow[2], ow[3]);
    }
  }
}

}  // namespace

BdLmPlan bd_lm_plan(bd_dtype dt, int M, int hidden, int V) {
  BdLmPlan p{};
  if (dt == BD_F32) {
    p.cols_per_wg = kThreads;
    p.rows_per_wg = kF32Rows;
  } else if (M > 64) {
    p.cols_per_wg = (M > kNarrowMaxRows ? 16 : 8) * 16;
    p.rows_per_wg = kBigRows;
  } else {  // streaming kernel: nvt work-groups, each a range of 16-column tiles in `passes` passes
    const int mt = (M + 15) / 16;
    p.rows_per_wg = 16 * (mt <= 1 ? 1 : (mt == 2 ? 2 : 4));
    const int T = (V + 15) / 16;
    const int wgs = hidden >= 2048 ? kStreamWGs : kStreamWGsNarrow;
    p.nvt = T < wgs ? T : wgs;
    const int per = (T + p.nvt - 1) / p.nvt;  // tiles of the largest range
    p.passes = (per + kNTW - 1) / kNTW;
    p.cols_per_wg = per * 16;
  }
  if (dt == BD_F32 || M > 64) p.nvt = (V + p.cols_per_wg - 1) / p.cols_per_wg;
  p.nmb = (M + p.rows_per_wg - 1) / p.rows_per_wg;
  p.ws_bytes = (size_t)M * p.nvt * (2 * sizeof(float) + sizeof(int32_t));
  p.ws_bytes = (p.ws_bytes + 15) / 16 * 16 + 16;  // then the skip flag of the fused call
  (void)hidden;
  return p;
}

hipError_t bd_lm_launch(bd_dtype dt, const BdLmPlan& p, const BdLmArgs& x, hipStream_t s, const BdLmUnmask* um) {
  const dim3 grid(p.nvt, p.nmb);
  if (dt == BD_F32) {
    LmF a{static_cast<const float*>(x.h), x.n_src, x.row_idx, static_cast<const float*>(x.w), x.logits,
          x.M, x.hidden, x.V, p.nvt, x.pmax, x.pidx, x.psum, x.m_dev};
    hipLaunchKernelGGL(lm_f32_kernel, grid, dim3(kThreads), 0, s, a);
  } else {
    LmK a{static_cast<const uint16_t*>(x.h), x.n_src, x.row_idx, static_cast<const uint16_t*>(x.w), x.logits,
          x.M, x.hidden, x.V, p.nvt, x.pmax, x.pidx, x.psum, x.m_dev, nullptr, 0, 0, nullptr};
    if (um != nullptr && p.rows_per_wg != kBigRows) {  // the fused call: skip when the window has no candidate
      a.skip_bits = um->mask_bits;
      a.skip_mask = (um->win_len >= 64 ? ~0ull : ((1ull << um->win_len) - 1ull)) << um->win_lo;
      a.skip_B = um->B;
      a.ran = lm_ran_flag(p, x);
    }
    switch (p.rows_per_wg / 16) {
      case kBigRows / 16: {
        const int cb8 = (p.nvt + 7) / 8 * 8;  // column blocks rounded up to whole XCD rounds
        if (p.cols_per_wg == 256)
          hipLaunchKernelGGL(lm_big_kernel<16>, dim3(cb8 * p.nmb), dim3(kBigThreads), 0, s, a, p.nmb, p.nvt);
        else
          hipLaunchKernelGGL(lm_big_kernel<8>, dim3(cb8 * p.nmb), dim3(kBigThreads), 0, s, a, p.nmb, p.nvt);
        break;
      }
      case 1: hipLaunchKernelGGL((lm_stream_kernel<1, kLmWaves>), grid, dim3(64 * kLmWaves), 0, s, a, p.passes); break;
      case 2: hipLaunchKernelGGL((lm_stream_kernel<2, kLmWaves>), grid, dim3(64 * kLmWaves), 0, s, a, p.passes); break;
      default: hipLaunchKernelGGL((lm_stream_kernel<4, kLmWaves>), grid, dim3(64 * kLmWaves), 0, s, a, p.passes); break;
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const bool row_major = dt != BD_F32 && p.rows_per_wg == kBigRows;  // partial layout, see the merge
  if (um != nullptr) {  // [tile][row] partials: the streaming and fp32 kernels (at most 64 rows)
    if (row_major || x.M != um->B * um->win_len) return hipErrorInvalidValue;
    int rp = 1;
    while (rp < um->win_len) rp <<= 1;
    hipLaunchKernelGGL(lm_merge_unmask_kernel, dim3(um->B), dim3(kFuseThreads), 0, s, x.row_idx, x.n_src, p.nvt,
                       x.pmax, x.pidx, x.psum, x.argmax, x.conf, x.max_logit, x.lse, x.M, rp,
                       dt == BD_F32 ? nullptr : lm_ran_flag(p, x), *um);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(lm_merge_kernel, dim3(x.M), dim3(kThreads), 0, s, x.row_idx, x.n_src, x.M, p.nvt,
                     row_major ? (size_t)1 : (size_t)x.M, row_major ? (size_t)p.nvt : (size_t)1, x.pmax, x.pidx, x.psum, x.argmax, x.conf, x.max_logit, x.lse, x.m_dev, x.out_pos,
                     x.n_out);
  return hipGetLastError();
}
