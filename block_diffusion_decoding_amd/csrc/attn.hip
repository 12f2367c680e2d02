// Hybrid-mask grouped-query attention of one block-diffusion refinement step.
//
// Method: "Fast-dLLM v2: Efficient Block-Diffusion LLM" notes, Framework and
// Key design 2 -- attention is bidirectional inside a block and causal across
// blocks, and the queries of the current block see every committed position
// plus the whole current block (masked positions included); Key design 3 --
// committed blocks are read from a block-level KV cache and, in a DualCache
// step, the in-block K/V outside the active sub-block come from a snapshot.
//
// bf16 path (MFMA): one work-group handles (sequence b, KV head, key chunk,
// query-tile group).  The G query heads that share a KV head and the n_q fresh
// block rows form R = n_q * G query rows; this is what turns the grouped-query
// attention into a real contraction for v_mfma_f32_16x16x32_bf16.  A
// work-group has 8 waves and up to 16 query tiles, so the key/value bytes of a
// chunk are read from HBM once; its 8-stage LDS ring (128 KiB) holds it to one
// work-group per CU, and the key chunks are sized for one work-group per CU.
// K and V tiles of KT keys stream into the ring by asynchronous global->LDS
// loads (both land XOR-swizzled; V is read transposed by ds_read_b64_tr_b16,
// issued while the score MFMAs run); the scores are computed transposed (S^T = K Q^T) so
// that the probabilities land in the B operand layout of the P.V product
// without any data movement; the softmax is an online (running max) softmax
// in base 2.  Key chunks of one (sequence, KV head) are merged by a second
// kernel when a sequence needs more than one.
//
// fp32 path: a plain VALU kernel (one work-group per query row and head),
// used for the tiny fp32 workload.
#include <climits>

#include "bd_device.h"
#include "bd_launch.h"

namespace {

constexpr int kThreads = 256;  // merge and fp32 kernels
// Tuning constants; the defaults were chosen by measurement on MI355X and can
// be overridden at build time (-DBD_ATTN_KT=...).
#ifndef BD_ATTN_KT
#define BD_ATTN_KT 32
#endif
#ifndef BD_ATTN_NS
#define BD_ATTN_NS 8
#endif
#ifndef BD_ATTN_WAVES
#define BD_ATTN_WAVES 8
#endif
#ifndef BD_ATTN_TARGET_WGS
#define BD_ATTN_TARGET_WGS 256
#endif
#ifndef BD_ATTN_MIN_CHUNK
#define BD_ATTN_MIN_CHUNK 128
#endif
// committed K/V of a call larger than this stream through with the
// non-temporal hint (they cannot stay cached until the next step anyway)
#ifndef BD_ATTN_NT_MIN_BYTES
#define BD_ATTN_NT_MIN_BYTES (256ll << 20)
#endif
#ifndef BD_ATTN_QPW_MAX
#define BD_ATTN_QPW_MAX 2
#endif
constexpr int kKT = BD_ATTN_KT;                 // keys per LDS tile (bf16 path)
constexpr int kNS = BD_ATTN_NS;                 // pipeline stages (bf16 path)
constexpr int kWaves = BD_ATTN_WAVES;           // waves per work-group (bf16 path)
constexpr int kAttnThreads = 64 * kWaves;
constexpr int kXcd = 8;                         // work-groups are dispatched round-robin over 8 XCDs
constexpr int kMinChunk = BD_ATTN_MIN_CHUNK;    // keys per work item, lower bound
constexpr int kTargetWGs = BD_ATTN_TARGET_WGS;  // one work-group per CU: the stage ring fills the LDS
// Calls whose committed K/V are at most this large (they sit in the
// last-level cache between steps, so their loads return sooner) run a
// shorter stage ring, two work-groups per CU and twice the work-groups.
#ifndef BD_ATTN_LIGHT_MAX_BYTES
#define BD_ATTN_LIGHT_MAX_BYTES (96ll << 20)
#endif
#ifndef BD_ATTN_LIGHT_NS
#define BD_ATTN_LIGHT_NS 4
#endif
constexpr int kLightNS = BD_ATTN_LIGHT_NS;
constexpr int kQpwMax = BD_ATTN_QPW_MAX;        // query tiles per wave, at most (1, 2 or 4)
constexpr float kLazyMax = 8.f;                 // running-max slack (log2 units), see the softmax

struct AttnK {
  const uint16_t* q;
  const uint16_t* kc;
  const uint16_t* vc;
  const int32_t* kv_len;
  const uint16_t* kb;
  const uint16_t* vb;
  uint16_t* o;
  float* lse;
  float* part_o;
  float* part_ml;
  int B, Hq, Hkv, G, D, n_q, q_off, cap, n_blk;
  int epc;  // entries (b) per cache slab: entry b reads cache slab b / epc
  int R, QT, nqg, chunk, nchunks, n_units;
  float scale_log2;
  const uint64_t* g_bits;  // guard (bd_guard): nothing is done when no g_bits[b],
  uint64_t g_mask;         // b < g_n, has a bit of g_mask set
  int g_n;
};

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// s_waitcnt immediate (gfx9 encoding) waiting for vmcnt <= n only.
__host__ __device__ constexpr int vm_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | (((n >> 4) & 3) << 14); }

typedef short bd_s16x4 __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16: inside each group of 16 lanes, lane j receives element
// j % 4 of the 8-byte pieces addressed by lanes j/4, j/4 + 4, j/4 + 8 and
// j/4 + 12.  With lanes 4t..4t+3 of a group pointing at four consecutive
// 8-byte pieces of key row k_t, lane j gets V[k_0..k_3][d0 + j]: four keys of
// one head-dim column, i.e. a transposed-V MFMA fragment, straight from the
// row-major tile.
__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t* p) {
  const bd_s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) bd_s16x4*)p);
  return make_uint2((uint32_t)(uint16_t)r[0] | ((uint32_t)(uint16_t)r[1] << 16),
                    (uint32_t)(uint16_t)r[2] | ((uint32_t)(uint16_t)r[3] << 16));
}

// Fragment loads of one 32-key tile at head dim 128, as inline asm that waits
// for its own results before the block ends.  The compiler cannot tell these
// LDS reads from the stages still being filled by global_load_lds and would
// otherwise put an s_waitcnt vmcnt(0) in front of them, draining the load
// pipeline; the stage read here is complete (explicit vmcnt wait + barrier).
typedef unsigned int bd_u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int bd_u32x2 __attribute__((ext_vector_type(2)));

// kf[kt][ks] = K fragment of 16-key tile kt, head-dim step ks; a[ks] is the
// LDS byte address of (kt = 0, ks); kt = 1 is 4096 bytes further.
__device__ __forceinline__ void lds_kfrags_128x32(const uint32_t (&a)[4], uint4 (&kf)[2][4]) {
  bd_u32x4 r[8];
  asm volatile(
      "ds_read_b128 %0, %8\n\t"
      "ds_read_b128 %1, %9\n\t"
      "ds_read_b128 %2, %10\n\t"
      "ds_read_b128 %3, %11\n\t"
      "ds_read_b128 %4, %8 offset:4096\n\t"
      "ds_read_b128 %5, %9 offset:4096\n\t"
      "ds_read_b128 %6, %10 offset:4096\n\t"
      "ds_read_b128 %7, %11 offset:4096\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
      : "memory");
#pragma unroll
  for (int i = 0; i < 8; ++i) kf[i / 4][i % 4] = make_uint4(r[i][0], r[i][1], r[i][2], r[i][3]);
}

// vf[dt] = transposed V fragment of head-dim tile dt (keys 4g..4g+3 from the
// read at a[dt], keys 16+4g.. from 4096 bytes further).
__device__ __forceinline__ void lds_vfrags_128x32(const uint32_t (&a)[8], uint4 (&vf)[8]) {
  bd_u32x2 r[16];
  asm volatile(
      "ds_read_b64_tr_b16 %0, %16\n\t"
      "ds_read_b64_tr_b16 %1, %16 offset:4096\n\t"
      "ds_read_b64_tr_b16 %2, %17\n\t"
      "ds_read_b64_tr_b16 %3, %17 offset:4096\n\t"
      "ds_read_b64_tr_b16 %4, %18\n\t"
      "ds_read_b64_tr_b16 %5, %18 offset:4096\n\t"
      "ds_read_b64_tr_b16 %6, %19\n\t"
      "ds_read_b64_tr_b16 %7, %19 offset:4096\n\t"
      "ds_read_b64_tr_b16 %8, %20\n\t"
      "ds_read_b64_tr_b16 %9, %20 offset:4096\n\t"
      "ds_read_b64_tr_b16 %10, %21\n\t"
      "ds_read_b64_tr_b16 %11, %21 offset:4096\n\t"
      "ds_read_b64_tr_b16 %12, %22\n\t"
      "ds_read_b64_tr_b16 %13, %22 offset:4096\n\t"
      "ds_read_b64_tr_b16 %14, %23\n\t"
      "ds_read_b64_tr_b16 %15, %23 offset:4096\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7]),
        "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11]), "=&v"(r[12]), "=&v"(r[13]), "=&v"(r[14]),
        "=&v"(r[15])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
      : "memory");
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) vf[dt] = make_uint4(r[2 * dt][0], r[2 * dt][1], r[2 * dt + 1][0], r[2 * dt + 1][1]);
}

// Two floats -> packed bf16 pair (round to nearest even; v_cvt_pk_bf16_f32).
typedef __bf16 bd_bf16x2 __attribute__((ext_vector_type(2)));
typedef float bd_f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((bd_f32x2){lo, hi}, bd_bf16x2));
}

// max(a, b, c) in one instruction (fmaxf chains add NaN-quieting copies of
// MFMA results)
__device__ __forceinline__ float vmax3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// Barrier without __syncthreads()' fences (they would wait for every
// outstanding global load and drain the pipeline); the kernel waits for what
// it needs with explicit s_waitcnt first.
__device__ __forceinline__ void pipe_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Wait until at most `later` stages of LW loads per wave are outstanding
// (s_waitcnt takes an immediate, hence the switch).
template <int LW, int NS>
__device__ __forceinline__ void wait_stages(int later) {
  switch (later) {
    case 1: if constexpr (NS > 2) __builtin_amdgcn_s_waitcnt(vm_imm(1 * LW)); break;
    case 2: if constexpr (NS > 3) __builtin_amdgcn_s_waitcnt(vm_imm(2 * LW)); break;
    case 3: if constexpr (NS > 4) __builtin_amdgcn_s_waitcnt(vm_imm(3 * LW)); break;
    case 4: if constexpr (NS > 5) __builtin_amdgcn_s_waitcnt(vm_imm(4 * LW)); break;
    case 5: if constexpr (NS > 6) __builtin_amdgcn_s_waitcnt(vm_imm(5 * LW)); break;
    case 6: if constexpr (NS > 7) __builtin_amdgcn_s_waitcnt(vm_imm(6 * LW)); break;
    case 7: if constexpr (NS > 8) __builtin_amdgcn_s_waitcnt(vm_imm(7 * LW)); break;
    default: __builtin_amdgcn_s_waitcnt(vm_imm(0)); break;
  }
}

// Pipeline stage layout (per KT-key tile): the K tile and then the V tile,
// each as rows of DH/8 16-byte chunks, XOR-swizzled (chunk c of key k at slot
// k*KCH + (c ^ (k & (KCH-1)))) so that both the K fragment reads and the
// transposing V reads hit distinct banks.  Both tiles arrive by
// global_load_lds_dwordx4: instruction i of a tile writes 64 consecutive
// 16-byte slots, and each lane's global address is chosen so that its slot
// receives the right chunk.
// Waves per SIMD: two work-groups of 8 waves per CU for the short stage ring
// of one query tile per wave (at most 128 VGPRs), else one work-group.
template <int DH, int KT, int QPW, int NS, int CAUX>
__global__ __launch_bounds__(kAttnThreads, (QPW == 4 ? 1 : (NS <= 4 && QPW == 1 ? 4 : 2))) void attn_bf16_kernel(
    AttnK a) {
  constexpr int KCH = DH / 8;             // 16-byte chunks per key row
  constexpr int TU4 = KT * KCH;           // 16-byte slots per K (or V) tile
  constexpr int NI = TU4 / 64;            // DMA instructions per K (or V) tile
  constexpr int LW = 2 * NI / kWaves;     // DMA instructions per wave per stage
  constexpr int KS = DH / 32;             // MFMA K-steps over the head dim
  constexpr int NKT = KT / 16;            // 16-key tiles per LDS tile
  static_assert(TU4 % 64 == 0 && (2 * NI) % kWaves == 0 && LW >= 1, "tile split");
  static_assert(NS >= 2 && NS <= 9 && (NS - 1) * LW < 64, "shape");

  __shared__ uint4 sStage[NS][2 * TU4];

  // ---- work item (XCD-aware: the query groups of one key chunk share an XCD)
  const int wid = blockIdx.x;
  const int xcd = wid % kXcd;
  const int t8 = wid / kXcd;
  const int qg = t8 % a.nqg;
  const int unit = (t8 / a.nqg) * kXcd + xcd;
  if (unit >= a.n_units) return;
  const int c = unit % a.nchunks;
  const int bh = unit / a.nchunks;
  const int kvh = bh % a.Hkv;
  const int b = bh / a.Hkv;

  int L = a.kv_len[b];
  L = L < 0 ? 0 : (L > a.cap ? a.cap : L);
  const int T = L + a.n_blk;
  const int kbeg = c * a.chunk;
  if (kbeg >= T) return;
  const int kend = min(T, kbeg + a.chunk);
  const bool single = (kbeg == 0 && kend == T);
  const int ntiles = (kend - kbeg + KT - 1) / KT;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar DMA bases
  const int g = lane >> 4;
  const int l16 = lane & 15;

  const size_t slab = (size_t)(b / a.epc) * a.Hkv + kvh;
  const uint16_t* kc_bh = a.kc + slab * a.cap * DH;
  const uint16_t* vc_bh = a.vc + slab * a.cap * DH;
  const uint16_t* kb_b = a.kb + ((size_t)b * a.n_blk * a.Hkv + kvh) * DH;
  const uint16_t* vb_b = a.vb + ((size_t)b * a.n_blk * a.Hkv + kvh) * DH;
  const size_t blk_stride = (size_t)a.Hkv * DH;

  // ---- this wave's query tiles, Q fragments kept in registers
  bool tact[QPW];
  int qblk[QPW];  // visibility limit (exclusive) per query row
  uint4 qf[QPW][KS];
  // running max (log2 units) and, for the lazy test, the raw score above which
  // it moves; running sums per lane (l_run, summed over the lanes at the end)
  // or from the P.V MFMAs (lsum, below)
  constexpr bool MS = NS > 4;  // not the 4-stage ring, whose 128 registers are full
  float m_run[QPW], m_raw[QPW], l_run[QPW];
  bd_f32x4 oacc[QPW][DH / 16], lsum[QPW];
#pragma unroll
  for (int j = 0; j < QPW; ++j) {
    const int t = (qg * kWaves + wave) * QPW + j;
    tact[j] = t < a.QT;
    const int r = t * 16 + l16;
    const bool rok = tact[j] && r < a.R;
    const int i = rok ? r / a.G : 0;
    const int hg = rok ? r % a.G : 0;
    // keys [0, vis_end) of the virtual sequence (cache rows, then in-block
    // rows) are visible: every cache row and the in-block rows of blocks up
    // to the query's own
    qblk[j] = rok ? L + ((a.q_off + i) / a.D + 1) * a.D : INT_MAX;
    const uint16_t* qp = a.q + (((size_t)b * a.n_q + i) * a.Hq + kvh * a.G + hg) * DH;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[j][ks] = rok ? *reinterpret_cast<const uint4*>(qp + 8 * g + 32 * ks) : make_uint4(0, 0, 0, 0);
    m_run[j] = BD_NEG_INF;
    m_raw[j] = BD_NEG_INF;
    l_run[j] = 0.f;
    lsum[j] = bd_f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < DH / 16; ++dt) oacc[j][dt] = bd_f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // Row sums of the probabilities (MS): one more P.V MFMA per query tile against
  // an all-ones V^T tile, whose 16 output rows all equal sum_k P[q][k] of the
  // same bf16 probabilities that weight V (no per-score adds in the softmax,
  // and no cross-lane sum at the end)
  const uint4 ones = make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u);
  const float inv_scale = 1.f / a.scale_log2;
  bool any_active = false;
#pragma unroll
  for (int j = 0; j < QPW; ++j) any_active |= tact[j];
  // keys below vis_all are inside the chunk and visible to every row of this
  // wave (a wave-uniform value)
  int vis_all = kend;
#pragma unroll
  for (int j = 0; j < QPW; ++j) vis_all = min(vis_all, qblk[j]);
  for (int off = 32; off > 0; off >>= 1) vis_all = min(vis_all, __shfl_xor(vis_all, off));

  // ---- asynchronous tile loads: this wave issues instructions wave + kWaves*u
  // of the stage (the first NI fill K, the next NI fill V)
  auto key_row = [&](const uint16_t* cache_bh, const uint16_t* blk_b, int key) -> const uint16_t* {
    key = key < kend ? key : kend - 1;  // rows past the chunk repeat a real row; their scores are masked
    return key < L ? cache_bh + (size_t)key * DH : blk_b + (size_t)(key - L) * blk_stride;
  };
  // per-lane element offset of the chunk this lane fetches, relative to the
  // first row of a tile (row kk, logical chunk ch), for each instruction
  int loff[LW];
#pragma unroll
  for (int u = 0; u < LW; ++u) {
    const int ins = wave + kWaves * u;
    const int p = (ins >= NI ? ins - NI : ins) * 64 + lane;
    const int kk = p / KCH, phys = p % KCH;
    loff[u] = kk * DH + (phys ^ (kk & (KCH - 1))) * 8;
  }
  const int cache_end = min(L, kend);  // tiles below this read only cache rows, none past the chunk
  auto issue = [&](int t) {
    uint4* st = sStage[t % NS];
    const int kbase = kbeg + t * KT;
    if (kbase + KT <= cache_end) {
#pragma unroll
      for (int u = 0; u < LW; ++u) {
        const int ins = wave + kWaves * u;
        const uint16_t* base = (ins >= NI ? vc_bh : kc_bh) + (size_t)kbase * DH;
        __builtin_amdgcn_global_load_lds((glb_void_t*)(base + loff[u]),
                                         (lds_void_t*)(st + (ins >= NI ? TU4 : 0) + (ins >= NI ? ins - NI : ins) * 64),
                                         16, 0, CAUX);
      }
    } else {
#pragma unroll
      for (int u = 0; u < LW; ++u) {
        const int ins = wave + kWaves * u;
        const bool isv = ins >= NI;
        const int kk = loff[u] / DH;
        const uint16_t* src = isv ? key_row(vc_bh, vb_b, kbase + kk) : key_row(kc_bh, kb_b, kbase + kk);
        __builtin_amdgcn_global_load_lds((glb_void_t*)(src + (loff[u] - kk * DH)),
                                         (lds_void_t*)(st + (isv ? TU4 : 0) + (isv ? ins - NI : ins) * 64), 16, 0, 0);
      }
    }
  };

  // The Q fragments (and every other global load so far) must be in
  // registers before the pipeline starts, so that no register wait on them
  // is left for the compiler to place inside the loop.  The prologue always
  // issues NS-1 stages: in a chunk of fewer tiles the extra stages re-read
  // the chunk's last rows (key_row clamps) into slots no tile uses, and the
  // loop's waits, which count them as older loads, still drain every load
  // before the work-group ends.
  __builtin_amdgcn_s_waitcnt(vm_imm(0));
#pragma unroll
  for (int t = 0; t < NS - 1; ++t) issue(t);
  // the guard's words load while the first stages are in flight
  if (bd_guard_dead(a.g_bits, a.g_mask, a.g_n)) {
    __builtin_amdgcn_s_waitcnt(vm_imm(0));  // no DMA into this LDS after the work-group ends
    return;
  }
  for (int t = 0; t < ntiles; ++t) {
    wait_stages<LW, NS>(min(ntiles - t - 1, NS - 2));
    pipe_barrier();  // tile t in LDS; every wave is done with tile t - 1
    if (t + NS - 1 < ntiles) issue(t + NS - 1);
    const uint4* sK = sStage[t % NS];
    const uint16_t* sV = reinterpret_cast<const uint16_t*>(sStage[t % NS] + TU4);
    if (any_active) {
      const int kbase = kbeg + t * KT;
      // S^T = K Q^T: lane holds keys 16*kt + 4g + r of query column l16
      bd_f32x4 s[QPW][NKT];
      constexpr bool kFast = (DH == 128 && KT == 32);
      uint4 vfr[kFast ? 8 : 1];
      auto load_vfrags = [&](uint4 (&out)[kFast ? 8 : 1]) {
        if constexpr (kFast) {
          uint32_t va[8];
          const uint32_t vb = lds_addr(sV);
          const int vrow = 4 * g + (l16 >> 2);
#pragma unroll
          for (int dt = 0; dt < 8; ++dt)
            va[dt] = vb + vrow * 256 + ((2 * dt + ((l16 & 3) >> 1)) ^ (vrow & 15)) * 16 + (l16 & 1) * 8;
          lds_vfrags_128x32(va, out);
        }
      };
      if constexpr (kFast) {
        uint4 kfr[2][4];
        uint32_t ka[4];
        const uint32_t kb = lds_addr(sK);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) ka[ks] = kb + (l16 * 16 + ((g + 4 * ks) ^ l16)) * 16;
        lds_kfrags_128x32(ka, kfr);
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) {
#pragma unroll
          for (int j = 0; j < QPW; ++j) s[j][kt] = bd_f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int j = 0; j < QPW; ++j)
              s[j][kt] = bd_mfma16(kfr[kt][ks], qf[j][ks], s[j][kt]);
        }
        // the V reads go out while the score MFMAs are still in the matrix pipe
        load_vfrags(vfr);
      } else {
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) {
#pragma unroll
          for (int j = 0; j < QPW; ++j) s[j][kt] = bd_f32x4{0.f, 0.f, 0.f, 0.f};
          const int kk = kt * 16 + l16;
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            const uint4 kf = sK[kk * KCH + ((g + 4 * ks) ^ (kk & (KCH - 1)))];
#pragma unroll
            for (int j = 0; j < QPW; ++j)
              s[j][kt] = bd_mfma16(kf, qf[j][ks], s[j][kt]);
          }
        }
      }
      // online softmax (base 2), probabilities packed as the B operand of P.V
      uint4 pf[QPW][KT / 32];
#pragma unroll
      for (int j = 0; j < QPW; ++j) {
        if (kbase + KT <= vis_all) {
          // Whole tile visible to every row: no mask, and a lazy running max.
          // Any common offset m gives the same softmax as long as every
          // contribution to a row uses it, so m_run only moves when some
          // score exceeds it by more than kLazyMax (probabilities stay below
          // 2^kLazyMax); otherwise no cross-lane reduction and no rescale.
          // (MS: the test is on raw scores, against m_raw = (m_run + kLazyMax) / scale)
          float mx;
          if constexpr (NKT == 2) {
            mx = vmax3(vmax3(s[j][0][0], s[j][0][1], s[j][0][2]), vmax3(s[j][0][3], s[j][1][0], s[j][1][1]),
                       vmax3(s[j][1][2], s[j][1][3], s[j][1][3]));
          } else {
            mx = s[j][0][0];
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
              for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[j][kt][r]);
          }
          bool up;
          if constexpr (MS) up = __ballot(mx > m_raw[j]) != 0;
          else up = __ballot(mx * a.scale_log2 > m_run[j] + kLazyMax) != 0;
          if (up) {
            const float smx = mx * a.scale_log2;
            float mall = fmaxf(smx, __shfl_xor(smx, 16));
            mall = fmaxf(mall, __shfl_xor(mall, 32));
            const float mnew = fmaxf(m_run[j], mall);
            const float alpha = bd_exp2(m_run[j] - mnew);
            m_run[j] = mnew;
            if constexpr (MS) m_raw[j] = (mnew + kLazyMax) * inv_scale;
            if constexpr (MS) lsum[j] *= alpha;
            else l_run[j] *= alpha;
#pragma unroll
            for (int dt = 0; dt < DH / 16; ++dt) oacc[j][dt] *= alpha;
          }
          const float mneg = -m_run[j];
          float ps = 0.f;
#pragma unroll
          for (int u = 0; u < KT / 32; ++u) {
            uint32_t w[4];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const bd_f32x4 sv = s[j][2 * u + h];
              const float p0 = bd_exp2(__builtin_fmaf(sv[0], a.scale_log2, mneg));
              const float p1 = bd_exp2(__builtin_fmaf(sv[1], a.scale_log2, mneg));
              const float p2 = bd_exp2(__builtin_fmaf(sv[2], a.scale_log2, mneg));
              const float p3 = bd_exp2(__builtin_fmaf(sv[3], a.scale_log2, mneg));
              if constexpr (!MS) ps += (p0 + p1) + (p2 + p3);
              w[2 * h] = cvt_pk_bf16(p0, p1);
              w[2 * h + 1] = cvt_pk_bf16(p2, p3);
            }
            pf[j][u] = make_uint4(w[0], w[1], w[2], w[3]);
          }
          if constexpr (!MS) l_run[j] += ps;
          continue;
        }
        float mx = BD_NEG_INF;
        {
          // key kbase + 16kt + 4g + r is visible iff 16kt + r < rel
          const int rel = min(kend, qblk[j]) - kbase - 4 * g;
#pragma unroll
          for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float v = kt * 16 + r < rel ? s[j][kt][r] * a.scale_log2 : BD_NEG_INF;
              s[j][kt][r] = v;
              mx = fmaxf(mx, v);
            }
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mnew = fmaxf(m_run[j], mx);
        const float muse = (mnew == BD_NEG_INF) ? 0.f : mnew;
        const float alpha = bd_exp2(m_run[j] - muse);
        m_run[j] = mnew;
        if constexpr (MS) m_raw[j] = (mnew + kLazyMax) * inv_scale;
        float ps = 0.f;
#pragma unroll
        for (int u = 0; u < KT / 32; ++u) {
          uint32_t w[4];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const bd_f32x4 sv = s[j][2 * u + h];
            const float p0 = bd_exp2(sv[0] - muse), p1 = bd_exp2(sv[1] - muse);
            const float p2 = bd_exp2(sv[2] - muse), p3 = bd_exp2(sv[3] - muse);
            if constexpr (!MS) ps += (p0 + p1) + (p2 + p3);
            w[2 * h] = cvt_pk_bf16(p0, p1);
            w[2 * h + 1] = cvt_pk_bf16(p2, p3);
          }
          pf[j][u] = make_uint4(w[0], w[1], w[2], w[3]);
        }
        if constexpr (!MS) l_run[j] = l_run[j] * alpha + ps;
        if (__ballot(alpha != 1.f) != 0) {  // the running max moved for some row
          if constexpr (MS) lsum[j] *= alpha;
#pragma unroll
          for (int dt = 0; dt < DH / 16; ++dt) oacc[j][dt] *= alpha;
        }
      }
      // O^T += V^T P^T: V^T fragment = two 4-key runs of one head-dim row
      // lane (g, l16) points at key 32u + 4g + l16/4 (and +16), head dims
      // 16dt + 4*(l16 % 4) .. +3; it receives keys 32u+4g..+3 (and +16..)
      // of head dim 16dt + l16, the slot order of the probabilities above
      const int vrow = 4 * g + (l16 >> 2);
#pragma unroll
      for (int u = 0; u < KT / 32; ++u) {
#pragma unroll
        for (int dt = 0; dt < DH / 16; ++dt) {
          uint4 vf;
          if constexpr (kFast) {
            vf = vfr[dt];
          } else {
            const int lch = 2 * dt + ((l16 & 3) >> 1);
            const int half = (l16 & 1) * 4;
            const int r0 = 32 * u + vrow, r1 = r0 + 16;
            const uint2 lo = lds_read_tr16(sV + r0 * DH + (lch ^ (r0 & (KCH - 1))) * 8 + half);
            const uint2 hi = lds_read_tr16(sV + r1 * DH + (lch ^ (r1 & (KCH - 1))) * 8 + half);
            vf = make_uint4(lo.x, lo.y, hi.x, hi.y);
          }
#pragma unroll
          for (int j = 0; j < QPW; ++j)
            oacc[j][dt] = bd_mfma16(vf, pf[j][u], oacc[j][dt]);
        }
        if constexpr (MS) {
#pragma unroll
          for (int j = 0; j < QPW; ++j) lsum[j] = bd_mfma16(ones, pf[j][u], lsum[j]);
        }
      }
    }
  }

  // ---- epilogue: normalised output (single chunk) or partials
#pragma unroll
  for (int j = 0; j < QPW; ++j) {
    if (!tact[j]) continue;
    float l;
    if constexpr (MS) {
      l = lsum[j][0];
    } else {
      l = l_run[j];
      l += __shfl_xor(l, 16);
      l += __shfl_xor(l, 32);
    }
    const int r = ((qg * kWaves + wave) * QPW + j) * 16 + l16;
    if (r >= a.R) continue;
    const int i = r / a.G, hg = r % a.G;
    if (single) {
      const float inv = l > 0.f ? 1.f / l : 0.f;
      uint16_t* op = a.o + (((size_t)b * a.n_q + i) * a.Hq + kvh * a.G + hg) * DH;
#pragma unroll
      for (int dt = 0; dt < DH / 16; ++dt) {
        const bd_f32x4 v = oacc[j][dt] * inv;
        *reinterpret_cast<uint2*>(op + dt * 16 + 4 * g) = make_uint2(cvt_pk_bf16(v[0], v[1]), cvt_pk_bf16(v[2], v[3]));
      }
      if (a.lse != nullptr && g == 0)
        a.lse[((size_t)b * a.Hq + kvh * a.G + hg) * a.n_q + i] = (m_run[j] + bd_log2(l)) * BD_LN2;
    } else {
      const size_t pi = (size_t)unit * (a.QT * 16) + r;
      float* po = a.part_o + pi * DH;
#pragma unroll
      for (int dt = 0; dt < DH / 16; ++dt)
        *reinterpret_cast<float4*>(po + dt * 16 + 4 * g) =
            make_float4(oacc[j][dt][0], oacc[j][dt][1], oacc[j][dt][2], oacc[j][dt][3]);
      if (g == 0) *reinterpret_cast<float2*>(a.part_ml + 2 * pi) = make_float2(m_run[j], l);
    }
  }
}

// Merge the key chunks of every (sequence, KV head) whose keys span more than
// one chunk: o = sum_c 2^(m_c - M) O_c / sum_c 2^(m_c - M) l_c.  One wave per
// query row; lane e holds head dims DH/64 * e .. (a 512-byte row per chunk).
// Chunks are taken NB at a time with an online maximum, so every load of a
// batch is in flight together and a row needs one round trip per batch;
// chunk indices past the end are clamped and weighted 0.
template <int DH, int NB>
__global__ __launch_bounds__(kThreads) void attn_merge_kernel(AttnK a) {
  if (bd_guard_dead(a.g_bits, a.g_mask, a.g_n)) return;
  constexpr int PER = DH / 64;  // head dims per lane
  const int lane = threadIdx.x & 63;
  const size_t row = (size_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (row >= (size_t)a.B * a.Hkv * a.R) return;
  const int r = (int)(row % a.R);
  const int bh = (int)(row / a.R);
  const int b = bh / a.Hkv, kvh = bh % a.Hkv;
  int L = a.kv_len[b];
  L = L < 0 ? 0 : (L > a.cap ? a.cap : L);
  const int nc = (L + a.n_blk + a.chunk - 1) / a.chunk;
  if (nc <= 1) return;
  const size_t rp = (size_t)a.QT * 16;
  const size_t base = (size_t)bh * a.nchunks * rp + r;  // partial index of chunk c: base + c * rp
  float M = BD_NEG_INF, lsum = 0.f;
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  for (int c0 = 0; c0 < nc; c0 += NB) {
    float mv[NB], lv[NB], ov[NB][PER];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const size_t pi = base + (size_t)min(c0 + u, nc - 1) * rp;
      const float2 ml = *reinterpret_cast<const float2*>(a.part_ml + 2 * pi);
      mv[u] = ml.x;
      lv[u] = ml.y;
      const float* po = a.part_o + pi * DH + PER * lane;
      if constexpr (PER == 2) {
        const float2 v = *reinterpret_cast<const float2*>(po);
        ov[u][0] = v.x;
        ov[u][1] = v.y;
      } else {
        ov[u][0] = po[0];
      }
    }
    float mb = M;
#pragma unroll
    for (int u = 0; u < NB; ++u)
      if (c0 + u < nc) mb = fmaxf(mb, mv[u]);
    const float muse = (mb == BD_NEG_INF) ? 0.f : mb;
    const float alpha = bd_exp2(M - muse);  // 0 while nothing has been seen
    lsum *= alpha;
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] *= alpha;
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const float w = (c0 + u < nc) ? bd_exp2(mv[u] - muse) : 0.f;
      lsum += w * lv[u];
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] += w * ov[u][e];
    }
    M = mb;
  }
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  const int i = r / a.G, hg = r % a.G;
  uint16_t* op = a.o + (((size_t)b * a.n_q + i) * a.Hq + kvh * a.G + hg) * DH + PER * lane;
  if constexpr (PER == 2)
    *reinterpret_cast<uint32_t*>(op) = cvt_pk_bf16(acc[0] * inv, acc[1] * inv);
  else
    op[0] = (uint16_t)(cvt_pk_bf16(acc[0] * inv, 0.f) & 0xffffu);
  if (a.lse != nullptr && lane == 0)
    a.lse[((size_t)b * a.Hq + kvh * a.G + hg) * a.n_q + i] = (M + bd_log2(lsum)) * BD_LN2;
}

// ---- fp32 path -------------------------------------------------------------
struct AttnF {
  const float* q;
  const float* kc;
  const float* vc;
  const int32_t* kv_len;
  const float* kb;
  const float* vb;
  float* o;
  float* lse;
  int Hq, Hkv, G, d, D, n_q, q_off, cap, n_blk, epc;
  float scale;
  const uint64_t* g_bits;
  uint64_t g_mask;
  int g_n;
};

__device__ float block_reduce(float v, bool is_max, float* red) {
  for (int off = 32; off > 0; off >>= 1) {
    const float w = __shfl_xor(v, off);
    v = is_max ? fmaxf(v, w) : v + w;
  }
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
  for (int w = 1; w < kThreads / 64; ++w) r = is_max ? fmaxf(r, red[w]) : r + red[w];
  return r;
}

__global__ __launch_bounds__(kThreads) void attn_f32_kernel(AttnF a) {
  if (bd_guard_dead(a.g_bits, a.g_mask, a.g_n)) return;
  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int kvh = h / a.G;
  int L = a.kv_len[b];
  L = L < 0 ? 0 : (L > a.cap ? a.cap : L);
  const int T = L + a.n_blk;
  const int qblk = (a.q_off + i) / a.D;
  __shared__ float sq[128];
  __shared__ float sp[kThreads];
  __shared__ float red[kThreads / 64];
  if (tid < a.d) sq[tid] = a.q[(((size_t)b * a.n_q + i) * a.Hq + h) * a.d + tid];
  __syncthreads();
  const size_t slab = (size_t)(b / a.epc) * a.Hkv + kvh;
  auto kp = [&](const float* cache, const float* blk, int key) -> const float* {
    return key < L ? cache + (slab * a.cap + key) * a.d
                   : blk + (((size_t)b * a.n_blk + (key - L)) * a.Hkv + kvh) * a.d;
  };
  float m = -__builtin_inff(), l = 0.f, acc = 0.f;
  for (int base = 0; base < T; base += kThreads) {
    const int key = base + tid;
    float s = -__builtin_inff();
    if (key < T && (key < L || (key - L) / a.D <= qblk)) {
      const float* k = kp(a.kc, a.kb, key);
      float dot = 0.f;
      for (int e = 0; e < a.d; ++e) dot += sq[e] * k[e];
      s = dot * a.scale;
    }
    const float cm = block_reduce(s, true, red);
    const float mnew = fmaxf(m, cm);
    const float muse = (mnew == -__builtin_inff()) ? 0.f : mnew;
    const float p = (s == -__builtin_inff()) ? 0.f : expf(s - muse);
    sp[tid] = p;
    const float ps = block_reduce(p, false, red);
    const float alpha = (m == -__builtin_inff()) ? 0.f : expf(m - muse);
    l = l * alpha + ps;
    if (tid < a.d) {
      float a2 = 0.f;
      const int n = min(kThreads, T - base);
      for (int kk = 0; kk < n; ++kk)
        if (sp[kk] != 0.f) a2 += sp[kk] * kp(a.vc, a.vb, base + kk)[tid];
      acc = acc * alpha + a2;
    }
    m = mnew;
    __syncthreads();
  }
  if (tid < a.d) a.o[(((size_t)b * a.n_q + i) * a.Hq + h) * a.d + tid] = acc / l;
  if (a.lse != nullptr && tid == 0) a.lse[((size_t)b * a.Hq + h) * a.n_q + i] = m + logf(l);
}

}  // namespace

BdAttnPlan bd_attn_plan(bd_dtype dt, int B, int Hq, int Hkv, int d, int n_q, int cap, int n_blk) {
  BdAttnPlan p{};
  const int G = Hq / Hkv;
  p.R = n_q * G;
  p.QT = (p.R + 15) / 16;
  p.qpw = p.QT <= kWaves ? 1 : (p.QT <= 2 * kWaves ? 2 : 4);
  p.qpw = p.qpw > kQpwMax ? kQpwMax : p.qpw;
  p.nqg = (p.QT + kWaves * p.qpw - 1) / (kWaves * p.qpw);
  const int tmax = cap + n_blk;
  p.stream_nt = (long long)B * Hkv * cap * d * 2 * (dt == BD_F32 ? 4 : 2) >= BD_ATTN_NT_MIN_BYTES;
  if (dt == BD_F32) {
    p.chunk = tmax;
    p.nchunks = 1;
    return p;
  }
  // one query tile per wave only (the register budget of two work-groups per
  // CU): exact steps split into two query groups measured slower
  p.light = (long long)B * Hkv * cap * d * 2 * 2 <= BD_ATTN_LIGHT_MAX_BYTES && p.qpw == 1;
  const long base = (long)B * Hkv * p.nqg;
  const long target = p.light ? 2 * kTargetWGs : kTargetWGs;
  int nch = (int)((target + base - 1) / base);
  const int max_ch = (tmax + kMinChunk - 1) / kMinChunk;
  nch = nch < 1 ? 1 : (nch > max_ch ? max_ch : nch);
  int chunk = (tmax + nch - 1) / nch;
  chunk = (chunk + kKT - 1) / kKT * kKT;
  p.chunk = chunk;
  p.nchunks = (tmax + chunk - 1) / chunk;
  if (p.nchunks > 1) {
    const size_t rows = (size_t)B * Hkv * p.nchunks * p.QT * 16;
    p.part_o = 0;
    p.part_ml = rows * d * sizeof(float);
    p.ws_bytes = p.part_ml + rows * 2 * sizeof(float);
  }
  return p;
}

hipError_t bd_attn_launch(bd_dtype dt, const BdAttnPlan& p, const BdAttnArgs& x, hipStream_t s) {
  if (dt == BD_F32) {
    AttnF a{static_cast<const float*>(x.q), static_cast<const float*>(x.k_cache),
            static_cast<const float*>(x.v_cache), x.kv_len, static_cast<const float*>(x.k_blk),
            static_cast<const float*>(x.v_blk), static_cast<float*>(x.o), x.lse,
            x.Hq, x.Hkv, x.G, x.d, x.D, x.n_q, x.q_off, x.cap, x.n_blk, x.epc, x.scale,
            x.guard ? x.guard->bits : nullptr, x.guard ? x.guard->mask : 0, x.guard ? x.guard->n : 0};
    hipLaunchKernelGGL(attn_f32_kernel, dim3(x.n_q, x.Hq, x.B), dim3(kThreads), 0, s, a);
    return hipGetLastError();
  }
  AttnK a{};
  a.q = static_cast<const uint16_t*>(x.q);
  a.kc = static_cast<const uint16_t*>(x.k_cache);
  a.vc = static_cast<const uint16_t*>(x.v_cache);
  a.kv_len = x.kv_len;
  a.kb = static_cast<const uint16_t*>(x.k_blk);
  a.vb = static_cast<const uint16_t*>(x.v_blk);
  a.o = static_cast<uint16_t*>(x.o);
  a.lse = x.lse;
  a.part_o = x.part_o;
  a.part_ml = x.part_ml;
  a.B = x.B; a.Hq = x.Hq; a.Hkv = x.Hkv; a.G = x.G; a.D = x.D; a.n_q = x.n_q; a.q_off = x.q_off;
  a.cap = x.cap; a.n_blk = x.n_blk; a.epc = x.epc;
  a.R = p.R; a.QT = p.QT; a.nqg = p.nqg; a.chunk = p.chunk; a.nchunks = p.nchunks;
  a.n_units = x.B * x.Hkv * p.nchunks;
  a.scale_log2 = x.scale * BD_LOG2E;
  a.g_bits = x.guard ? x.guard->bits : nullptr;
  a.g_mask = x.guard ? x.guard->mask : 0;
  a.g_n = x.guard ? x.guard->n : 0;
  const int n_wg = kXcd * a.nqg * ((a.n_units + kXcd - 1) / kXcd);
#define BD_ATTN_LAUNCH(DH, QPW)                                                                               \
  do {                                                                                                        \
    if (p.stream_nt)                                                                                          \
      hipLaunchKernelGGL((attn_bf16_kernel<DH, kKT, QPW, kNS, 2>), dim3(n_wg), dim3(kAttnThreads), 0, s, a);     \
    else if (p.light)                                                                                         \
      hipLaunchKernelGGL((attn_bf16_kernel<DH, kKT, QPW, kLightNS, 0>), dim3(n_wg), dim3(kAttnThreads), 0, s, a); \
    else                                                                                                      \
      hipLaunchKernelGGL((attn_bf16_kernel<DH, kKT, QPW, kNS, 0>), dim3(n_wg), dim3(kAttnThreads), 0, s, a);     \
  } while (0)
  if (x.d == 128) {
    if (p.qpw == 1) BD_ATTN_LAUNCH(128, 1);
#if BD_ATTN_QPW_MAX >= 2
    else if (p.qpw == 2) BD_ATTN_LAUNCH(128, 2);
#endif
#if BD_ATTN_QPW_MAX >= 4
    else BD_ATTN_LAUNCH(128, 4);
#endif
  } else {
    if (p.qpw == 1) BD_ATTN_LAUNCH(64, 1);
#if BD_ATTN_QPW_MAX >= 2
    else if (p.qpw == 2) BD_ATTN_LAUNCH(64, 2);
#endif
#if BD_ATTN_QPW_MAX >= 4
    else BD_ATTN_LAUNCH(64, 4);
#endif
  }
#undef BD_ATTN_LAUNCH
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.nchunks == 1) return e;
  const size_t rows = (size_t)x.B * x.Hkv * p.R;
  const dim3 grid((unsigned)((rows + kThreads / 64 - 1) / (kThreads / 64)));
#define BD_MERGE_LAUNCH(DH, NB) hipLaunchKernelGGL((attn_merge_kernel<DH, NB>), grid, dim3(kThreads), 0, s, a)
  const int nb = p.nchunks <= 2 ? 2 : (p.nchunks <= 4 ? 4 : 8);
  if (x.d == 128) {
    if (nb == 2) BD_MERGE_LAUNCH(128, 2);
    else if (nb == 4) BD_MERGE_LAUNCH(128, 4);
    else BD_MERGE_LAUNCH(128, 8);
  } else {
    if (nb == 2) BD_MERGE_LAUNCH(64, 2);
    else if (nb == 4) BD_MERGE_LAUNCH(64, 4);
    else BD_MERGE_LAUNCH(64, 8);
  }
#undef BD_MERGE_LAUNCH
  return hipGetLastError();
}
