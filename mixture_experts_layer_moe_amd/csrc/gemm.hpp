// bf16 MFMA GEMM for gfx950:  C[m, n] = sum_k A[m, k] * B[n, k]  (fp32 accumulate)
//
// Both operands are K-contiguous ("NT" layout: every weight of the layer is
// stored [out, in]), so one 16-byte load along K feeds one MFMA operand lane.
//
// Design
//   * Persistent, XCD-balanced: the grid is a multiple of 8 workgroups, one per
//     CU; workgroup b runs on XCD b % 8.  The CUs of one XCD work on
//     neighbouring tiles, so tiles that share an expert's weight panel or an
//     activation panel share that XCD's L2.  With a queue (grouped GEMMs) the
//     tile list (known only on the device) is cut into chunks of n_tiles
//     consecutive tiles dealt to the XCDs in turn, and each workgroup takes
//     the next tile of its XCD's chunks from an atomic counter when it
//     finishes one, so the tiles in flight on an XCD stay a contiguous window
//     (workgroups never drift apart, and M tiles that read the same weight
//     tile run together) and the 8 XCDs stream neighbouring experts (1-3%
//     faster than 8 contiguous ranges).  Without a queue (dense GEMMs) the
//     list is cut into 8 contiguous ranges walked round-robin.  Either way
//     each tile is computed the same way, so results do not depend on the
//     assignment.
//   * Operands go global -> LDS directly (buffer_load_dwordx4 ... lds), no
//     register staging, in an NSTAGE-deep ring of BK-wide K stages (BK = 64:
//     128-byte LDS rows; BK = 32: 64-byte rows, so a 256x256 tile fits four
//     stages in LDS), so NSTAGE-1 stages of loads are in flight while the
//     MFMAs run.  Each load instruction fills 1 KB (8 or 16 rows); the 16-byte
//     chunks of a row are XOR-swizzled by row bits so that the 16 rows one
//     fragment read touches fall on distinct LDS banks.  Rows past the end of
//     the matrix (ragged expert segments, N tails) are out of the buffer
//     descriptor's range and load as zeros.  BNT marks the weight (B) loads
//     non-temporal: weights streamed once should not evict reused activations.
//   * Each wave owns a (BM/WM) x (BN/WN) sub-tile of 32x32 blocks of
//     v_mfma_f32_32x32x16_bf16 (on gfx950 this shape sustains ~88% of the
//     bf16 peak back to back, the 16x16x32 shape ~64%); 32-row blocks past
//     the tile's last valid row are skipped (a small expert costs MFMA time
//     in proportion to its rows).
//   * Up to three K segments (A_s, B_s, K_s) chain in one accumulation: the
//     split-bf16 router (x against the hi/mid/lo parts of W_r) and the
//     up-projection with the shared expert's down-projection appended along K.
//     The segment count is a template parameter and every segment's buffer
//     descriptors are built once per tile, so the K loop does no scalar
//     memory loads (whose lgkmcnt waits would also drain the LDS reads).
//   * GROUPED: M is the expert-ordered row list; tiles never straddle two
//     experts.  Device tables (prefix of per-expert M-tile counts and the
//     expert of every M-tile) map a tile index to (expert, M-tile, N-tile)
//     with no host sync; an expert's rows are split into its M tiles evenly
//     (heights a multiple of 32 rows).  Order: expert, then groups of
//     GROUPED_GM M tiles, then N tile, then M tile, so M tiles of one expert
//     that read the same weight tile run side by side, and an expert with
//     many M tiles does not re-stream its activation panels once per N tile.
//     GATHER: A row r is row row_token[r] of the activations (the token
//     permutation is fused into the A load).
//   * EPI_SWIGLU: the B tile interleaves 32-row blocks of W_g and W_u for the
//     same output columns, so each lane holds the gate and up values of the
//     same (row, column) and applies silu(g) * u before one bf16 store.
//   * F8: both operands are FP8 E4M3 bytes with per-tensor scales (A: one
//     activation scale; B: one scale per expert).  A stage row is still 128
//     (or 64) bytes, now 128 (64) K values, consumed by
//     v_mfma_scale_f32_32x32x64_f8f6f4 with unit block scales (a lane takes
//     32 contiguous bytes of its row, the same assignment for A and B); the
//     epilogue multiplies by 1 / (s_A s_B).  EPI_Q8 / EPI_SWIGLU_Q8 write the
//     bf16-rounded result as FP8 instead (quantized with an output scale, the
//     conversion clamped to +-448, because the hardware conversion does not
//     saturate) and record the largest |bf16 value| for delayed scaling: a
//     running maximum per wave, one integer atomic max per wave at the end
//     (the bit patterns of non-negative floats order like unsigned integers,
//     so the result does not depend on the order).
//   * F8 = F8_E5M2_A (the backward's data-gradient GEMMs): A is an E5M2
//     gradient (scale 128 s_A), B an E4M3 weight; the MFMA takes A's format
//     as its source-0 format code.  With two K segments each segment has its
//     own scales: at the second segment's first stage the accumulators are
//     multiplied by dq_1 / dq_2 and the epilogue by dq_2 (so each segment's
//     products end up divided by their own scales).
//   * EPI_F32_ADD: fp32 C += the product (each element read and written by
//     the one lane that owns it: deterministic).
//   * EPI_GU_BWD / EPI_GU_BWD_Q8: the gate/up GEMM of the backward
//     (recomputation) with the SwiGLU backward in the epilogue; the _Q8
//     variant also writes dg and du as E5M2 codes and records their maxima.
#pragma once

#include <type_traits>

#include "common.hpp"

namespace moe {

constexpr uint32_t RSRC_WORD3 = 0x00020000u;   // raw buffer, 32-bit data format (gfx9)
constexpr int DENSE_GM = 4;                     // M panels per tile group (dense GEMMs)
// M tiles per tile group inside one expert of a grouped GEMM.  An expert with
// many M tiles (a hot expert of an imbalanced routing: 128 tiles of 256 rows)
// would otherwise have all its M tiles read one weight tile after another,
// re-streaming each activation panel once per N tile; in groups, the ~32
// tiles an XCD runs side by side span a few M panels and a few N tiles
// (4 x 8), so both operands are shared through its L2.
constexpr int GROUPED_GM = 4;

enum GemmEpi { EPI_BF16 = 0, EPI_F32 = 1, EPI_F32_BIAS = 2, EPI_SWIGLU = 3, EPI_Q8 = 4,
               EPI_SWIGLU_Q8 = 5, EPI_GU_BWD = 6, EPI_GU_BWD_Q8 = 7, EPI_F32_ADD = 8 };

// FP8 operand formats of a GEMM (template parameter F8): none (bf16), both
// operands E4M3, or the activation operand (A) E5M2 and the weights E4M3
enum GemmF8 { F8_NONE = 0, F8_E4M3 = 1, F8_E5M2_A = 2 };

// B tiles that interleave the gate and up matrices (a lane holds g and u of
// the same element)
constexpr bool epi_swiglu(int epi) {
  return epi == EPI_SWIGLU || epi == EPI_SWIGLU_Q8 || epi == EPI_GU_BWD || epi == EPI_GU_BWD_Q8;
}
constexpr bool epi_gu_bwd(int epi) { return epi == EPI_GU_BWD || epi == EPI_GU_BWD_Q8; }
constexpr float E4M3_MAX = 448.0f;

struct GemmSeg {
  const void* A;        // row r at A + arow(r) * lda elements
  const void* B;        // row n at B + n * ldb (+ expert * b_expert_stride) elements
  const void* B2;       // SwiGLU: the up matrix (B holds the gate matrix)
  int64_t lda, ldb;     // in elements (bf16 or fp8)
  int K;
};

struct GemmArgs {
  GemmSeg seg[3];
  int nseg;
  int M;                       // dense: rows of A and C; GATHER: rows of A
  int N;                       // output columns (EPI_SWIGLU: columns of H)
  const int32_t* offsets;      // grouped: [E+1] expert row offsets
  const int32_t* tile_prefix;  // grouped: [E+1] prefix of per-expert M-tile counts
  const int32_t* tile_expert;  // grouped: expert of every M tile
  int E;
  int64_t b_expert_stride;
  const int32_t* row_token;    // GATHER
  int32_t* queue;              // optional: 8 per-XCD tile counters, zero at launch
  void* C;
  int64_t ldc;
  const float* bias;           // EPI_F32_BIAS
  int n_tiles;
  int m_tiles;                 // dense
  // FP8 operands: quantization scales of A (1 value) and of B / B2 (one per
  // expert; dense: one); EPI_Q8 / EPI_SWIGLU_Q8: output scale and amax slot
  const float* a_scale;
  const float* b_scale;
  const float* b2_scale;
  const float* out_scale;
  uint32_t* amax;
  // FP8 with two K segments: the A scale of the second segment (its B scale
  // is b2_scale).  The products of each segment are divided by their own
  // scales.
  const float* a2_scale;
  // grouped, multi-round schedule: expert e's rows this round are
  // [offsets[e], seg_end[e]) (seg_end null: offsets[e + 1]); with h_base,
  // row r of expert e sits at row h_base[e] + (r - offsets[e]) of the round's
  // activation buffer, which is C (h_side 1: gate/up) or A (h_side 2: down)
  const int32_t* seg_end;
  const int32_t* h_base;
  int h_side;
  // backward.  EPI_GU_BWD (the gate/up GEMM recomputed): with g, u the
  // accumulators and dh = aux_g at the same (row, column) (leading dimension
  // ldc, fp32): dg = dh u silu'(g) -> C and du = dh silu(g) -> C2 as bf16,
  // rounded to nearest even (sr == 0) or stochastically with the random
  // stream keys sr_key_c, sr_key_c2 (element index row * ldc + column), and
  // h = bf16(silu(g) u) -> C3 (the forward's h, bit for bit).
  // KG (K-grouped tiles, weight gradients): tile -> (expert, M tile, N tile)
  // with expert e's K range [kpre[e], kpre[e + 1]) of A and B (multiples of
  // the stage width), C of expert e at C + e * c_expert_stride.
  // EPI_GU_BWD_Q8 also writes dg and du as E5M2 codes -> C4, C5, scaled by
  // 128 out_scale[1] and 128 out_scale[2], rounded to nearest (sr == 0) or
  // stochastically with the keys sr_key_c4, sr_key_c5 (same element index),
  // and records max |dg|, max |du| (fp32, before scaling) in amax[1], amax[2].
  void* C2;
  void* C3;
  void* C4;
  void* C5;
  const float* aux_g;
  uint32_t sr_key_c, sr_key_c2, sr_key_c4, sr_key_c5;
  int sr;
  const int32_t* kpre;
  int64_t c_expert_stride;
  // dense, split K (ksplit > 1): the concatenated K stages are cut into
  // ksplit chunks of equal length (the last may be shorter or empty); tile
  // -> (chunk, M tile, N tile), chunk s writing its partial result to
  // C + s * c_split (the caller sums the chunks)
  int ksplit;
  int64_t c_split;
};

// fp32 -> FP8 E4M3 byte, round to nearest even, saturating at +-448
__device__ __forceinline__ uint8_t f32_to_e4m3_sat(float v) {
  v = fminf(fmaxf(v, -E4M3_MAX), E4M3_MAX);
  return (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(v, 0.0f, 0, false) & 0xff);
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  if (bytes < 0) bytes = 0;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, RSRC_WORD3);
}

// One 16-byte load per lane straight into LDS at lds + 16 * lane.  NT sets the
// non-temporal cache policy bit.
template <bool NT = false>
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint4* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 16, voff, 0, 0, NT ? 2 : 0);
}

// Position of 16-byte chunk c of LDS row r (KCH chunks per row).  gfx950's
// LDS has 64 four-byte banks and serves a 16-byte-per-lane read 16 lanes
// (256 bytes) at a time, so the 16 consecutive rows one such group of a
// fragment read touches must cover all 16 bank quads.  128-byte rows: rows
// r and r + 8 share a bank half, so c ^ (r & 7) ^ ((r >> 3) & 1) (measured:
// 166 B/clk/CU of fragment reads against 103 for c ^ (r & 7)).  64-byte rows:
// c ^ ((r >> 1) & 3) ^ ((r >> 3) & 1), which maps rows r, r + 4, r + 8,
// r + 12 (same bank quad) to different chunks.  Both depend on r & 15 only.
template <int KCH>
__device__ __forceinline__ int swz(int r) {
  if constexpr (KCH == 8) return (r & 7) ^ ((r >> 3) & 1);
  else return ((r >> 1) & 3) ^ ((r >> 3) & 1);
}

// Workgroup barrier that orders LDS reads and writes only.  __syncthreads()
// (and any compiler fence that covers LDS) also waits for every outstanding
// vector-memory access, LDS DMA included, i.e. it would drain the whole load
// ring; the ring's completion is tracked with explicit vmcnt waits instead.
// The "memory" clobber keeps the compiler from moving memory accesses across.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int BM, int BN, int BK, int WM, int WN, int NSTAGE, bool GROUPED, bool GATHER, int EPI,
          bool BNT, int NSEG, int F8, bool KG>
__global__ __launch_bounds__(64 * WM * WN, 1) void gemm_kernel(GemmArgs a) {
  constexpr int ES = F8 ? 1 : 2;                   // operand bytes per element
  constexpr int KE = BK * 2 / ES;                  // K values per stage (BK * 2 bytes per row)
  constexpr bool SWG = epi_swiglu(EPI);
  constexpr bool Q8 = EPI == EPI_Q8 || EPI == EPI_SWIGLU_Q8;
  constexpr bool GBQ8 = EPI == EPI_GU_BWD_Q8;
  // FP8 with two K segments: separate dequantization of each segment
  constexpr bool SEG_DQ = F8 != F8_NONE && NSEG == 2 && !epi_swiglu(EPI);
  // the A operand's scale multiplier: E5M2 gradients take 128 s
  constexpr float A_SMUL = F8 == F8_E5M2_A ? E5M2_OVER_E4M3 : 1.0f;
  static_assert(!GBQ8 || F8 == F8_NONE, "the gate/up recompute runs on bf16 operands");
  constexpr int NW = WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  constexpr int KCH = BK / 8;                      // 16-byte chunks per LDS row
  constexpr int RPI = 64 / KCH;                    // rows per DMA instruction (1 KB)
  constexpr int A_INS = BM / RPI / NW;             // DMA instructions per wave per stage
  constexpr int B_INS = BN / RPI / NW;
  constexpr int LPS = A_INS + B_INS;
  constexpr int STAGE = (BM + BN) * KCH;           // 16-byte slots per stage
  static_assert(BK == 32 || BK == 64, "stage width");
  static_assert(BM % (RPI * NW) == 0 && BN % (RPI * NW) == 0, "tile / waves");
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile");
  (void)WTM;
  static_assert(!SWG || WTN % 64 == 0, "swiglu pairs");
  static_assert(NSTAGE >= 2 && NSTAGE <= 4 && LPS * (NSTAGE - 2) < 64, "stages");
  static_assert(NSEG >= 1 && NSEG <= 3 && (!GATHER || NSEG == 1), "K segments");
  __shared__ uint4 smem[NSTAGE * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
  // The tile's 32-row blocks are dealt to the WM wave rows in turn (block b
  // to wave row b % WM), so a tile with few valid rows still spreads its
  // MFMA work over every SIMD.
  const int wrow = wave / WN;
  const int wn0 = (wave % WN) * WTN;
  const int lrow = lane / KCH;                     // row inside a DMA row group
  // chunk this lane fetches: the swizzle of its LDS row, which is
  // (wave + i NW) RPI + lrow for DMA instruction i and equals
  // wave RPI + lrow in its low four bits
  static_assert((NW * RPI) % 16 == 0, "DMA row groups keep the swizzle per lane");
  const int lchunk = (lane % KCH) ^ swz<KCH>(wave * RPI + lrow);
  const int fr = lane & 31;                        // fragment row inside a 32-row block
  const int fq = lane >> 5;                        // which half of a sub-step's K this lane holds

  int total;
  static_assert(!(KG && (GROUPED || GATHER || NSEG != 1)), "K-grouped tiles: one plain segment");
  if constexpr (GROUPED) total = a.tile_prefix[a.E] * a.n_tiles;
  else if constexpr (KG) total = a.E * a.m_tiles * a.n_tiles;
  else total = a.m_tiles * a.n_tiles * (a.ksplit > 1 ? a.ksplit : 1);
  const int xcd = blockIdx.x & 7;
  const int nj = gridDim.x >> 3;
  const int t_begin = (int)((int64_t)total * xcd / 8);
  const int t_end = (int)((int64_t)total * (xcd + 1) / 8);

  // K segment boundaries and strides, read once (static indices only, so
  // they stay in scalar registers instead of being re-read in the K loop)
  int kseg[3] = {0, 0, 0};
  uint32_t lda2[3] = {0, 0, 0}, ldb2[3] = {0, 0, 0};
  int ktotal = 0;
  static_for<0, NSEG>([&](auto sc) {
    constexpr int S = decltype(sc)::value;
    kseg[S] = a.seg[S].K;
    lda2[S] = (uint32_t)(a.seg[S].lda * ES);
    ldb2[S] = (uint32_t)(a.seg[S].ldb * ES);
    ktotal += kseg[S];
  });
  const int nk_all = ktotal / KE;
  int nk = nk_all;           // K-grouped and split-K tiles: set per tile
  float amax_run = 0.f;     // Q8: largest |bf16 output| this lane wrote
  float amax_dg = 0.f, amax_du = 0.f;   // GBQ8: largest |dg|, |du| of this lane

  // The queue's tile index is broadcast through the first 16 bytes of the
  // ring's last stage (one LDS object only, so the compiler's LDS-DMA alias
  // tracking does not add waits in the K loop; and the ring can take the
  // whole LDS).  That stage is free here: the previous tile's loads have all
  // landed and its reads ended at its last barrier; the next tile's first
  // stages go to the other slots, and the loop loads into the last one only
  // after its first barrier, which every wave reaches after reading the
  // index.
  auto next_tile = [&](int prev) -> int {
    if (a.queue == nullptr) return prev < 0 ? t_begin + (blockIdx.x >> 3) : prev + nj;
    int* slot = (int*)&smem[(NSTAGE - 1) * STAGE];
    if (tid == 0) {
      // the XCD's kq-th tile: chunks of n_tiles consecutive tiles are dealt
      // to the XCDs in turn (chunk c to XCD c % 8)
      const int kq = atomicAdd(&a.queue[xcd], 1);
      const int ch = a.n_tiles > 0 ? a.n_tiles : 1;
      const int64_t tt = (int64_t)(xcd + 8 * (kq / ch)) * ch + kq % ch;
      *slot = tt < total ? (int)tt : total;
    }
    lds_barrier();     // every thread read the previous value before the end-of-tile barrier
    // the same value in every lane: make it wave-uniform, so the tile's
    // indices and buffer descriptors live in scalar registers (a descriptor
    // in vector registers turns every DMA into a waterfall loop)
    return __builtin_amdgcn_readfirstlane(*slot);
  };
  const int t_stop = a.queue ? total : t_end;
  for (int t = next_tile(-1); t < t_stop; t = next_tile(t)) {
    // ---- decode the tile ----
    int r0, mrows, n_tile;
    int a_r0, c_r0;                    // first row of the tile in A (no gather) and in C
    int64_t b_off = 0;
    float dq_b = 1.f, dq_b2 = 1.f;     // F8: 1 / (s_A s_B), 1 / (s_A s_B2)
    int kg_e = 0, kg_k0 = 0, kg_k = 0; // KG: expert, first K column and K extent
    int kt0 = 0, ks = 0;               // split K: the chunk's first stage, the chunk
    if constexpr (GROUPED) {
      // table reads at a uniform address: every lane gets the same value
      const int e = __builtin_amdgcn_readfirstlane(a.tile_expert[t / a.n_tiles]);
      const int p0 = __builtin_amdgcn_readfirstlane(a.tile_prefix[e]);
      const int mt = __builtin_amdgcn_readfirstlane(a.tile_prefix[e + 1]) - p0;
      const int rem = t - p0 * a.n_tiles;
      // inside the expert, groups of GROUPED_GM M tiles: a group goes N tile
      // by N tile with the M tile fastest (an expert with at most GROUPED_GM
      // M tiles is one group: N tile, then M tile)
      const int grp = rem / (GROUPED_GM * a.n_tiles);
      const int gm = min(GROUPED_GM, mt - grp * GROUPED_GM);
      const int rg = rem - grp * GROUPED_GM * a.n_tiles;
      n_tile = rg / gm;
      const int m_local = grp * GROUPED_GM + (rg - n_tile * gm);
      const int rs = __builtin_amdgcn_readfirstlane(a.offsets[e]);
      const int re = __builtin_amdgcn_readfirstlane(a.seg_end ? a.seg_end[e] : a.offsets[e + 1]);
      // the expert's rows split into mt tiles of equal height (a multiple of
      // 32, at most BM): no tile is mostly empty, e.g. 574 rows -> 3 x 192
      const int th = ((re - rs + mt - 1) / mt + 31) / 32 * 32;
      r0 = rs + m_local * th;
      mrows = min(th, re - r0);
      const int hr0 = a.h_base ? __builtin_amdgcn_readfirstlane(a.h_base[e]) + (r0 - rs) : r0;
      a_r0 = a.h_side == 2 ? hr0 : r0;
      c_r0 = a.h_side == 1 ? hr0 : r0;
      b_off = (int64_t)e * a.b_expert_stride * ES;
      if constexpr (F8 != F8_NONE) {
        dq_b = 1.0f / (A_SMUL * a.a_scale[0] * a.b_scale[e]);
        if constexpr (SWG) dq_b2 = 1.0f / (A_SMUL * a.a_scale[0] * a.b2_scale[e]);
        if constexpr (SEG_DQ) dq_b2 = 1.0f / (A_SMUL * a.a2_scale[0] * a.b2_scale[e]);
      }
    } else if constexpr (KG) {
      // expert, then N tile, then M tile (M fastest)
      const int per = a.m_tiles * a.n_tiles;
      kg_e = t / per;
      const int rem = t - kg_e * per;
      n_tile = rem / a.m_tiles;
      r0 = (rem - n_tile * a.m_tiles) * BM;
      mrows = min(BM, a.M - r0);
      a_r0 = c_r0 = r0;
      kg_k0 = __builtin_amdgcn_readfirstlane(a.kpre[kg_e]);
      kg_k = __builtin_amdgcn_readfirstlane(a.kpre[kg_e + 1]) - kg_k0;
      nk = kg_k / KE;
      // accumulating (a later round of the multi-round backward): an expert
      // with no rows adds nothing, so its tiles are skipped (K-grouped
      // launches take the static tile order, whose next_tile touches no LDS,
      // so skipping the tile's barriers is safe)
      if constexpr (EPI == EPI_F32_ADD)
        if (kg_k == 0) continue;
    } else {
      // Groups of DENSE_GM M panels: inside a group the tiles go N tile by N
      // tile with the M panel fastest, so a window of concurrent tiles spans a
      // few M panels and a few N tiles and both operands are re-read rarely.
      int td = t;
      if (a.ksplit > 1) {
        const int per = a.m_tiles * a.n_tiles;
        const int ch = (nk_all + a.ksplit - 1) / a.ksplit;
        ks = td / per;
        td -= ks * per;
        kt0 = ks * ch;
        nk = max(0, min(ch, nk_all - kt0));
      }
      const int g = td / (DENSE_GM * a.n_tiles);
      const int gm = min(DENSE_GM, a.m_tiles - g * DENSE_GM);
      const int r = td - g * DENSE_GM * a.n_tiles;
      n_tile = r / gm;
      r0 = (g * DENSE_GM + (r - n_tile * gm)) * BM;
      mrows = min(BM, a.M - r0);
      a_r0 = c_r0 = r0;
      if constexpr (F8 != F8_NONE) {
        dq_b = 1.0f / (A_SMUL * a.a_scale[0] * a.b_scale[0]);
        if constexpr (SWG) dq_b2 = 1.0f / (A_SMUL * a.a_scale[0] * a.b2_scale[0]);
        if constexpr (SEG_DQ) dq_b2 = 1.0f / (A_SMUL * a.a2_scale[0] * a.b2_scale[0]);
      }
    }
    const int n0 = SWG ? n_tile * (BN / 2) : n_tile * BN;   // first output col
    const int nrows = min(SWG ? BN / 2 : BN, a.N - n0);     // valid B rows per matrix

    // per-lane A row byte offsets for GATHER (fixed over the K loop)
    uint32_t a_goff[A_INS];
    if constexpr (GATHER) {
#pragma unroll
      for (int i = 0; i < A_INS; ++i) {
        const int rl = (wave + i * NW) * RPI + lrow;
        uint32_t off = 0x80000000u;                      // out of range -> zeros
        if (rl < mrows) {
          int src = a.row_token[r0 + rl];
          if ((unsigned)src >= (unsigned)a.M) src = 0;   // malformed metadata: row 0
          off = (uint32_t)((int64_t)src * a.seg[0].lda * ES);
        }
        a_goff[i] = off;
      }
    }

    // Buffer descriptors of every K segment for this tile (scalar registers).
    __amdgpu_buffer_rsrc_t rA[NSEG], rB[NSEG], rU[NSEG];
    static_for<0, NSEG>([&](auto sc) {
      constexpr int S = decltype(sc)::value;
      const GemmSeg& g = a.seg[S];
      const char* A = (const char*)g.A;
      const char* B = (const char*)g.B;
      if constexpr (GATHER) {
        rA[S] = make_rsrc(A, (int64_t)a.M * g.lda * ES);
      } else if constexpr (KG) {
        // rows of this tile, columns [kg_k0, kg_k0 + kg_k) of each
        rA[S] = make_rsrc(A + ((int64_t)a_r0 * g.lda + kg_k0) * ES,
                          mrows > 0 ? ((int64_t)(mrows - 1) * g.lda + kg_k) * ES : 0);
      } else {
        rA[S] = make_rsrc(A + (int64_t)a_r0 * g.lda * ES, (int64_t)mrows * g.lda * ES);
      }
      if constexpr (KG)
        rB[S] = make_rsrc(B + ((int64_t)n0 * g.ldb + kg_k0) * ES,
                          nrows > 0 ? ((int64_t)(nrows - 1) * g.ldb + kg_k) * ES : 0);
      else
        rB[S] = make_rsrc(B + b_off + (int64_t)n0 * g.ldb * ES, (int64_t)nrows * g.ldb * ES);
      if constexpr (SWG)
        rU[S] = make_rsrc((const char*)g.B2 + b_off + (int64_t)n0 * g.ldb * ES,
                          (int64_t)nrows * g.ldb * ES);
    });

    // DMA loads of stage kt.  A stage's instructions are split into DPART
    // parts (instruction i belongs to part i % DPART; PART < 0 = all), issued
    // at the first DPART MFMA sub-steps of the stage being computed instead of
    // stalling in one block.  With a two-stage ring a prefetched stage has
    // only the current stage's compute to land in, so its loads go out in the
    // first half of it (spread over all four sub-steps, the last part arrives
    // late: 6% slower on the MFMA-bound grouped GEMMs).
    constexpr int NPART = F8 ? BK / 32 : BK / 16;   // MFMA sub-steps per stage
    constexpr int DPART = NSTAGE == 2 && NPART > 2 ? 2 : NPART;
    auto issue_seg = [&](auto seg_c, int kt, int k0, auto part_c) {
      constexpr int S = decltype(seg_c)::value;
      constexpr int PART = decltype(part_c)::value;
      uint4* sa = smem + (kt % NSTAGE) * STAGE;
      uint4* sb = sa + BM * KCH;
      const uint32_t kbytes = (uint32_t)k0 * ES + (uint32_t)lchunk * 16;
#pragma unroll
      for (int i = 0; i < A_INS; ++i) {
        if (!(PART < 0 || i % DPART == PART)) continue;
        if constexpr (GATHER) {
          dma16(rA[S], sa + (wave + i * NW) * 64, a_goff[i] + kbytes);
        } else {
          const int rl = (wave + i * NW) * RPI + lrow;
          dma16(rA[S], sa + (wave + i * NW) * 64, (uint32_t)rl * lda2[S] + kbytes);
        }
      }
#pragma unroll
      for (int i = 0; i < B_INS; ++i) {
        if (!(PART < 0 || (A_INS + i) % DPART == PART)) continue;
        const int rho0 = (wave + i * NW) * RPI;     // a DMA group never straddles a 32-row block
        if constexpr (SWG) {
          const int hrow = (rho0 >> 6) * 32 + (rho0 & 31) + lrow;
          const uint32_t off = (uint32_t)hrow * ldb2[S] + kbytes;
          if ((rho0 >> 5) & 1) dma16<BNT>(rU[S], sb + rho0 * KCH, off);
          else dma16<BNT>(rB[S], sb + rho0 * KCH, off);
        } else {
          dma16<BNT>(rB[S], sb + rho0 * KCH, (uint32_t)(rho0 + lrow) * ldb2[S] + kbytes);
        }
      }
    };
    auto issue = [&](int kt, auto part_c) {   // kt: the tile's stage (its ring slot)
      int k0 = (kt0 + kt) * KE;
      if constexpr (NSEG == 1) {
        issue_seg(std::integral_constant<int, 0>{}, kt, k0, part_c);
      } else {
        if (k0 < kseg[0]) {
          issue_seg(std::integral_constant<int, 0>{}, kt, k0, part_c);
        } else {
          k0 -= kseg[0];
          if (NSEG == 2 || k0 < kseg[1]) {
            issue_seg(std::integral_constant<int, 1>{}, kt, k0, part_c);
          } else {
            issue_seg(std::integral_constant<int, NSEG - 1>{}, kt, k0 - kseg[1], part_c);
          }
        }
      }
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

#pragma unroll
    for (int p = 0; p < NSTAGE - 1; ++p)
      if (p < nk) issue(p, std::integral_constant<int, -1>{});

    // The K loop, specialised on how many of this wave's 32-row blocks hold
    // valid rows (uniform per tile), so every variant is a static, freely
    // scheduled sequence of LDS reads and MFMAs.  All variants run the same
    // waits, barriers and DMA issues, so waves in different variants stay in
    // step.
    auto mainloop = [&](auto nact_c) {
      constexpr int NACT = decltype(nact_c)::value;
      for (int kt = 0; kt < nk; ++kt) {
        // stage kt is complete once at most (stages issued after it) * LPS loads remain
        const int ahead = min(NSTAGE - 2, nk - 1 - kt);
        if constexpr (NSTAGE == 4) {
          if (ahead >= 2) wait_vmcnt<2 * LPS>();
          else if (ahead == 1) wait_vmcnt<LPS>();
          else wait_vmcnt<0>();
        } else if constexpr (NSTAGE == 3) {
          if (ahead >= 1) wait_vmcnt<LPS>();
          else wait_vmcnt<0>();
        } else {
          wait_vmcnt<0>();
        }
        lds_barrier();     // every wave's DMA for stage kt landed; stage kt-1 fully consumed
        if constexpr (SEG_DQ) {
          // the first segment's products are complete: bring them to the
          // second segment's scale, so that the final dq_b2 divides each
          // segment by its own scales
          if ((kt0 + kt) * KE == kseg[0]) {
            const float ratio = dq_b / dq_b2;
#pragma unroll
            for (int i = 0; i < NACT; ++i)
#pragma unroll
              for (int j = 0; j < TN; ++j) acc[i][j] *= ratio;
          }
        }
        const bool prefetch = kt + NSTAGE - 1 < nk;
        const uint4* sa = smem + (kt % NSTAGE) * STAGE;
        const uint4* sb = sa + BM * KCH;
        static_for<0, NPART>([&](auto kk_c) {
          constexpr int kk = decltype(kk_c)::value;
          if constexpr (kk < DPART)
            if (prefetch) issue(kt + NSTAGE - 1, kk_c);
          if constexpr (NACT > 0 && F8 == F8_NONE) {
            // rows 32 (i WM + wrow) + fr all have the same swizzle as row fr
            const int ch = (kk * 2 + fq) ^ swz<KCH>(fr);
            bf16x8 bfr[TN], afr[NACT];
#pragma unroll
            for (int j = 0; j < TN; ++j)
              bfr[j] = __builtin_bit_cast(bf16x8, sb[(wn0 + j * 32 + fr) * KCH + ch]);
#pragma unroll
            for (int i = 0; i < NACT; ++i)
              afr[i] = __builtin_bit_cast(bf16x8, sa[((i * WM + wrow) * 32 + fr) * KCH + ch]);
#pragma unroll
            for (int i = 0; i < NACT; ++i)
#pragma unroll
              for (int j = 0; j < TN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afr[i], bfr[j], acc[i][j],
                                                                    0, 0, 0);
          } else if constexpr (NACT > 0) {
            // FP8: a sub-step is 64 K values = 4 chunks; lane half fq takes
            // chunks 2 fq and 2 fq + 1 (32 contiguous bytes of its row)
            const int c0 = (kk * 4 + fq * 2) ^ swz<KCH>(fr);
            const int c1 = (kk * 4 + fq * 2 + 1) ^ swz<KCH>(fr);
            i32x8 bfr[TN], afr[NACT];
#pragma unroll
            for (int j = 0; j < TN; ++j) {
              const uint4 lo = sb[(wn0 + j * 32 + fr) * KCH + c0];
              const uint4 hi = sb[(wn0 + j * 32 + fr) * KCH + c1];
              bfr[j] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                             (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            }
#pragma unroll
            for (int i = 0; i < NACT; ++i) {
              const uint4 lo = sa[((i * WM + wrow) * 32 + fr) * KCH + c0];
              const uint4 hi = sa[((i * WM + wrow) * 32 + fr) * KCH + c1];
              afr[i] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                             (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            }
#pragma unroll
            for (int i = 0; i < NACT; ++i)
#pragma unroll
              for (int j = 0; j < TN; ++j)
                // A format 0 (E4M3) or 1 (E5M2), B format 0 (E4M3); block scales 2^0
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    afr[i], bfr[j], acc[i][j], F8 == F8_E5M2_A ? 1 : 0, 0, 0, 127, 0, 127);
          }
        });
      }
    };
    const int nblk = (mrows + 31) / 32;   // valid 32-row blocks of the tile
    const int nact = nblk > wrow ? min(TM, (nblk - wrow + WM - 1) / WM) : 0;
    static_assert(TM <= 16, "row blocks");
    switch (nact) {
#define MOE_NACT_CASE(n) \
      case n: if constexpr (n <= TM) mainloop(std::integral_constant<int, n>{}); break;
      MOE_NACT_CASE(0) MOE_NACT_CASE(1) MOE_NACT_CASE(2) MOE_NACT_CASE(3) MOE_NACT_CASE(4)
      MOE_NACT_CASE(5) MOE_NACT_CASE(6) MOE_NACT_CASE(7) MOE_NACT_CASE(8) MOE_NACT_CASE(9)
      MOE_NACT_CASE(10) MOE_NACT_CASE(11) MOE_NACT_CASE(12) MOE_NACT_CASE(13)
      MOE_NACT_CASE(14) MOE_NACT_CASE(15) MOE_NACT_CASE(16)
#undef MOE_NACT_CASE
      default: break;
    }

    // ---- epilogue: in a 32x32 block, lane l holds column l & 31 and, in
    // register r, row 8 * (r / 4) + 4 * (l / 32) + r % 4 ----
    const float oscale = Q8 ? a.out_scale[0] : 1.f;
    // GBQ8: the E5M2 scales of dg and du (128 s, exact)
    const float q5_dg = GBQ8 ? E5M2_OVER_E4M3 * a.out_scale[1] : 1.f;
    const float q5_du = GBQ8 ? E5M2_OVER_E4M3 * a.out_scale[2] : 1.f;
    // FP8 with two K segments: the accumulators hold the second segment's scale
    const float dq_out = SEG_DQ ? dq_b2 : dq_b;
    // KG: the expert's block; split K: the chunk's partial result
    const int64_t c_off = KG ? (int64_t)kg_e * a.c_expert_stride : (int64_t)ks * a.c_split;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rl = (i * WM + wrow) * 32 + 8 * (r >> 2) + 4 * fq + (r & 3);
        if (rl >= mrows) continue;
        const int64_t row = c_r0 + rl;
        if constexpr (SWG) {
#pragma unroll
          for (int j = 0; j < TN; j += 2) {
            const int cl = ((wn0 + j * 32) >> 6) * 32 + fr;
            if (cl < nrows) {
              const float g = acc[i][j][r] * dq_b, u = acc[i][j + 1][r] * dq_b2;
              // silu(g) = g sigmoid(g), the sigmoid's reciprocal on the
              // hardware's v_rcp_f32 (<= 1 ulp) instead of an IEEE division
              // (~10 instructions per output while the matrix cores idle:
              // 1.5% of the compute-bound gate/up); the backward's recompute
              // below uses the same expression, so its h is the forward's
              const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-g));
              const uint16_t hb = f32_to_bf16_rne(g * sg * u);
              if constexpr (epi_gu_bwd(EPI)) {
                const int64_t o = row * a.ldc + n0 + cl;
                // the random stream's element index is the row's place in the
                // permutation order (r0 + rl), also when the rows sit in a
                // round buffer (h_side 1)
                const int64_t osr = (a.h_side == 1 ? (int64_t)(r0 + rl) : row) * a.ldc + n0 + cl;
                const float dh = a.aux_g[o];
                const float dg = dh * u * (sg * (1.0f + g * (1.0f - sg)));
                const float du = dh * (g * sg);
                if (a.sr) {
                  ((uint16_t*)a.C)[o] = f32_to_bf16_sr(dg, a.sr_key_c, (uint64_t)osr);
                  ((uint16_t*)a.C2)[o] = f32_to_bf16_sr(du, a.sr_key_c2, (uint64_t)osr);
                } else {
                  ((uint16_t*)a.C)[o] = f32_to_bf16_rne(dg);
                  ((uint16_t*)a.C2)[o] = f32_to_bf16_rne(du);
                }
                ((uint16_t*)a.C3)[o] = hb;
                if constexpr (GBQ8) {
                  amax_dg = fmaxf(amax_dg, fabsf(dg));
                  amax_du = fmaxf(amax_du, fabsf(du));
                  ((uint8_t*)a.C4)[o] = f32_to_e5m2(dg * q5_dg, a.sr, a.sr_key_c4, (uint64_t)osr);
                  ((uint8_t*)a.C5)[o] = f32_to_e5m2(du * q5_du, a.sr, a.sr_key_c5, (uint64_t)osr);
                }
              } else if constexpr (EPI == EPI_SWIGLU_Q8) {
                const float hv = bf16_to_f32(hb);
                amax_run = fmaxf(amax_run, fabsf(hv));
                ((uint8_t*)a.C)[row * a.ldc + n0 + cl] = f32_to_e4m3_sat(hv * oscale);
              } else {
                ((uint16_t*)a.C)[row * a.ldc + n0 + cl] = hb;
              }
            }
          }
        } else {
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const int cl = wn0 + j * 32 + fr;
            if (cl >= nrows) continue;
            const int col = n0 + cl;
            const float val = acc[i][j][r] * dq_out;
            if constexpr (EPI == EPI_BF16) {
              ((uint16_t*)a.C)[row * a.ldc + col] = f32_to_bf16_rne(val);
            } else if constexpr (EPI == EPI_Q8) {
              const float zv = bf16_to_f32(f32_to_bf16_rne(val));
              amax_run = fmaxf(amax_run, fabsf(zv));
              ((uint8_t*)a.C)[row * a.ldc + col] = f32_to_e4m3_sat(zv * oscale);
            } else if constexpr (EPI == EPI_F32_BIAS) {
              ((float*)a.C)[c_off + row * a.ldc + col] = val + (a.bias ? a.bias[col] : 0.f);
            } else if constexpr (EPI == EPI_F32_ADD) {
              // C += result: every element is owned by one lane of one tile
              ((float*)a.C)[c_off + row * a.ldc + col] += val;
            } else {
              ((float*)a.C)[c_off + row * a.ldc + col] = val;
            }
          }
        }
      }
    }
    lds_barrier();     // LDS ring is reused by the next tile's first stages
  }
  if constexpr (Q8) {
    // wave maximum, then one atomic per wave (order-independent: max)
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) amax_run = fmaxf(amax_run, __shfl_xor(amax_run, o));
    if (lane == 0 && amax_run > 0.f) atomicMax(a.amax, __float_as_uint(amax_run));
  }
  if constexpr (GBQ8) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      amax_dg = fmaxf(amax_dg, __shfl_xor(amax_dg, o));
      amax_du = fmaxf(amax_du, __shfl_xor(amax_du, o));
    }
    if (lane == 0 && amax_dg > 0.f) atomicMax(a.amax + 1, __float_as_uint(amax_dg));
    if (lane == 0 && amax_du > 0.f) atomicMax(a.amax + 2, __float_as_uint(amax_du));
  }
}

// Compute units of the current device (cached per device).
int device_cu_count();

// Workgroups for a persistent GEMM: one per CU, at most one per tile, a
// multiple of 8 (the XCD count).
inline int persistent_grid(int64_t tiles_upper_bound) {
  int64_t g = tiles_upper_bound < device_cu_count() ? tiles_upper_bound : device_cu_count();
  if (g < 8) g = 8;
  return (int)((g + 7) / 8 * 8);
}

// Tile shapes used by the layer.  Eight waves per workgroup (two per SIMD):
// while one wave of a SIMD waits on LDS, a barrier or its DMA issue, the other
// keeps the matrix core busy (measured ~1.2x over four waves on MI355X).
//   Stream : 128 x 256, BK 64, 2 x 4 waves, 3 stages (144 KB), non-temporal
//            weight loads -- few rows per expert, HBM-bound weight streaming
//   Big    : 256 x 256, BK 64, 2 x 4 waves, 2 stages (128 KB) -- MFMA-bound
//   Mid    : 128 x 256, BK 64, 2 x 4 waves, 3 stages -- smaller dense GEMMs
//            and the routing GEMM at mid and small batches
//   Wide   : 256 x 192 (below)
//   StreamF8: 128 x 512 (below)
// (the dense GEMMs choose among Big, Wide and Mid by rounds x tile area /
// efficiency)
template <int BM, int BN, int BK, int WM, int WN, int NSTAGE, bool BNT>
struct TileCfg {
  static constexpr int bm = BM, bn = BN, bk = BK, wm = WM, wn = WN, nstage = NSTAGE;
  static constexpr bool bnt = BNT;
};
using TileStream = TileCfg<128, 256, 64, 2, 4, 3, true>;
using TileBig = TileCfg<256, 256, 64, 2, 4, 2, false>;
using TileMid = TileCfg<128, 256, 64, 2, 4, 3, false>;
// Wide : 256 x 192, BK 64, 4 x 2 waves (64 x 96 each), 2 stages (112 KB) --
//        e.g. M 4,096 x N 3,072: 256 tiles fill the chip exactly once, where
//        128 x 256 tiles take 1.5 waves
using TileWide = TileCfg<256, 192, 64, 4, 2, 2, false>;
// StreamF8 : 128 x 512, BK 64 (a 128-byte stage row holds 128 FP8 K values),
//            2 x 4 waves (64 x 128 each), 2 stages (160 KB, the whole LDS),
//            non-temporal weight loads -- the FP8 weight stream: a K step of
//            FP8 weights is half the bytes of a bf16 one, so the tile is twice
//            as wide as Stream to move as many weight bytes per tile (the
//            per-tile fixed cost of queue, tables and first-stage latency
//            then weighs as little as in bf16; measured 7.6 -> 5.7 ms for the
//            Base-1 gate/up at T = 4,096)
using TileStreamF8 = TileCfg<128, 512, 64, 2, 4, 2, true>;

template <class C, bool GROUPED, bool GATHER, int EPI, int NSEG = 1, int F8 = F8_NONE,
          bool KG = false>
hipError_t launch_gemm(const GemmArgs& a, int64_t tiles_upper_bound, hipStream_t s) {
  if (tiles_upper_bound <= 0) return hipSuccess;
  if (a.nseg != NSEG) return hipErrorInvalidValue;
  if (KG && a.queue != nullptr) return hipErrorInvalidValue;   // K-grouped: static tile order
  const int grid = persistent_grid(tiles_upper_bound);
  hipLaunchKernelGGL((gemm_kernel<C::bm, C::bn, C::bk, C::wm, C::wn, C::nstage, GROUPED, GATHER,
                                  EPI, C::bnt, NSEG, F8, KG>),
                     dim3(grid), dim3(64 * C::wm * C::wn), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
