// bf16 MFMA GEMM for gfx950:  C[m, n] = sum_k A[m, k] * B[n, k]  (fp32 accumulate)
//
// Both operands are K-contiguous ("NT" layout: every weight of the layer is
// stored [out, in]), so one 16-byte load along K feeds one MFMA operand lane.
//
// Design
//   * Persistent, XCD-balanced: the grid is a multiple of 8 workgroups, one per
//     CU; workgroup b runs on XCD b % 8.  The tile list (known only on the
//     device for grouped GEMMs) is cut into 8 contiguous ranges, one per XCD,
//     and the workgroups of an XCD walk their range round-robin, so the CUs of
//     one XCD work on neighbouring tiles at the same time: tiles that share an
//     expert's weight panel or an activation panel share that XCD's L2.
//   * Operands go global -> LDS directly (buffer_load_dwordx4 ... lds), no
//     register staging, in an NSTAGE-deep ring of 64-wide K stages, so
//     NSTAGE-1 stages of loads are in flight while the MFMAs run.  Each load
//     instruction fills 8 rows x 128 bytes; the 16-byte chunks of a row are
//     XOR-swizzled by (row & 7) so that fragment reads of 16 consecutive rows
//     spread over the LDS banks.  Rows past the end of the matrix (ragged
//     expert segments, N tails) are out of the buffer descriptor's range and
//     load as zeros.
//   * Each wave owns a (BM/WM) x (BN/WN) sub-tile of 16x16 blocks of
//     v_mfma_f32_16x16x32_bf16; 16-row blocks past the tile's last valid row
//     are skipped (a small expert costs MFMA time in proportion to its rows).
//   * Up to three K segments (A_s, B_s, K_s) chain in one accumulation: the
//     split-bf16 router (x against the hi/mid/lo parts of W_r) and the
//     up-projection with the shared expert's down-projection appended along K.
//   * GROUPED: M is the expert-ordered row list; tiles never straddle two
//     experts.  Device tables (prefix of per-expert M-tile counts and the
//     expert of every M-tile) map a tile index to (expert, M-tile, N-tile)
//     with no host sync.  Order: expert, then N tile, then M tile, so M tiles
//     of one expert that read the same weight tile run side by side.
//     GATHER: A row r is row row_token[r] of the activations (the token
//     permutation is fused into the A load).
//   * EPI_SWIGLU: the B tile interleaves 16-row blocks of W_g and W_u for the
//     same output columns, so each lane holds the gate and up values of the
//     same (row, column) and applies silu(g) * u before one bf16 store.
#pragma once

#include <type_traits>

#include "common.hpp"

namespace moe {

constexpr int GEMM_BK = 64;
constexpr uint32_t RSRC_WORD3 = 0x00020000u;   // raw buffer, 32-bit data format (gfx9)

enum GemmEpi { EPI_BF16 = 0, EPI_F32 = 1, EPI_F32_BIAS = 2, EPI_SWIGLU = 3 };

struct GemmSeg {
  const uint16_t* A;    // row r at A + arow(r) * lda
  const uint16_t* B;    // row n at B + n * ldb (+ expert * b_expert_stride)
  const uint16_t* B2;   // EPI_SWIGLU: the up matrix (B holds the gate matrix)
  int64_t lda, ldb;
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
  void* C;
  int64_t ldc;
  const float* bias;           // EPI_F32_BIAS
  int n_tiles;
  int m_tiles;                 // dense
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  if (bytes < 0) bytes = 0;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, RSRC_WORD3);
}

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint4* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 16, voff, 0, 0, 0);
}

// Workgroup barrier that orders LDS reads and writes only.  __syncthreads()
// (and any compiler fence that covers LDS) also waits for every outstanding
// vector-memory access, LDS DMA included, i.e. it would drain the whole load
// ring; the ring's completion is tracked with explicit vmcnt waits instead.
// The "memory" clobber keeps the compiler from moving memory accesses across.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int BM, int BN, int WM, int WN, int NSTAGE, bool GROUPED, bool GATHER, int EPI>
__global__ __launch_bounds__(64 * WM * WN, 1) void gemm_kernel(GemmArgs a) {
  constexpr int NW = WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 16, TN = WTN / 16;
  constexpr int A_INS = BM / 8 / NW;               // DMA instructions per wave per stage
  constexpr int B_INS = BN / 8 / NW;
  constexpr int LPS = A_INS + B_INS;
  constexpr int STAGE = (BM + BN) * 8;             // 16-byte slots per stage
  static_assert(BM % (8 * NW) == 0 && BN % (8 * NW) == 0, "tile / waves");
  static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile");
  static_assert(EPI != EPI_SWIGLU || WTN % 32 == 0, "swiglu pairs");
  static_assert(NSTAGE >= 2 && NSTAGE <= 4 && LPS * (NSTAGE - 2) < 64, "stages");
  __shared__ uint4 smem[NSTAGE * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
  const int wm0 = (wave / WN) * WTM;
  const int wn0 = (wave % WN) * WTN;
  const int lrow = lane >> 3;                      // row inside an 8-row DMA group
  const int lchunk = (lane & 7) ^ lrow;            // chunk this lane fetches (swizzle)
  const int fr = lane & 15;                        // fragment row inside a 16-row block
  const int fq = lane >> 4;                        // 8-wide k group inside a 32-wide step

  int total;
  if constexpr (GROUPED) total = a.tile_prefix[a.E] * a.n_tiles;
  else total = a.m_tiles * a.n_tiles;
  const int xcd = blockIdx.x & 7;
  const int nj = gridDim.x >> 3;
  const int t_begin = (int)((int64_t)total * xcd / 8);
  const int t_end = (int)((int64_t)total * (xcd + 1) / 8);

  int ktotal = 0;
#pragma unroll
  for (int s = 0; s < 3; ++s) if (s < a.nseg) ktotal += a.seg[s].K;
  const int nk = ktotal / GEMM_BK;

  for (int t = t_begin + (blockIdx.x >> 3); t < t_end; t += nj) {
    // ---- decode the tile ----
    int r0, mrows, n_tile;
    int64_t b_off = 0;
    if constexpr (GROUPED) {
      const int e = a.tile_expert[t / a.n_tiles];
      const int p0 = a.tile_prefix[e];
      const int mt = a.tile_prefix[e + 1] - p0;
      const int rem = t - p0 * a.n_tiles;
      n_tile = rem / mt;
      const int m_local = rem - n_tile * mt;
      r0 = a.offsets[e] + m_local * BM;
      mrows = min(BM, a.offsets[e + 1] - r0);
      b_off = (int64_t)e * a.b_expert_stride;
    } else {
      n_tile = t / a.m_tiles;
      r0 = (t - n_tile * a.m_tiles) * BM;
      mrows = min(BM, a.M - r0);
    }
    const int n0 = EPI == EPI_SWIGLU ? n_tile * (BN / 2) : n_tile * BN;   // first output col
    const int nrows = min(EPI == EPI_SWIGLU ? BN / 2 : BN, a.N - n0);     // valid B rows per matrix

    // per-lane A row byte offsets for GATHER (fixed over the K loop)
    uint32_t a_goff[A_INS];
    if constexpr (GATHER) {
#pragma unroll
      for (int i = 0; i < A_INS; ++i) {
        const int rl = (wave + i * NW) * 8 + lrow;
        uint32_t off = 0x80000000u;                      // out of range -> zeros
        if (rl < mrows) {
          int src = a.row_token[r0 + rl];
          if ((unsigned)src >= (unsigned)a.M) src = 0;   // malformed metadata: row 0
          off = (uint32_t)((int64_t)src * a.seg[0].lda * 2);
        }
        a_goff[i] = off;
      }
    }

    auto issue = [&](int kt) {
      int s = 0, k0 = kt * GEMM_BK;
      if (a.nseg > 1 && k0 >= a.seg[0].K) {
        k0 -= a.seg[0].K; s = 1;
        if (a.nseg > 2 && k0 >= a.seg[1].K) { k0 -= a.seg[1].K; s = 2; }
      }
      const GemmSeg& g = a.seg[s];
      uint4* sa = smem + (kt % NSTAGE) * STAGE;
      uint4* sb = sa + BM * 8;
      const uint32_t kbytes = (uint32_t)(k0 + lchunk * 8) * 2;
      if constexpr (GATHER) {
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(g.A, (int64_t)a.M * g.lda * 2);
#pragma unroll
        for (int i = 0; i < A_INS; ++i) dma16(ra, sa + (wave + i * NW) * 64, a_goff[i] + kbytes);
      } else {
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(g.A + (int64_t)r0 * g.lda,
                                                   (int64_t)mrows * g.lda * 2);
#pragma unroll
        for (int i = 0; i < A_INS; ++i) {
          const int rl = (wave + i * NW) * 8 + lrow;
          dma16(ra, sa + (wave + i * NW) * 64, (uint32_t)(rl * g.lda * 2) + kbytes);
        }
      }
      if constexpr (EPI == EPI_SWIGLU) {
        const __amdgpu_buffer_rsrc_t rg = make_rsrc(g.B + b_off + (int64_t)n0 * g.ldb,
                                                   (int64_t)nrows * g.ldb * 2);
        const __amdgpu_buffer_rsrc_t ru = make_rsrc(g.B2 + b_off + (int64_t)n0 * g.ldb,
                                                   (int64_t)nrows * g.ldb * 2);
#pragma unroll
        for (int i = 0; i < B_INS; ++i) {
          const int rho0 = (wave + i * NW) * 8;
          const int hrow = (rho0 >> 5) * 16 + (rho0 & 15) + lrow;
          const uint32_t off = (uint32_t)(hrow * g.ldb * 2) + kbytes;
          if ((rho0 >> 4) & 1) dma16(ru, sb + rho0 * 8, off);
          else dma16(rg, sb + rho0 * 8, off);
        }
      } else {
        const __amdgpu_buffer_rsrc_t rb = make_rsrc(g.B + b_off + (int64_t)n0 * g.ldb,
                                                   (int64_t)nrows * g.ldb * 2);
#pragma unroll
        for (int i = 0; i < B_INS; ++i) {
          const int rho0 = (wave + i * NW) * 8;
          dma16(rb, sb + rho0 * 8, (uint32_t)((rho0 + lrow) * g.ldb * 2) + kbytes);
        }
      }
    };

    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int p = 0; p < NSTAGE - 1; ++p)
      if (p < nk) issue(p);

    // The K loop, specialised on how many of this wave's 16-row blocks hold
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
        if (kt + NSTAGE - 1 < nk) issue(kt + NSTAGE - 1);
        if constexpr (NACT > 0) {
          const uint4* sa = smem + (kt % NSTAGE) * STAGE;
          const uint4* sb = sa + BM * 8;
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
            const int ch = (kk * 4 + fq) ^ (fr & 7);
            bf16x8 bfr[TN], afr[NACT];
#pragma unroll
            for (int j = 0; j < TN; ++j)
              bfr[j] = __builtin_bit_cast(bf16x8, sb[(wn0 + j * 16 + fr) * 8 + ch]);
#pragma unroll
            for (int i = 0; i < NACT; ++i)
              afr[i] = __builtin_bit_cast(bf16x8, sa[(wm0 + i * 16 + fr) * 8 + ch]);
#pragma unroll
            for (int i = 0; i < NACT; ++i)
#pragma unroll
              for (int j = 0; j < TN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr[i], bfr[j], acc[i][j],
                                                                    0, 0, 0);
          }
        }
      }
    };
    const int nact = max(0, min(TM, (mrows - wm0 + 15) / 16));
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

    // ---- epilogue: lane holds rows 4*(lane>>4)+v, column lane&15 of each block ----
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int rl = wm0 + i * 16 + fq * 4 + v;
        if (rl >= mrows) continue;
        const int64_t row = r0 + rl;
        if constexpr (EPI == EPI_SWIGLU) {
          uint16_t* out = (uint16_t*)a.C + row * a.ldc;
#pragma unroll
          for (int j = 0; j < TN; j += 2) {
            const int cl = ((wn0 + j * 16) >> 5) * 16 + fr;
            if (cl < nrows) {
              const float g = acc[i][j][v], u = acc[i][j + 1][v];
              out[n0 + cl] = f32_to_bf16_rne(g / (1.0f + __expf(-g)) * u);
            }
          }
        } else {
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const int cl = wn0 + j * 16 + fr;
            if (cl >= nrows) continue;
            const int col = n0 + cl;
            const float val = acc[i][j][v];
            if constexpr (EPI == EPI_BF16) {
              ((uint16_t*)a.C)[row * a.ldc + col] = f32_to_bf16_rne(val);
            } else if constexpr (EPI == EPI_F32_BIAS) {
              ((float*)a.C)[row * a.ldc + col] = val + (a.bias ? a.bias[col] : 0.f);
            } else {
              ((float*)a.C)[row * a.ldc + col] = val;
            }
          }
        }
      }
    }
    lds_barrier();     // LDS ring is reused by the next tile's first stages
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

template <int BM, int BN, int WM, int WN, int NSTAGE, bool GROUPED, bool GATHER, int EPI>
hipError_t launch_gemm(const GemmArgs& a, int64_t tiles_upper_bound, hipStream_t s) {
  if (tiles_upper_bound <= 0) return hipSuccess;
  const int grid = persistent_grid(tiles_upper_bound);
  hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, NSTAGE, GROUPED, GATHER, EPI>), dim3(grid),
                     dim3(64 * WM * WN), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
