// bf16 MFMA GEMM for gfx950:  C[m, n] = sum_k A[m, k] * B[n, k]  (fp32 accumulate)
//
// Both operands are K-contiguous ("NT" layout: every weight of the layer is
// stored [out, in]), so one 16-byte load along K feeds one MFMA operand lane.
//
// Work decomposition
//   * one workgroup per BM x BN output tile; 64*WM*WN threads; each wave owns a
//     (BM/WM) x (BN/WN) sub-tile built from 16x16 blocks of
//     v_mfma_f32_16x16x32_bf16 (A: 16 rows x 32 k, B: 32 k x 16 cols).
//   * K is walked in 64-wide stages, double-buffered in LDS.  The next stage's
//     global loads are issued before the current stage's MFMAs, so their
//     latency hides behind the math; rows are 128 bytes with the 16-byte
//     chunks XOR-swizzled by (row & 7) so fragment reads of 16 consecutive
//     rows hit distinct banks.
//   * up to three K segments (A_s, B_s, K_s) are chained in one accumulation:
//     used for the split-bf16 router (x against the hi/mid/lo parts of W_r) and
//     for the up-projection with the shared expert's down-projection appended
//     along K.
//   * GROUPED: the M dimension is the expert-ordered row list; tiles never
//     straddle two experts.  A device-side prefix of per-expert M-tile counts
//     maps a tile index to (expert, M-tile, N-tile) with no host sync.
//     GATHER: A row r is read from row row_token[r] (the permutation is fused
//     into the A load; no permuted copy of the activations is materialised).
//   * XCD-aware tile order: workgroup i runs on XCD i % 8, so consecutive
//     logical tiles are given to workgroups of the same XCD; tiles that share
//     an expert's weights or an activation panel then share that XCD's L2.
//   * EPI_SWIGLU: the B tile interleaves 16-row blocks of W_g and W_u for the
//     same output columns, so each lane holds gate and up values of the same
//     (row, column) and applies silu(g) * u before a single bf16 store.
#pragma once

#include "common.hpp"

namespace moe {

constexpr int GEMM_BK = 64;

enum GemmEpi { EPI_BF16 = 0, EPI_F32 = 1, EPI_F32_BIAS = 2, EPI_SWIGLU = 3 };

struct GemmSeg {
  const uint16_t* A;    // row r at A + (int64)arow(r) * lda
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
  int E;
  int64_t b_expert_stride;
  const int32_t* row_token;    // GATHER
  void* C;
  int64_t ldc;
  const float* bias;           // EPI_F32_BIAS
  int n_tiles;
  int m_tiles;                 // dense
  int grid;                    // launched workgroups, a multiple of 8
};

template <int BM, int BN, int WM, int WN, bool GROUPED, bool GATHER, int EPI>
__global__ __launch_bounds__(64 * WM * WN, 1) void gemm_kernel(GemmArgs a) {
  constexpr int NT = 64 * WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 16, TN = WTN / 16;
  constexpr int ROWS_PER_PASS = NT / 8;            // 8 chunks of 16 B per 64-wide row
  constexpr int A_CH = BM / ROWS_PER_PASS;
  constexpr int B_CH = BN / ROWS_PER_PASS;
  constexpr int STAGE = (BM + BN) * 8;             // uint4 slots per stage
  static_assert(BM % ROWS_PER_PASS == 0 && BN % ROWS_PER_PASS == 0, "tile/threads");
  static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile");
  static_assert(EPI != EPI_SWIGLU || WTN % 32 == 0, "swiglu pairs");
  __shared__ uint4 smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm0 = (wave / WN) * WTM;
  const int wn0 = (wave % WN) * WTN;

  // ---- which tile (XCD-aware order) ----
  const int bid = blockIdx.x;
  const int logical = (bid & 7) * (a.grid >> 3) + (bid >> 3);
  int m0, m_end, n_tile;
  int64_t b_off = 0;
  if constexpr (GROUPED) {
    const int total = a.tile_prefix[a.E] * a.n_tiles;
    if (logical >= total) return;
    int lo = 0, hi = a.E;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.tile_prefix[mid] * a.n_tiles <= logical) lo = mid; else hi = mid;
    }
    const int mt = a.tile_prefix[lo + 1] - a.tile_prefix[lo];
    const int rem = logical - a.tile_prefix[lo] * a.n_tiles;
    n_tile = rem / mt;
    const int m_local = rem - n_tile * mt;
    m0 = a.offsets[lo] + m_local * BM;
    m_end = min(m0 + BM, (int)a.offsets[lo + 1]);
    b_off = (int64_t)lo * a.b_expert_stride;
  } else {
    if (logical >= a.m_tiles * a.n_tiles) return;
    n_tile = logical / a.m_tiles;
    m0 = (logical - n_tile * a.m_tiles) * BM;
    m_end = min(m0 + BM, a.M);
  }

  // ---- per-thread load slots ----
  const int c = tid & 7;                 // 16-byte chunk along K inside a 64-wide stage
  const int r_base = tid >> 3;
  int arow[A_CH];
  bool aval[A_CH];
#pragma unroll
  for (int i = 0; i < A_CH; ++i) {
    const int r = m0 + r_base + i * ROWS_PER_PASS;
    aval[i] = r < m_end;
    int src = r;
    if constexpr (GATHER) {
      // a.M = rows of the gathered matrix; an out-of-range index (malformed
      // metadata) reads row 0 instead of faulting
      src = aval[i] ? a.row_token[r] : 0;
      if ((unsigned)src >= (unsigned)a.M) src = 0;
    }
    arow[i] = aval[i] ? src : 0;
  }
  int brow[B_CH];
  bool bval[B_CH], bsec[B_CH];
#pragma unroll
  for (int i = 0; i < B_CH; ++i) {
    const int nl = r_base + i * ROWS_PER_PASS;
    int col;
    if constexpr (EPI == EPI_SWIGLU) {
      col = n_tile * (BN / 2) + (nl >> 5) * 16 + (nl & 15);
      bsec[i] = (nl & 16) != 0;
    } else {
      col = n_tile * BN + nl;
      bsec[i] = false;
    }
    bval[i] = col < a.N;
    brow[i] = bval[i] ? col : 0;
  }

  int ktotal = 0;
#pragma unroll
  for (int s = 0; s < 3; ++s) if (s < a.nseg) ktotal += a.seg[s].K;
  const int nk = ktotal / GEMM_BK;

  uint4 ra[A_CH], rb[B_CH];
  auto load_stage = [&](int kt) {
    int s = 0, k0 = kt * GEMM_BK;
    if (a.nseg > 1 && k0 >= a.seg[0].K) { k0 -= a.seg[0].K; s = 1;
      if (a.nseg > 2 && k0 >= a.seg[1].K) { k0 -= a.seg[1].K; s = 2; } }
    const GemmSeg& g = a.seg[s];
    const int kc = k0 + c * 8;
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      ra[i] = make_uint4(0, 0, 0, 0);
      if (aval[i]) ra[i] = *(const uint4*)(g.A + (int64_t)arow[i] * g.lda + kc);
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      rb[i] = make_uint4(0, 0, 0, 0);
      const uint16_t* bm = (EPI == EPI_SWIGLU && bsec[i]) ? g.B2 : g.B;
      if (bval[i]) rb[i] = *(const uint4*)(bm + b_off + (int64_t)brow[i] * g.ldb + kc);
    }
  };
  auto store_stage = [&](int st) {
    uint4* sa = smem + st * STAGE;
    uint4* sb = sa + BM * 8;
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int r = r_base + i * ROWS_PER_PASS;
      sa[r * 8 + (c ^ (r & 7))] = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      const int r = r_base + i * ROWS_PER_PASS;
      sb[r * 8 + (c ^ (r & 7))] = rb[i];
    }
  };

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  load_stage(0);
  store_stage(0);
  __syncthreads();

  const int fr = lane & 15;          // row of the fragment inside a 16-row block
  const int fq = lane >> 4;          // which 8-wide k group (of 4) inside a 32-wide MFMA step
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load_stage(kt + 1);
    const uint4* sa = smem + cur * STAGE;
    const uint4* sb = sa + BM * 8;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int ch = (kk * 4 + fq) ^ (fr & 7);
      bf16x8 af[TM], bf[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = __builtin_bit_cast(bf16x8, sa[(wm0 + i * 16 + fr) * 8 + ch]);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bf[j] = __builtin_bit_cast(bf16x8, sb[(wn0 + j * 16 + fr) * 8 + ch]);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store_stage(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds rows 4*(lane>>4)+v, column lane&15 of each block ----
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = m0 + wm0 + i * 16 + fq * 4 + v;
      if (row >= m_end) continue;
      if constexpr (EPI == EPI_SWIGLU) {
        uint16_t* out = (uint16_t*)a.C + (int64_t)row * a.ldc;
#pragma unroll
        for (int j = 0; j < TN; j += 2) {
          const int col = n_tile * (BN / 2) + ((wn0 + j * 16) >> 5) * 16 + fr;
          if (col < a.N) {
            const float g = acc[i][j][v], u = acc[i][j + 1][v];
            out[col] = f32_to_bf16_rne(g / (1.0f + __expf(-g)) * u);
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int col = n_tile * BN + wn0 + j * 16 + fr;
          if (col >= a.N) continue;
          const float val = acc[i][j][v];
          if constexpr (EPI == EPI_BF16) {
            ((uint16_t*)a.C)[(int64_t)row * a.ldc + col] = f32_to_bf16_rne(val);
          } else if constexpr (EPI == EPI_F32_BIAS) {
            ((float*)a.C)[(int64_t)row * a.ldc + col] = val + (a.bias ? a.bias[col] : 0.f);
          } else {
            ((float*)a.C)[(int64_t)row * a.ldc + col] = val;
          }
        }
      }
    }
  }
}

// Workgroups to launch for a grouped GEMM over T*k rows and E experts: an
// upper bound of sum_e ceil(M_e / BM) over any routing, times the N tiles,
// rounded up to a multiple of 8 (the XCD count).
inline int grouped_grid(int64_t rows, int E, int BM, int n_tiles, int* m_tile_bound) {
  const int64_t nonempty = rows < E ? rows : E;
  const int64_t mt = (rows + nonempty * (BM - 1)) / BM;
  *m_tile_bound = (int)mt;
  const int64_t g = mt * n_tiles;
  return (int)(((g + 7) / 8) * 8);
}

template <int BM, int BN, int WM, int WN, bool GROUPED, bool GATHER, int EPI>
hipError_t launch_gemm(GemmArgs a, hipStream_t s) {
  if (a.grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, GROUPED, GATHER, EPI>), dim3(a.grid),
                     dim3(64 * WM * WN), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
