// Latent down-projection and the routed SwiGLU experts as grouped bf16 MFMA
// GEMMs ("The Training and RL Infrastructure Behind MAI-Thinking-1": model
// table — shared down-projection before dispatch, expert FFN, SwiGLU;
// section 3 "Custom kernels" — grouped GEMMs for MoE; "Frontier Pre-training
// at Microsoft AI", "Reducing per-expert overhead" — grouped computation per
// expert group, device-resident token metadata).  Also the Base-2 shared
// expert's gate/up half, on the full hidden width ("MAI-Base-2: Microsoft's
// 2.8T base model...", section "The model").
#include <atomic>

#include "launch.hpp"
#include "gemm.hpp"
#include "scan.hpp"

namespace moe {

ExpertGemmPlan plan_expert_gemms(int64_t rows, int E) {
  // Few rows per expert (small batches, weight streaming): 128-row M tiles
  // usually hold an expert's rows in one tile, so each weight byte is read
  // from HBM once; a 3-deep load ring keeps two 48 KB stages in flight per CU.
  // Otherwise (compute-bound) 256 x 256 tiles.
  const int64_t avg = rows / (E > 0 ? E : 1);
  ExpertGemmPlan p;
  p.bm_gate_up = avg <= 128 ? 128 : 256;
  p.bm_down = p.bm_gate_up;
  return p;
}

// Dense GEMM tile choice by the cost rounds x tile area / efficiency (rounds
// = tiles over CUs, rounded up; areas 4 : 3 : 2 for 256 x 256 : 256 x 192 :
// 128 x 256, efficiencies 1 : 0.94 : 0.83 -- a smaller tile reads more operand
// bytes per MFMA), ties to the larger tile.  E.g. M 4,096 x N 3,072: 256 x 192
// (one round of 256 tiles); M 4,096 x N 6,656: 256 x 256 (416 tiles, two
// rounds) rather than 128 x 256 (832 tiles, four); M 16,384 x N 8,704: 256 x
// 256 (9 rounds) rather than 128 x 256 (17).
enum DenseTile { DT_BIG, DT_WIDE, DT_MID };
static DenseTile dense_tile(int64_t M, int64_t Ncols, bool wide_ok) {
  const int64_t cus = device_cu_count();
  auto rounds = [&](int bm, int bn) { return ceil_div(ceil_div(M, bm) * ceil_div(Ncols, bn), cus); };
  const int64_t big = 40 * rounds(256, 256), wide = 32 * rounds(256, 192),
                mid = 24 * rounds(128, 256);
  if (big <= mid && (!wide_ok || big <= wide)) return DT_BIG;
  if (wide_ok && wide <= mid) return DT_WIDE;
  return DT_MID;
}

template <class C, int EPI, int NSEG>
static hipError_t dense_gemm(GemmArgs a, int64_t M, hipStream_t s) {
  a.M = (int)M;
  a.m_tiles = (int)ceil_div(M, C::bm);
  a.n_tiles = (int)ceil_div(epi_swiglu(EPI) ? 2 * (int64_t)a.N : a.N, C::bn);
  return launch_gemm<C, false, false, EPI, NSEG>(a, (int64_t)a.m_tiles * a.n_tiles, s);
}

template <int EPI, int NSEG>
hipError_t dense_gemm_auto(GemmArgs a, int64_t M, hipStream_t s) {
  const int64_t ncols = epi_swiglu(EPI) ? 2 * (int64_t)a.N : a.N;
  // the 256 x 192 tile splits 192 columns into 2 waves of 96: not for the
  // interleaved gate/up pairs of the SwiGLU epilogue
  switch (dense_tile(M, ncols, !epi_swiglu(EPI))) {
    case DT_BIG: return dense_gemm<TileBig, EPI, NSEG>(a, M, s);
    case DT_WIDE:
      if constexpr (!epi_swiglu(EPI)) return dense_gemm<TileWide, EPI, NSEG>(a, M, s);
      return hipErrorInvalidValue;
    default: return dense_gemm<TileMid, EPI, NSEG>(a, M, s);
  }
}
template hipError_t dense_gemm_auto<EPI_F32, 1>(GemmArgs, int64_t, hipStream_t);
template hipError_t dense_gemm_auto<EPI_F32, 2>(GemmArgs, int64_t, hipStream_t);
template hipError_t dense_gemm_auto<EPI_F32_ADD, 2>(GemmArgs, int64_t, hipStream_t);

hipError_t launch_latent_down(const uint16_t* x, const uint16_t* w_dn, int64_t T, int d, int L,
                              uint16_t* z, hipStream_t s) {
  GemmArgs a = {};
  a.seg[0].A = x; a.seg[0].lda = d; a.seg[0].B = w_dn; a.seg[0].ldb = d; a.seg[0].K = d;
  a.nseg = 1;
  a.N = L;
  a.C = z;
  a.ldc = L;
  return dense_gemm_auto<EPI_BF16, 1>(a, T, s);
}

// FP8 path: z = bf16(x W_dn^T) quantized to E4M3 with the scale z_scale in
// the epilogue; the largest |z| goes to amax (one uint32 holding float bits).
hipError_t launch_latent_down_q8(const uint16_t* x, const uint16_t* w_dn, int64_t T, int d,
                                 int L, const float* z_scale, uint32_t* amax, uint8_t* z8,
                                 hipStream_t s) {
  GemmArgs a = {};
  a.seg[0].A = x; a.seg[0].lda = d; a.seg[0].B = w_dn; a.seg[0].ldb = d; a.seg[0].K = d;
  a.nseg = 1;
  a.N = L;
  a.C = z8;
  a.ldc = L;
  a.out_scale = z_scale;
  a.amax = amax;
  return dense_gemm_auto<EPI_Q8, 1>(a, T, s);
}

hipError_t launch_shared_gate_up(const uint16_t* x, const uint16_t* wsg, const uint16_t* wsu,
                                 int64_t T, int d, int Fs, uint16_t* hs, hipStream_t s) {
  GemmArgs a = {};
  a.seg[0].A = x; a.seg[0].lda = d; a.seg[0].B = wsg; a.seg[0].B2 = wsu; a.seg[0].ldb = d;
  a.seg[0].K = d;
  a.nseg = 1;
  a.N = Fs;
  a.C = hs;
  a.ldc = Fs;
  return dense_gemm_auto<EPI_SWIGLU, 1>(a, T, s);
}

// Backward of the shared expert (Base-2): its gate/up GEMM on x again
// (recomputation: the forward's tiles, so g, u and hs are the forward's bit
// for bit) with the SwiGLU backward in the epilogue: dgs = dhs us silu'(gs),
// dus = dhs silu(gs) cast to bf16 (nearest or stochastic with the stream
// keys), and hs.
hipError_t launch_shared_gate_up_bwd(const uint16_t* x, const uint16_t* wsg, const uint16_t* wsu,
                                     const float* dhs, int64_t T, int d, int Fs, int sr,
                                     uint32_t key_dg, uint32_t key_du, uint16_t* dgs_b,
                                     uint16_t* dus_b, uint16_t* hs_b, hipStream_t s) {
  GemmArgs a = {};
  a.seg[0].A = x; a.seg[0].lda = d; a.seg[0].B = wsg; a.seg[0].B2 = wsu; a.seg[0].ldb = d;
  a.seg[0].K = d;
  a.nseg = 1;
  a.N = Fs;
  a.C = dgs_b;
  a.C2 = dus_b;
  a.C3 = hs_b;
  a.aux_g = dhs;
  a.sr = sr;
  a.sr_key_c = key_dg;
  a.sr_key_c2 = key_du;
  a.ldc = Fs;
  return dense_gemm_auto<EPI_GU_BWD, 1>(a, T, s);
}

// Per-expert M-tile counts -> exclusive prefix, and the expert of every M
// tile, for two tile heights at once (gate/up and down GEMMs).
__global__ __launch_bounds__(1024) void tile_prefix_kernel(const int32_t* __restrict__ offsets,
                                                           int E, int bm_a, int bm_b,
                                                           int32_t* __restrict__ pre_a,
                                                           int32_t* __restrict__ pre_b,
                                                           int32_t* __restrict__ exp_a,
                                                           int32_t* __restrict__ exp_b,
                                                           int32_t* __restrict__ queues) {
  const int e = threadIdx.x;
  if (e < 16) queues[e] = 0;   // per-XCD tile counters of the two grouped GEMMs
  int rows = 0;
  if (e < E) rows = offsets[e + 1] - offsets[e];
  const int ma = e < E ? (rows + bm_a - 1) / bm_a : 0;
  const int mb = e < E ? (rows + bm_b - 1) / bm_b : 0;
  int ta, tb;
  const int ea = block_exclusive_scan(ma, &ta);
  const int eb = block_exclusive_scan(mb, &tb);
  if (e < E) {
    pre_a[e] = ea;
    pre_b[e] = eb;
    for (int i = 0; i < ma; ++i) exp_a[ea + i] = e;
    for (int i = 0; i < mb; ++i) exp_b[eb + i] = e;
  }
  if (e == 0) {
    pre_a[E] = ta;
    pre_b[E] = tb;
  }
}

hipError_t launch_tile_prefix(const int32_t* offsets, int E, int bm_a, int bm_b, int32_t* pre_a,
                              int32_t* pre_b, int32_t* exp_a, int32_t* exp_b, int32_t* queues,
                              hipStream_t s) {
  hipLaunchKernelGGL(tile_prefix_kernel, dim3(1), dim3(1024), 0, s, offsets, E, bm_a, bm_b, pre_a,
                     pre_b, exp_a, exp_b, queues);
  return hipGetLastError();
}

// One round of the multi-round dropless schedule (the schedule is described
// with moe_latent_ffn_forward_rounds in include/moe.h): expert e's rows this
// round, their place in the round's activation buffer, and the same tile
// tables as tile_prefix_kernel for the clipped row ranges.  Round 0 also
// writes the number of rounds the routing needs.
__global__ __launch_bounds__(1024) void round_tables_kernel(
    const int32_t* __restrict__ offsets, int E, int G, int C, int round, int bm_a, int bm_b,
    int32_t* __restrict__ seg_start, int32_t* __restrict__ seg_end, int32_t* __restrict__ h_base,
    int32_t* __restrict__ pre_a, int32_t* __restrict__ pre_b, int32_t* __restrict__ exp_a,
    int32_t* __restrict__ exp_b, int32_t* __restrict__ queues, int32_t* __restrict__ rounds_out,
    int32_t* __restrict__ h_end) {
  __shared__ int red[32];
  const int e = threadIdx.x;
  if (e < 16) queues[e] = 0;
  int rows = 0, need = 0, hb = 0;
  if (e < E) {
    const int g0 = e / G * G, g1 = min(g0 + G, E);
    const int64_t cap = (int64_t)(g1 - g0) * C;
    const int64_t lo = offsets[g0], hi = offsets[g1];
    const int64_t w0 = min(lo + (int64_t)round * cap, hi);
    const int64_t w1 = min(hi, w0 + cap);
    const int64_t b = min(max((int64_t)offsets[e], w0), (int64_t)offsets[e + 1]);
    const int64_t en = max(min((int64_t)offsets[e + 1], w1), b);
    seg_start[e] = (int32_t)b;
    seg_end[e] = (int32_t)en;
    hb = (int)((int64_t)g0 * C + min(max(b - w0, (int64_t)0), cap));
    rows = (int)(en - b);
    if (e == g0) need = (int)((hi - lo + cap - 1) / cap);   // this group's rounds
  }
  // h_end given (the backward): the round's rows packed in expert order, so
  // the buffers need only as many rows as the round holds (at most
  // min(T k, E C)); else the forward's slot layout (group g's slots from row
  // first_expert(g) * C)
  int packed_total;
  const int packed = block_exclusive_scan(rows, &packed_total);
  if (e < E) {
    h_base[e] = h_end ? packed : hb;
    if (h_end) h_end[e] = packed + rows;   // the rows' end in the round buffer
  }
  const int ma = e < E ? (rows + bm_a - 1) / bm_a : 0;
  const int mb = e < E ? (rows + bm_b - 1) / bm_b : 0;
  int ta, tb;
  const int ea = block_exclusive_scan(ma, &ta);
  const int eb = block_exclusive_scan(mb, &tb);
  if (e < E) {
    pre_a[e] = ea;
    pre_b[e] = eb;
    for (int i = 0; i < ma; ++i) exp_a[ea + i] = e;
    for (int i = 0; i < mb; ++i) exp_b[eb + i] = e;
  }
  if (e == 0) {
    pre_a[E] = ta;
    pre_b[E] = tb;
  }
  if (round == 0 && rounds_out != nullptr) {
    // maximum over groups (integer, order-independent)
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) need = max(need, __shfl_xor(need, o));
    if ((e & 63) == 0) red[e >> 6] = need;
    __syncthreads();
    if (e == 0) {
      int m = 0;
      for (int w = 0; w < (int)(blockDim.x >> 6); ++w) m = max(m, red[w]);
      rounds_out[0] = m;
    }
  }
}

hipError_t launch_round_tables(const int32_t* offsets, int E, int G, int C, int round, int bm_a,
                               int bm_b, int32_t* seg_start, int32_t* seg_end, int32_t* h_base,
                               int32_t* pre_a, int32_t* pre_b, int32_t* exp_a, int32_t* exp_b,
                               int32_t* queues, int32_t* rounds_out, hipStream_t s,
                               int32_t* h_end) {
  hipLaunchKernelGGL(round_tables_kernel, dim3(1), dim3(1024), 0, s, offsets, E, G, C, round, bm_a,
                     bm_b, seg_start, seg_end, h_base, pre_a, pre_b, exp_a, exp_b, queues,
                     rounds_out, h_end);
  return hipGetLastError();
}

template <int BM, bool GATHER, int EPI, int F8 = F8_NONE, int NSEG = 1>
static hipError_t grouped_gemm(GemmArgs a, int64_t rows, hipStream_t s) {
  // the forward's FP8 weight stream takes the wide FP8 tile; the FP8
  // gradient GEMMs (E5M2 A, K segments) keep the bf16 stream tile
  using CS = std::conditional_t<F8 == F8_E4M3 && NSEG == 1, TileStreamF8, TileStream>;
  using C = std::conditional_t<BM == 128, CS, TileBig>;
  static_assert(C::bm == BM, "tile height");
  a.n_tiles = (int)ceil_div(epi_swiglu(EPI) ? 2 * (int64_t)a.N : a.N, C::bn);
  const int64_t bound = grouped_mtile_bound(rows, a.E, BM) * a.n_tiles;
  return launch_gemm<C, true, GATHER, EPI, NSEG, F8>(a, bound, s);
}

hipError_t launch_gate_up(const uint16_t* z, const int32_t* offsets, const int32_t* row_token,
                          const int32_t* tile_prefix, const int32_t* tile_expert,
                          int32_t* queue, const uint16_t* w_gate, const uint16_t* w_up, int64_t T,
                          int64_t rows, int E, int L, int F, int bm, uint16_t* H, hipStream_t s) {
  GemmArgs a = {};
  a.seg[0].A = z; a.seg[0].lda = L; a.seg[0].B = w_gate; a.seg[0].B2 = w_up; a.seg[0].ldb = L;
  a.seg[0].K = L;
  a.nseg = 1;
  a.N = F;
  a.offsets = offsets;
  a.tile_prefix = tile_prefix;
  a.tile_expert = tile_expert;
  a.E = E;
  a.b_expert_stride = (int64_t)F * L;
  a.row_token = row_token;
  a.queue = queue;
  a.M = (int)T;   // rows of z, the gathered matrix
  a.C = H;
  a.ldc = F;
  if (bm == 128) return grouped_gemm<128, true, EPI_SWIGLU>(a, rows, s);
  return grouped_gemm<256, true, EPI_SWIGLU>(a, rows, s);
}

hipError_t launch_expert_down(const uint16_t* H, const int32_t* offsets,
                              const int32_t* tile_prefix, const int32_t* tile_expert,
                              int32_t* queue, const uint16_t* w_down, int64_t rows, int E, int L,
                              int F, int bm, float* Y, hipStream_t s) {
  GemmArgs a = {};
  a.seg[0].A = H; a.seg[0].lda = F; a.seg[0].B = w_down; a.seg[0].ldb = F; a.seg[0].K = F;
  a.nseg = 1;
  a.N = L;
  a.offsets = offsets;
  a.tile_prefix = tile_prefix;
  a.tile_expert = tile_expert;
  a.queue = queue;
  a.E = E;
  a.b_expert_stride = (int64_t)L * F;
  a.C = Y;
  a.ldc = L;
  if (bm == 128) return grouped_gemm<128, false, EPI_F32>(a, rows, s);
  return grouped_gemm<256, false, EPI_F32>(a, rows, s);
}

// Backward, first: dh = dy W_d[e] per expert (B = W_d[e]^T [F, L]), fp32.
hipError_t launch_expert_dh(const uint16_t* dy_b, const int32_t* offsets,
                            const int32_t* tile_prefix, const int32_t* tile_expert,
                            int32_t* queue, const uint16_t* w_down_t, int64_t rows, int E, int L,
                            int F, int bm, float* dh, hipStream_t s) {
  GemmArgs a = {};
  a.seg[0].A = dy_b; a.seg[0].lda = L; a.seg[0].B = w_down_t; a.seg[0].ldb = L; a.seg[0].K = L;
  a.nseg = 1;
  a.N = F;
  a.offsets = offsets;
  a.tile_prefix = tile_prefix;
  a.tile_expert = tile_expert;
  a.queue = queue;
  a.E = E;
  a.b_expert_stride = (int64_t)F * L;
  a.C = dh;
  a.ldc = F;
  if (bm == 128) return grouped_gemm<128, false, EPI_F32>(a, rows, s);
  return grouped_gemm<256, false, EPI_F32>(a, rows, s);
}

// Backward, then: the gate/up GEMM again (recomputation: same tiles and order
// as the forward, so g, u and h are the forward's bit for bit), with the
// SwiGLU backward in its epilogue: dg = dh u silu'(g), du = dh silu(g) cast
// to bf16 (RNE or stochastic rounding with the stream keys), and h.
hipError_t launch_gate_up_bwd(const uint16_t* z, const int32_t* offsets, const int32_t* row_token,
                              const int32_t* tile_prefix, const int32_t* tile_expert,
                              int32_t* queue, const uint16_t* w_gate, const uint16_t* w_up,
                              const float* dh, int64_t T, int64_t rows, int E, int L, int F, int bm,
                              int sr, uint32_t key_dg, uint32_t key_du, uint16_t* dg_b,
                              uint16_t* du_b, uint16_t* h, hipStream_t s) {
  GemmArgs a = {};
  a.seg[0].A = z; a.seg[0].lda = L; a.seg[0].B = w_gate; a.seg[0].B2 = w_up; a.seg[0].ldb = L;
  a.seg[0].K = L;
  a.nseg = 1;
  a.N = F;
  a.offsets = offsets;
  a.tile_prefix = tile_prefix;
  a.tile_expert = tile_expert;
  a.E = E;
  a.b_expert_stride = (int64_t)F * L;
  a.row_token = row_token;
  a.queue = queue;
  a.M = (int)T;
  a.C = dg_b;
  a.C2 = du_b;
  a.C3 = h;
  a.aux_g = dh;
  a.sr = sr;
  a.sr_key_c = key_dg;
  a.sr_key_c2 = key_du;
  a.ldc = F;
  if (bm == 128) return grouped_gemm<128, true, EPI_GU_BWD>(a, rows, s);
  return grouped_gemm<256, true, EPI_GU_BWD>(a, rows, s);
}

// Backward: the rows' latent gradient dzp = dg W_g[e] + du W_u[e] (fp32), one
// accumulation over the two K segments (B = W_g[e]^T, W_u[e]^T [L, F]).
hipError_t launch_dzp(const uint16_t* dg_b, const uint16_t* du_b, const int32_t* offsets,
                      const int32_t* tile_prefix, const int32_t* tile_expert, int32_t* queue,
                      const uint16_t* w_gate_t, const uint16_t* w_up_t, int64_t rows, int E,
                      int L, int F, int bm, float* dzp, hipStream_t s) {
  GemmArgs a = {};
  a.seg[0].A = dg_b; a.seg[0].lda = F; a.seg[0].B = w_gate_t; a.seg[0].ldb = F; a.seg[0].K = F;
  a.seg[1].A = du_b; a.seg[1].lda = F; a.seg[1].B = w_up_t; a.seg[1].ldb = F; a.seg[1].K = F;
  a.nseg = 2;
  a.N = L;
  a.offsets = offsets;
  a.tile_prefix = tile_prefix;
  a.tile_expert = tile_expert;
  a.queue = queue;
  a.E = E;
  a.b_expert_stride = (int64_t)L * F;
  a.C = dzp;
  a.ldc = L;
  if (bm == 128) return grouped_gemm<128, false, EPI_F32, F8_NONE, 2>(a, rows, s);
  return grouped_gemm<256, false, EPI_F32, F8_NONE, 2>(a, rows, s);
}

// Backward with FP8 data gradients: the gate/up recompute as above that also
// writes dg and du as E5M2 codes (dg8, du8; scales 128 grad_scale[1], 128
// grad_scale[2]; rounding as for the bf16 casts, stream keys key_dg8 and
// key_du8) and records max |dg|, max |du| in grad_amax[1], grad_amax[2].
hipError_t launch_gate_up_bwd_q8(const uint16_t* z, const int32_t* offsets,
                                 const int32_t* row_token, const int32_t* tile_prefix,
                                 const int32_t* tile_expert, int32_t* queue,
                                 const uint16_t* w_gate, const uint16_t* w_up, const float* dh,
                                 int64_t T, int64_t rows, int E, int L, int F, int bm, int sr,
                                 uint32_t key_dg, uint32_t key_du, uint32_t key_dg8,
                                 uint32_t key_du8, const float* grad_scale, uint32_t* grad_amax,
                                 uint16_t* dg_b, uint16_t* du_b, uint16_t* h, uint8_t* dg8,
                                 uint8_t* du8, hipStream_t s) {
  GemmArgs a = {};
  a.seg[0].A = z; a.seg[0].lda = L; a.seg[0].B = w_gate; a.seg[0].B2 = w_up; a.seg[0].ldb = L;
  a.seg[0].K = L;
  a.nseg = 1;
  a.N = F;
  a.offsets = offsets;
  a.tile_prefix = tile_prefix;
  a.tile_expert = tile_expert;
  a.E = E;
  a.b_expert_stride = (int64_t)F * L;
  a.row_token = row_token;
  a.queue = queue;
  a.M = (int)T;
  a.C = dg_b;
  a.C2 = du_b;
  a.C3 = h;
  a.C4 = dg8;
  a.C5 = du8;
  a.aux_g = dh;
  a.sr = sr;
  a.sr_key_c = key_dg;
  a.sr_key_c2 = key_du;
  a.sr_key_c4 = key_dg8;
  a.sr_key_c5 = key_du8;
  a.out_scale = grad_scale;
  a.amax = grad_amax;
  a.ldc = F;
  if (bm == 128) return grouped_gemm<128, true, EPI_GU_BWD_Q8>(a, rows, s);
  return grouped_gemm<256, true, EPI_GU_BWD_Q8>(a, rows, s);
}

// FP8 data gradient dh = (q_dy Q(W_d[e])) / (128 s_dy s_Wd[e]): dy8 [rows, L]
// E5M2 codes, w_down_t8 = Q(W_d[e])^T [E, F, L] E4M3 (the transpose of the
// forward's quantized weight), dy_scale the E4M3-convention scale s_dy.
hipError_t launch_expert_dh_fp8(const uint8_t* dy8, const int32_t* offsets,
                                const int32_t* tile_prefix, const int32_t* tile_expert,
                                int32_t* queue, const uint8_t* w_down_t8, const float* dy_scale,
                                const float* wd_scale, int64_t rows, int E, int L, int F, int bm,
                                float* dh, hipStream_t s) {
  GemmArgs a = {};
  a.seg[0].A = dy8; a.seg[0].lda = L; a.seg[0].B = w_down_t8; a.seg[0].ldb = L; a.seg[0].K = L;
  a.nseg = 1;
  a.N = F;
  a.offsets = offsets;
  a.tile_prefix = tile_prefix;
  a.tile_expert = tile_expert;
  a.queue = queue;
  a.E = E;
  a.b_expert_stride = (int64_t)F * L;
  a.C = dh;
  a.ldc = F;
  a.a_scale = dy_scale;
  a.b_scale = wd_scale;
  if (bm == 128) return grouped_gemm<128, false, EPI_F32, F8_E5M2_A>(a, rows, s);
  return grouped_gemm<256, false, EPI_F32, F8_E5M2_A>(a, rows, s);
}

// FP8 rows' latent gradient dzp = (q_dg Q(W_g[e])) / (128 s_dg s_Wg[e]) +
// (q_du Q(W_u[e])) / (128 s_du s_Wu[e]), one accumulation over two K
// segments with separate dequantization (w_gate_t8, w_up_t8 = Q(W_g[e])^T,
// Q(W_u[e])^T [E, L, F] E4M3).
hipError_t launch_dzp_fp8(const uint8_t* dg8, const uint8_t* du8, const int32_t* offsets,
                          const int32_t* tile_prefix, const int32_t* tile_expert, int32_t* queue,
                          const uint8_t* w_gate_t8, const uint8_t* w_up_t8,
                          const float* dg_scale, const float* du_scale, const float* wg_scale,
                          const float* wu_scale, int64_t rows, int E, int L, int F, int bm,
                          float* dzp, hipStream_t s) {
  GemmArgs a = {};
  a.seg[0].A = dg8; a.seg[0].lda = F; a.seg[0].B = w_gate_t8; a.seg[0].ldb = F; a.seg[0].K = F;
  a.seg[1].A = du8; a.seg[1].lda = F; a.seg[1].B = w_up_t8; a.seg[1].ldb = F; a.seg[1].K = F;
  a.nseg = 2;
  a.N = L;
  a.offsets = offsets;
  a.tile_prefix = tile_prefix;
  a.tile_expert = tile_expert;
  a.queue = queue;
  a.E = E;
  a.b_expert_stride = (int64_t)L * F;
  a.C = dzp;
  a.ldc = L;
  a.a_scale = dg_scale;
  a.b_scale = wg_scale;
  a.a2_scale = du_scale;
  a.b2_scale = wu_scale;
  if (bm == 128) return grouped_gemm<128, false, EPI_F32, F8_E5M2_A, 2>(a, rows, s);
  return grouped_gemm<256, false, EPI_F32, F8_E5M2_A, 2>(a, rows, s);
}

// FP8 experts: z8 and the weights are E4M3 with scales (z: one, weights: one
// per expert); h = bf16(silu(g) u) is written as E4M3 with h_scale and its
// largest |h| goes to amax.
hipError_t launch_gate_up_fp8(const uint8_t* z8, const int32_t* offsets, const int32_t* row_token,
                              const int32_t* tile_prefix, const int32_t* tile_expert,
                              int32_t* queue, const uint8_t* w_gate, const uint8_t* w_up,
                              const float* z_scale, const float* wg_scale, const float* wu_scale,
                              const float* h_scale, uint32_t* amax, int64_t T, int64_t rows,
                              int E, int L, int F, int bm, uint8_t* H8, hipStream_t s) {
  GemmArgs a = {};
  a.seg[0].A = z8; a.seg[0].lda = L; a.seg[0].B = w_gate; a.seg[0].B2 = w_up; a.seg[0].ldb = L;
  a.seg[0].K = L;
  a.nseg = 1;
  a.N = F;
  a.offsets = offsets;
  a.tile_prefix = tile_prefix;
  a.tile_expert = tile_expert;
  a.E = E;
  a.b_expert_stride = (int64_t)F * L;
  a.row_token = row_token;
  a.queue = queue;
  a.M = (int)T;
  a.C = H8;
  a.ldc = F;
  a.a_scale = z_scale;
  a.b_scale = wg_scale;
  a.b2_scale = wu_scale;
  a.out_scale = h_scale;
  a.amax = amax;
  if (bm == 128) return grouped_gemm<128, true, EPI_SWIGLU_Q8, F8_E4M3>(a, rows, s);
  return grouped_gemm<256, true, EPI_SWIGLU_Q8, F8_E4M3>(a, rows, s);
}

hipError_t launch_expert_down_fp8(const uint8_t* H8, const int32_t* offsets,
                                  const int32_t* tile_prefix, const int32_t* tile_expert,
                                  int32_t* queue, const uint8_t* w_down, const float* h_scale,
                                  const float* wd_scale, int64_t rows, int E, int L, int F,
                                  int bm, float* Y, hipStream_t s) {
  GemmArgs a = {};
  a.seg[0].A = H8; a.seg[0].lda = F; a.seg[0].B = w_down; a.seg[0].ldb = F; a.seg[0].K = F;
  a.nseg = 1;
  a.N = L;
  a.offsets = offsets;
  a.tile_prefix = tile_prefix;
  a.tile_expert = tile_expert;
  a.queue = queue;
  a.E = E;
  a.b_expert_stride = (int64_t)L * F;
  a.C = Y;
  a.ldc = L;
  a.a_scale = h_scale;
  a.b_scale = wd_scale;
  if (bm == 128) return grouped_gemm<128, false, EPI_F32, F8_E4M3>(a, rows, s);
  return grouped_gemm<256, false, EPI_F32, F8_E4M3>(a, rows, s);
}

// A round of the multi-round schedule: gate/up over the round's rows of every
// expert into the round buffer Hr, then down from Hr into y_rows (rows in
// permutation order).  rows_bound: the most rows a round can hold.
hipError_t launch_round_experts(const uint16_t* z, const int32_t* seg_start,
                                const int32_t* seg_end, const int32_t* h_base,
                                const int32_t* row_token, const int32_t* pre_a,
                                const int32_t* exp_a, const int32_t* pre_b, const int32_t* exp_b,
                                int32_t* queues, const uint16_t* w_gate, const uint16_t* w_up,
                                const uint16_t* w_down, int64_t T, int64_t rows_bound, int E,
                                int L, int F, int bm_a, int bm_b, uint16_t* Hr, float* Y,
                                hipStream_t s) {
  GemmArgs a = {};
  a.seg[0].A = z; a.seg[0].lda = L; a.seg[0].B = w_gate; a.seg[0].B2 = w_up; a.seg[0].ldb = L;
  a.seg[0].K = L;
  a.nseg = 1;
  a.N = F;
  a.offsets = seg_start;
  a.seg_end = seg_end;
  a.h_base = h_base;
  a.h_side = 1;
  a.tile_prefix = pre_a;
  a.tile_expert = exp_a;
  a.E = E;
  a.b_expert_stride = (int64_t)F * L;
  a.row_token = row_token;
  a.queue = queues;
  a.M = (int)T;
  a.C = Hr;
  a.ldc = F;
  hipError_t err = bm_a == 128 ? grouped_gemm<128, true, EPI_SWIGLU>(a, rows_bound, s)
                               : grouped_gemm<256, true, EPI_SWIGLU>(a, rows_bound, s);
  if (err != hipSuccess) return err;
  GemmArgs b = {};
  b.seg[0].A = Hr; b.seg[0].lda = F; b.seg[0].B = w_down; b.seg[0].ldb = F; b.seg[0].K = F;
  b.nseg = 1;
  b.N = L;
  b.offsets = seg_start;
  b.seg_end = seg_end;
  b.h_base = h_base;
  b.h_side = 2;
  b.tile_prefix = pre_b;
  b.tile_expert = exp_b;
  b.queue = queues + 8;
  b.E = E;
  b.b_expert_stride = (int64_t)L * F;
  b.C = Y;
  b.ldc = L;
  return bm_b == 128 ? grouped_gemm<128, false, EPI_F32>(b, rows_bound, s)
                     : grouped_gemm<256, false, EPI_F32>(b, rows_bound, s);
}

// One round of the multi-round backward (the forward's round tables: expert
// e's rows this round are [seg_start[e], seg_end[e]) of the permutation, at
// rows h_base[e].. of the round buffers):
//   dh = dy W_d[e]                     dy rows (permutation order) -> dh (round rows)
//   g, u recomputed from the gathered z; dg, du, h by the SwiGLU backward
//                                      -> dg_b, du_b, h (round rows)
//   dzp = dg W_g[e] + du W_u[e]        round rows -> dzp (permutation order)
// with the tile plans of the single-pass backward, so every row's values
// are the single pass's bit for bit.  queues: 24 per-XCD counters, zeroed by
// the round-table kernel (first 16) and here (last 8).
hipError_t launch_round_expert_bwd(const uint16_t* dy_b, const uint16_t* z,
                                   const int32_t* row_token, const int32_t* seg_start,
                                   const int32_t* seg_end, const int32_t* h_base,
                                   const int32_t* pre_a, const int32_t* exp_a,
                                   const int32_t* pre_b, const int32_t* exp_b, int32_t* queues,
                                   const uint16_t* w_gate, const uint16_t* w_up,
                                   const uint16_t* w_gate_t, const uint16_t* w_up_t,
                                   const uint16_t* w_down_t, int64_t T, int64_t rows_bound, int E,
                                   int L, int F, int bm_a, int bm_b, int sr, uint32_t key_dg,
                                   uint32_t key_du, float* dh, uint16_t* dg_b, uint16_t* du_b,
                                   uint16_t* h, float* dzp, hipStream_t s) {
  hipError_t err = launch_zero_u32((uint32_t*)queues + 16, 8, s);
  if (err != hipSuccess) return err;
  // dh = dy W_d[e] (B = W_d[e]^T [F, L]): A rows in permutation order, C rows
  // in the round buffer
  GemmArgs a = {};
  a.seg[0].A = dy_b; a.seg[0].lda = L; a.seg[0].B = w_down_t; a.seg[0].ldb = L; a.seg[0].K = L;
  a.nseg = 1;
  a.N = F;
  a.offsets = seg_start;
  a.seg_end = seg_end;
  a.h_base = h_base;
  a.h_side = 1;
  a.tile_prefix = pre_b;
  a.tile_expert = exp_b;
  a.queue = queues;
  a.E = E;
  a.b_expert_stride = (int64_t)F * L;
  a.C = dh;
  a.ldc = F;
  err = bm_b == 128 ? grouped_gemm<128, false, EPI_F32>(a, rows_bound, s)
                    : grouped_gemm<256, false, EPI_F32>(a, rows_bound, s);
  if (err != hipSuccess) return err;
  // the gate/up GEMM again with the SwiGLU backward in its epilogue: A = the
  // gathered z of the round's rows; dh (aux), dg, du and h at round rows
  GemmArgs g = {};
  g.seg[0].A = z; g.seg[0].lda = L; g.seg[0].B = w_gate; g.seg[0].B2 = w_up; g.seg[0].ldb = L;
  g.seg[0].K = L;
  g.nseg = 1;
  g.N = F;
  g.offsets = seg_start;
  g.seg_end = seg_end;
  g.h_base = h_base;
  g.h_side = 1;
  g.tile_prefix = pre_a;
  g.tile_expert = exp_a;
  g.E = E;
  g.b_expert_stride = (int64_t)F * L;
  g.row_token = row_token;
  g.queue = queues + 8;
  g.M = (int)T;
  g.C = dg_b;
  g.C2 = du_b;
  g.C3 = h;
  g.aux_g = dh;
  g.sr = sr;
  g.sr_key_c = key_dg;
  g.sr_key_c2 = key_du;
  g.ldc = F;
  err = bm_a == 128 ? grouped_gemm<128, true, EPI_GU_BWD>(g, rows_bound, s)
                    : grouped_gemm<256, true, EPI_GU_BWD>(g, rows_bound, s);
  if (err != hipSuccess) return err;
  // dzp = dg W_g[e] + du W_u[e] (B = W_g[e]^T, W_u[e]^T [L, F]): A rows in the
  // round buffer, C rows in permutation order
  GemmArgs b = {};
  b.seg[0].A = dg_b; b.seg[0].lda = F; b.seg[0].B = w_gate_t; b.seg[0].ldb = F; b.seg[0].K = F;
  b.seg[1].A = du_b; b.seg[1].lda = F; b.seg[1].B = w_up_t; b.seg[1].ldb = F; b.seg[1].K = F;
  b.nseg = 2;
  b.N = L;
  b.offsets = seg_start;
  b.seg_end = seg_end;
  b.h_base = h_base;
  b.h_side = 2;
  b.tile_prefix = pre_b;
  b.tile_expert = exp_b;
  b.queue = queues + 16;
  b.E = E;
  b.b_expert_stride = (int64_t)L * F;
  b.C = dzp;
  b.ldc = L;
  return bm_b == 128 ? grouped_gemm<128, false, EPI_F32, F8_NONE, 2>(b, rows_bound, s)
                     : grouped_gemm<256, false, EPI_F32, F8_NONE, 2>(b, rows_bound, s);
}

// Compute units of the current device, queried once per device.  The cache
// entries are atomics: threads that race on a first query store the same
// value, so calls from several host threads are safe.
int device_cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

}  // namespace moe
