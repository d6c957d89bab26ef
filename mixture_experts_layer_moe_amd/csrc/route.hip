// Router: FP32 routing GEMM on the full hidden state, softmax over all
// experts, stable top-k ("The Training and RL Infrastructure Behind
// MAI-Thinking-1": model table MoE row; section 2 "Pre-training and
// mid-training precision" — router weights, routing GEMM and logits in FP32;
// section 2 "Bitwise determinism" — stable top-k).
//
// FP32 routing GEMM on bf16 matrix cores: x is exactly bf16, and an fp32
// weight w splits exactly into three bf16 parts, w = hi + mid + lo (each part
// takes the next 8 significant bits; no part underflows for these weights).
// Every product x*part is exact in fp32 (8-bit x 8-bit significands), and
// the MFMA accumulates them in fp32, so x W_r^T is an FP32 GEMM computed in
// a different summation order, at bf16 MFMA speed (three passes along K).
#include "launch.hpp"
#include "gemm.hpp"

namespace moe {

__global__ void split_router_kernel(const float* __restrict__ w, uint16_t* __restrict__ w3,
                                    int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float v = w[i];
  const uint16_t hi = f32_to_bf16_rne(v);
  const float r1 = v - bf16_to_f32(hi);       // exact
  const uint16_t mid = f32_to_bf16_rne(r1);
  const float r2 = r1 - bf16_to_f32(mid);     // exact
  const uint16_t lo = f32_to_bf16_rne(r2);
  w3[i] = hi;
  w3[n + i] = mid;
  w3[2 * n + i] = lo;
}

hipError_t launch_router_gemm(const uint16_t* x, const float* w_router, const float* bias,
                              int64_t T, int d, int E, uint16_t* w3, float* logits,
                              hipStream_t s) {
  const int64_t n = (int64_t)E * d;
  hipLaunchKernelGGL(split_router_kernel, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, s,
                     w_router, w3, n);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  GemmArgs a = {};
  for (int p = 0; p < 3; ++p) {
    a.seg[p].A = x;
    a.seg[p].lda = d;
    a.seg[p].B = w3 + p * n;
    a.seg[p].ldb = d;
    a.seg[p].K = d;
  }
  a.nseg = 3;
  a.M = (int)T;
  a.N = E;
  a.C = logits;
  a.ldc = E;
  a.bias = bias;
  // the K split is decided from the shapes first (the top-k kernel sums as
  // many partial arrays)
  const int ks = router_ksplit(T, E);
  // large batches: 256 x 256 tiles already give every CU a tile
  if (ks == 1 && ceil_div(T, TileBig::bm) * ceil_div(E, TileBig::bn) >= device_cu_count()) {
    a.m_tiles = (int)ceil_div(T, TileBig::bm);
    a.n_tiles = (int)ceil_div(E, TileBig::bn);
    return launch_gemm<TileBig, false, false, EPI_F32_BIAS, 3>(a, (int64_t)a.m_tiles * a.n_tiles,
                                                            s);
  }
  // mid batches (e.g. T = 16,384 at E = 512): 128 x 256 tiles, one per CU
  a.m_tiles = (int)ceil_div(T, TileMid::bm);
  a.n_tiles = (int)ceil_div(E, TileMid::bn);
  if (ks == 1)
    return launch_gemm<TileMid, false, false, EPI_F32_BIAS, 3>(a, (int64_t)a.m_tiles * a.n_tiles,
                                                            s);
  // small batches (e.g. T = 4,096): the same tiles, K split into ks chunks
  // (each a run of 3 d / ks of the hi/mid/lo K), so that ks times as many
  // workgroups share the long K loop; each chunk writes partial logits
  // without bias and the top-k kernel sums them in chunk order
  a.ksplit = ks;
  a.c_split = T * (int64_t)E;
  a.bias = nullptr;
  return launch_gemm<TileMid, false, false, EPI_F32_BIAS, 3>(
      a, (int64_t)a.m_tiles * a.n_tiles * ks, s);
}

// Chunks so that the 128 x 256 tiles times the chunks come near the 256 CUs
// of an MI355X (at most 4), unless the 128 x 256 tiles fill them already.
// A function of the shapes only, so that workspace sizes are too.
int router_ksplit(int64_t T, int E) {
  constexpr int64_t CUS = 256;
  const int64_t tiles = ceil_div(T, 128) * ceil_div(E, 256);
  if (tiles >= CUS) return 1;
  const int64_t ks = CUS / (tiles > 0 ? tiles : 1);
  return (int)(ks < 1 ? 1 : (ks > 4 ? 4 : ks));
}

// ---------------------------------------------------------------------------
// softmax over all E logits + top-k.  A workgroup is 4 waves; each wave
// handles TOPK_TOK_PER_WAVE consecutive tokens, one at a time (one token per
// wave: at T = 4,096 that is 1,024 workgroups, enough waves in flight to hide
// the loads of the logits; four per wave took 2.5x as long there).
// Lane l holds logits l, l+64, ...; the max, the sum of exponentials and each
// of the k argmax rounds are wave reductions with a fixed butterfly order, so
// the result is deterministic.  Ranking key: (selection value descending,
// index ascending) == a stable sort; the selection value is the logit plus
// the optional selection-only bias (a loss-free balancer).
// Optional load-balancing statistics: every workgroup writes the sum of each
// expert's probability over its tokens (tokens in order within a wave, then
// the 4 waves in order) to prob_part[chunk][E]; reduce_prob_kernel sums the
// chunks in order.
// ---------------------------------------------------------------------------
constexpr int TOPK_TOK_PER_WAVE = 1;
constexpr int TOPK_CHUNK = 4 * TOPK_TOK_PER_WAVE;   // tokens per workgroup

template <int PER_LANE>
__global__ __launch_bounds__(256) void softmax_topk_kernel(const float* __restrict__ logits,
                                                           int nsplit,
                                                           const float* __restrict__ lbias,
                                                           float* __restrict__ logits_out,
                                                           const float* __restrict__ sel_bias,
                                                           int64_t T, int E, int k,
                                                           int32_t* __restrict__ topk_idx,
                                                           float* __restrict__ topk_w,
                                                           float* __restrict__ prob_part) {
  const int64_t split_stride = T * (int64_t)E;
  __shared__ float part[4][PER_LANE * 64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  float bsel[PER_LANE];
#pragma unroll
  for (int i = 0; i < PER_LANE; ++i) {
    const int e = lane + 64 * i;
    bsel[i] = (sel_bias != nullptr && e < E) ? sel_bias[e] : 0.f;
  }
  float psum[PER_LANE];
#pragma unroll
  for (int i = 0; i < PER_LANE; ++i) psum[i] = 0.f;

  for (int q = 0; q < TOPK_TOK_PER_WAVE; ++q) {
    const int64_t t = (int64_t)blockIdx.x * TOPK_CHUNK + wave * TOPK_TOK_PER_WAVE + q;
    if (t >= T) break;
    const float* row = logits + t * E;
    float v[PER_LANE];
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) {
      const int e = lane + 64 * i;
      if (e < E) {
        // K chunks of the routing GEMM in order, then the logit bias
        float l = row[e];
        for (int c = 1; c < nsplit; ++c) l += row[c * split_stride + e];
        if (lbias != nullptr) l += lbias[e];
        if (logits_out != nullptr) logits_out[t * E + e] = l;
        v[i] = l;
      } else {
        v[i] = -INFINITY;
      }
      m = fmaxf(m, v[i]);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) sum += (lane + 64 * i < E) ? expf(v[i] - m) : 0.f;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
    const float inv = 1.0f / sum;
    if (prob_part != nullptr) {
#pragma unroll
      for (int i = 0; i < PER_LANE; ++i)
        if (lane + 64 * i < E) psum[i] += expf(v[i] - m) * inv;
    }

    unsigned taken = 0;   // bit i: element i of this lane already selected
    for (int j = 0; j < k; ++j) {
      float bs = -INFINITY, bv = 0.f;
      int be = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < PER_LANE; ++i) {
        const int e = lane + 64 * i;
        const float sv = v[i] + bsel[i];
        if (e < E && !((taken >> i) & 1u) && (sv > bs || (sv == bs && e < be))) {
          bs = sv;
          bv = v[i];
          be = e;
        }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const float os = __shfl_xor(bs, o);
        const float ov = __shfl_xor(bv, o);
        const int oe = __shfl_xor(be, o);
        if (os > bs || (os == bs && oe < be)) { bs = os; bv = ov; be = oe; }
      }
      if ((be & 63) == lane) taken |= 1u << (be >> 6);
      if (lane == 0) {
        topk_idx[t * k + j] = be;
        topk_w[t * k + j] = expf(bv - m) * inv;
      }
    }
  }
  if (prob_part != nullptr) {
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) part[wave][lane + 64 * i] = psum[i];
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x)
      prob_part[(int64_t)blockIdx.x * E + e] = ((part[0][e] + part[1][e]) + part[2][e]) + part[3][e];
  }
}

// Fixed-order two-stage sum of the per-chunk partials.  Stage 1: workgroup
// (column block, group g) sums chunks [64g, 64g + 64) of 64 experts, each of
// its 4 waves a run of 16 chunks in order, then the 4 runs in order.  Stage 2:
// the groups in order.
constexpr int PROB_GROUP = 64;

__global__ __launch_bounds__(256) void reduce_prob_groups_kernel(const float* __restrict__ prob_part,
                                                                 int64_t nchunks, int E,
                                                                 float* __restrict__ group_part) {
  __shared__ float run[4][64];
  const int lane = threadIdx.x & 63;
  const int sub = threadIdx.x >> 6;
  const int e = blockIdx.x * 64 + lane;
  const int64_t c0 = (int64_t)blockIdx.y * PROB_GROUP + sub * (PROB_GROUP / 4);
  float acc = 0.f;
  if (e < E) {
#pragma unroll
    for (int i = 0; i < PROB_GROUP / 4; ++i)
      if (c0 + i < nchunks) acc += prob_part[(c0 + i) * E + e];
  }
  run[sub][lane] = acc;
  __syncthreads();
  if (sub == 0 && e < E)
    group_part[(int64_t)blockIdx.y * E + e] = ((run[0][lane] + run[1][lane]) + run[2][lane]) +
                                              run[3][lane];
}

__global__ __launch_bounds__(256) void reduce_prob_kernel(const float* __restrict__ group_part,
                                                          int64_t ngroups, int E,
                                                          float* __restrict__ prob_sum) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= E) return;
  float acc = 0.f;
#pragma unroll 8
  for (int64_t g = 0; g < ngroups; ++g) acc += group_part[g * E + e];
  prob_sum[e] = acc;
}

int64_t topk_chunks(int64_t T) { return ceil_div(T, TOPK_CHUNK); }
int64_t topk_partial_floats(int64_t T, int E) {
  const int64_t n = topk_chunks(T);
  return (n + ceil_div(n, PROB_GROUP)) * E;
}

hipError_t launch_softmax_topk(const float* logits, int nsplit, const float* lbias,
                               float* logits_out, const float* sel_bias, int64_t T, int E, int k,
                               int32_t* topk_idx, float* topk_w, float* prob_part,
                               float* prob_sum, hipStream_t s) {
  const dim3 grid((unsigned)topk_chunks(T)), block(256);
  const int per = (int)ceil_div(E, 64);
#define MOE_TOPK_LAUNCH(P)                                                                      \
  hipLaunchKernelGGL(softmax_topk_kernel<P>, grid, block, 0, s, logits, nsplit, lbias,          \
                     logits_out, sel_bias, T, E, k, topk_idx, topk_w, prob_part)
  if (per <= 1) MOE_TOPK_LAUNCH(1);
  else if (per <= 2) MOE_TOPK_LAUNCH(2);
  else if (per <= 4) MOE_TOPK_LAUNCH(4);
  else if (per <= 8) MOE_TOPK_LAUNCH(8);
  else MOE_TOPK_LAUNCH(16);
#undef MOE_TOPK_LAUNCH
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || prob_sum == nullptr) return err;
  const int64_t nchunks = topk_chunks(T), ngroups = ceil_div(nchunks, PROB_GROUP);
  float* group_part = prob_part + nchunks * E;
  hipLaunchKernelGGL(reduce_prob_groups_kernel, dim3((unsigned)ceil_div(E, 64), (unsigned)ngroups),
                     dim3(256), 0, s, prob_part, nchunks, E, group_part);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(reduce_prob_kernel, dim3((unsigned)ceil_div(E, 256)), dim3(256), 0, s,
                     group_part, ngroups, E, prob_sum);
  return hipGetLastError();
}

}  // namespace moe
