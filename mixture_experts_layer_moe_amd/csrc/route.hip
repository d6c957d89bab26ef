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
  // large batches: 256 x 256 tiles already give every CU a tile
  if (ceil_div(T, TileBig::bm) * ceil_div(E, TileBig::bn) >= device_cu_count()) {
    a.m_tiles = (int)ceil_div(T, TileBig::bm);
    a.n_tiles = (int)ceil_div(E, TileBig::bn);
    return launch_gemm<TileBig, false, false, EPI_F32_BIAS>(a, (int64_t)a.m_tiles * a.n_tiles,
                                                            s);
  }
  a.m_tiles = (int)ceil_div(T, TileRouter::bm);
  a.n_tiles = (int)ceil_div(E, TileRouter::bn);
  return launch_gemm<TileRouter, false, false, EPI_F32_BIAS>(a, (int64_t)a.m_tiles * a.n_tiles,
                                                             s);
}

// ---------------------------------------------------------------------------
// softmax over all E logits + top-k, one wave per token.
// Lane l holds logits l, l+64, ...; the max, the sum of exponentials and each
// of the k argmax rounds are wave reductions with a fixed butterfly order, so
// the result is deterministic.  Ranking key: (logit descending, index
// ascending) == a stable sort of the logits.
// ---------------------------------------------------------------------------
template <int PER_LANE>
__global__ __launch_bounds__(256) void softmax_topk_kernel(const float* __restrict__ logits,
                                                           int64_t T, int E, int k,
                                                           int32_t* __restrict__ topk_idx,
                                                           float* __restrict__ topk_w) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + t * E;
  float v[PER_LANE];
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < PER_LANE; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < E ? row[e] : -INFINITY;
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

  unsigned taken = 0;   // bit i: element i of this lane already selected
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) {
      const int e = lane + 64 * i;
      if (e < E && !((taken >> i) & 1u) && (v[i] > bv || (v[i] == bv && e < be))) {
        bv = v[i];
        be = e;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o);
      const int oe = __shfl_xor(be, o);
      if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
    }
    if ((be & 63) == lane) taken |= 1u << (be >> 6);
    if (lane == 0) {
      topk_idx[t * k + j] = be;
      topk_w[t * k + j] = expf(bv - m) * inv;
    }
  }
}

hipError_t launch_softmax_topk(const float* logits, int64_t T, int E, int k, int32_t* topk_idx,
                               float* topk_w, hipStream_t s) {
  const dim3 grid((unsigned)ceil_div(T, 4)), block(256);
  const int per = (int)ceil_div(E, 64);
  if (per <= 1)
    hipLaunchKernelGGL(softmax_topk_kernel<1>, grid, block, 0, s, logits, T, E, k, topk_idx, topk_w);
  else if (per <= 2)
    hipLaunchKernelGGL(softmax_topk_kernel<2>, grid, block, 0, s, logits, T, E, k, topk_idx, topk_w);
  else if (per <= 4)
    hipLaunchKernelGGL(softmax_topk_kernel<4>, grid, block, 0, s, logits, T, E, k, topk_idx, topk_w);
  else if (per <= 8)
    hipLaunchKernelGGL(softmax_topk_kernel<8>, grid, block, 0, s, logits, T, E, k, topk_idx, topk_w);
  else
    hipLaunchKernelGGL(softmax_topk_kernel<16>, grid, block, 0, s, logits, T, E, k, topk_idx, topk_w);
  return hipGetLastError();
}

}  // namespace moe
