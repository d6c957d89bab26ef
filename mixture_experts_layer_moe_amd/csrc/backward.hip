// Backward pass of the LatentMoE layer: the non-GEMM kernels (gradient casts
// with round-to-nearest or stochastic rounding, padded transposes, combine
// and gather backward, router softmax backward, FP32 router GEMMs) and the
// backward GEMM launchers.
//
// Pages: "The Training and RL Infrastructure Behind MAI-Thinking-1",
// section 2 "Numerics", "Pre-training and mid-training precision" (weight
// gradients BF16 with FP32 accumulation; router and MoE combine FP32;
// stochastic rounding whenever a gradient is cast to lower precision),
// section 2 "Bitwise determinism" (fixed-order accumulation, no atomics),
// section 3 "Custom kernels" (one kernel writes a tensor and its transpose,
// since the backward needs both) and "Checkpointing and offloading" (finer
// recomputation inside a layer: the experts' gate/up activations are
// recomputed here, not stored by the forward).
#include "launch.hpp"
#include "gemm.hpp"
#include "scan.hpp"

namespace moe {

template <int EPI, int NSEG>
hipError_t dense_gemm_auto(GemmArgs a, int64_t M, hipStream_t s);   // expert.hip

__device__ __forceinline__ uint16_t round_grad(float v, int sr, uint32_t key, uint64_t idx) {
  return sr ? f32_to_bf16_sr(v, key, idx) : f32_to_bf16_rne(v);
}

// ---------------------------------------------------------------------------
// fp32 -> bf16 gradient cast (element index = flat row-major index)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void cvt_grad_kernel(const float* __restrict__ src, int64_t n,
                                                       int sr, uint32_t key,
                                                       uint16_t* __restrict__ dst) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x * 4;
  for (int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4; i < n; i += stride) {
    const float4 v = *(const float4*)(src + i);
    ushort4 o;
    o.x = round_grad(v.x, sr, key, (uint64_t)i);
    o.y = round_grad(v.y, sr, key, (uint64_t)i + 1);
    o.z = round_grad(v.z, sr, key, (uint64_t)i + 2);
    o.w = round_grad(v.w, sr, key, (uint64_t)i + 3);
    *(ushort4*)(dst + i) = o;
  }
}

hipError_t launch_cvt_grad(const float* src, int64_t n, int sr, uint32_t key, uint16_t* dst,
                           hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = ceil_div(n / 4, 256);
  hipLaunchKernelGGL(cvt_grad_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256),
                     0, s, src, n, sr, key, dst);
  return hipGetLastError();
}

// fp32 -> E5M2 gradient cast: dst[i] = e5m2(src[i] * 128 scale[0]) with the
// gradient rounding (element index = flat index); n a multiple of 4.
__global__ __launch_bounds__(256) void cvt_e5m2_kernel(const float* __restrict__ src, int64_t n,
                                                       const float* __restrict__ scale, int sr,
                                                       uint32_t key, uint8_t* __restrict__ dst) {
  const float s5 = E5M2_OVER_E4M3 * scale[0];
  const int64_t stride = (int64_t)gridDim.x * blockDim.x * 4;
  for (int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4; i < n; i += stride) {
    const float4 v = *(const float4*)(src + i);
    uchar4 o;
    o.x = f32_to_e5m2(v.x * s5, sr, key, (uint64_t)i);
    o.y = f32_to_e5m2(v.y * s5, sr, key, (uint64_t)i + 1);
    o.z = f32_to_e5m2(v.z * s5, sr, key, (uint64_t)i + 2);
    o.w = f32_to_e5m2(v.w * s5, sr, key, (uint64_t)i + 3);
    *(uchar4*)(dst + i) = o;
  }
}

hipError_t launch_cvt_e5m2(const float* src, int64_t n, const float* scale, int sr, uint32_t key,
                           uint8_t* dst, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = ceil_div(n / 4, 256);
  hipLaunchKernelGGL(cvt_e5m2_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256),
                     0, s, src, n, scale, sr, key, dst);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// padded K layout of the per-expert weight-gradient GEMMs: expert e's rows
// become columns [kpre[e], kpre[e] + rows_e) of a transposed matrix, each
// expert's range padded with zero columns to a multiple of 64 (the GEMM's
// K stage width), kpre[E] the padded total
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void kpad_prefix_kernel(const int32_t* __restrict__ offsets,
                                                           const int32_t* __restrict__ ends,
                                                           int E, int32_t* __restrict__ kpre) {
  const int e = threadIdx.x;
  // expert e's rows: offsets[e] .. ends[e] (ends null: offsets[e + 1])
  const int rows = e < E ? (ends ? ends[e] : offsets[e + 1]) - offsets[e] : 0;
  int total;
  const int ex = block_exclusive_scan((rows + 63) / 64 * 64, &total);
  if (e < E) kpre[e] = ex;
  if (e == 0) kpre[E] = total;
}

hipError_t launch_kpad_prefix(const int32_t* offsets, int E, int32_t* kpre, hipStream_t s,
                              const int32_t* ends) {
  hipLaunchKernelGGL(kpad_prefix_kernel, dim3(1), dim3(1024), 0, s, offsets, ends, E, kpre);
  return hipGetLastError();
}

// Transpose of a bf16 matrix through LDS in 64 x 64 tiles, into the padded
// K layout.  Source rows of group e: off[e] .. off_end[e] (off_end null:
// off[e + 1]) (rows of src, or
// rows gather[r] of src when gather is given); they land in destination
// columns kpre[e] .. and the rest of the group's padded range is zero.
// Without groups (off == nullptr) the single group is rows 0 .. nrows with
// padded extent ldd.  grid: x = padded 64-column chunks, y = source column
// chunks, z = batch (src / dst advance by the batch strides).
__global__ __launch_bounds__(256) void transpose_pad_kernel(
    const uint16_t* __restrict__ src, int64_t lds_, const int32_t* __restrict__ gather,
    int64_t gather_rows, int C, const int32_t* __restrict__ off,
    const int32_t* __restrict__ off_end, const int32_t* __restrict__ kpre, int G, int64_t nrows,
    uint16_t* __restrict__ dst, int64_t ldd, int64_t src_batch, int64_t dst_batch) {
  __shared__ uint16_t tile[64][66];
  const int64_t kc0 = (int64_t)blockIdx.x * 64;     // first padded destination column
  const int c0 = blockIdx.y * 64;                    // first source column
  src += (int64_t)blockIdx.z * src_batch;
  dst += (int64_t)blockIdx.z * dst_batch;
  int64_t r_begin, r_end;                            // source rows of this chunk's group
  int64_t k_begin;                                   // padded column of r_begin
  if (off == nullptr) {
    if (kc0 >= ldd) return;
    r_begin = 0;
    r_end = nrows;
    k_begin = 0;
  } else {
    const int64_t ktot = kpre[G];
    if (kc0 >= ktot) return;
    int lo = 0, hi = G - 1;                          // largest e with kpre[e] <= kc0
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (kpre[mid] <= kc0) lo = mid; else hi = mid - 1;
    }
    r_begin = off[lo];
    r_end = off_end ? off_end[lo] : off[lo + 1];
    k_begin = kpre[lo];
  }
  const int tid = threadIdx.x;
  // load: 64 source rows x 64 columns, 8 threads per row, 8 values each
  for (int pass = 0; pass < 2; ++pass) {
    const int i = pass * 32 + (tid >> 3);
    const int cc = (tid & 7) * 8;
    const int64_t r = r_begin + (kc0 - k_begin) + i;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r < r_end && c0 + cc < C) {
      int64_t sr = r;
      if (gather != nullptr) {
        sr = gather[r];
        if (sr < 0 || sr >= gather_rows) sr = 0;   // malformed metadata: row 0
      }
      v = *(const uint4*)(src + sr * lds_ + c0 + cc);
    }
    const uint16_t* pv = (const uint16_t*)&v;
#pragma unroll
    for (int q = 0; q < 8; ++q) tile[i][cc + q] = pv[q];
  }
  __syncthreads();
  // store: destination rows c0 .. c0 + 63, 64 padded columns from kc0
  for (int pass = 0; pass < 2; ++pass) {
    const int c = pass * 32 + (tid >> 3);
    const int ii = (tid & 7) * 8;
    if (c0 + c >= C) continue;
    uint4 v;
    uint16_t* pv = (uint16_t*)&v;
#pragma unroll
    for (int q = 0; q < 8; ++q) pv[q] = tile[ii + q][c];
    *(uint4*)(dst + (int64_t)(c0 + c) * ldd + kc0 + ii) = v;
  }
}

// dense: src [nrows, C] -> dst [C, ldd] (ldd >= ceil64(nrows), zero padded)
hipError_t launch_transpose_dense(const uint16_t* src, int64_t nrows, int C, uint16_t* dst,
                                  int64_t ldd, int batch, int64_t src_batch, int64_t dst_batch,
                                  hipStream_t s) {
  if (nrows <= 0 || C <= 0) return hipSuccess;
  hipLaunchKernelGGL(transpose_pad_kernel, dim3((unsigned)(ldd / 64), (unsigned)ceil_div(C, 64),
                                                (unsigned)batch),
                     dim3(256), 0, s, src, (int64_t)C, (const int32_t*)nullptr, (int64_t)0, C,
                     (const int32_t*)nullptr, (const int32_t*)nullptr, (const int32_t*)nullptr, 0,
                     nrows, dst, ldd, src_batch, dst_batch);
  return hipGetLastError();
}

// grouped: rows of E experts (src rows, or rows gather[r] of a src with
// gather_rows rows; expert e's rows offsets[e] .. ends[e], ends null:
// offsets[e + 1]) -> dst [C, ldd] in the padded K layout kpre
hipError_t launch_transpose_grouped(const uint16_t* src, const int32_t* gather, int64_t gather_rows,
                                    int C, const int32_t* offsets, const int32_t* kpre, int E,
                                    uint16_t* dst, int64_t ldd, hipStream_t s,
                                    const int32_t* ends) {
  hipLaunchKernelGGL(transpose_pad_kernel, dim3((unsigned)(ldd / 64), (unsigned)ceil_div(C, 64), 1),
                     dim3(256), 0, s, src, (int64_t)C, gather, gather_rows, C, offsets, ends, kpre,
                     E, (int64_t)0, dst, ldd, (int64_t)0, (int64_t)0);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// combine backward: for each (t, j), r = assign_row[t, j]:
//   dy[r] = w[t, j] dc[t]            (FP32, then cast to bf16 for the GEMMs)
//   dw[t, j] = dc[t] . y[r]          (FP32, fixed-order reduction)
// One workgroup per token.  Q8 (FP8 data gradients) also writes dy as E5M2
// codes (dy8, scale 128 grad_scale[0], stream key key8) and records max |dy|
// in grad_amax[0] (one integer atomic max per wave: order-independent).
// ---------------------------------------------------------------------------
template <bool Q8>
__global__ __launch_bounds__(256) void combine_bwd_kernel(
    const float* __restrict__ dc, const float* __restrict__ y, const float* __restrict__ w,
    const int32_t* __restrict__ assign_row, int64_t T, int L, int k, int sr, uint32_t key,
    uint16_t* __restrict__ dy_b, float* __restrict__ dw, uint8_t* __restrict__ dy8,
    const float* __restrict__ grad_scale, uint32_t key8, uint32_t* __restrict__ grad_amax) {
  const int64_t t = blockIdx.x;
  const float s5 = Q8 ? E5M2_OVER_E4M3 * grad_scale[0] : 1.f;
  float amax = 0.f;
  __shared__ int rows[16];
  __shared__ float ws[16];
  __shared__ float red[16][4];
  const int tid = threadIdx.x;
  if (tid < k) {
    const int r = assign_row[t * k + tid];
    rows[tid] = (r >= 0 && (int64_t)r < T * k) ? r : 0;
    ws[tid] = w[t * k + tid];
  }
  __syncthreads();
  float part[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) part[j] = 0.f;
  for (int l = tid * 4; l < L; l += 256 * 4) {
    const float4 g = *(const float4*)(dc + t * L + l);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (j >= k) break;
      const int64_t r = rows[j];
      const float wj = ws[j];
      const float4 yv = *(const float4*)(y + r * L + l);
      part[j] += g.x * yv.x + g.y * yv.y + g.z * yv.z + g.w * yv.w;
      const uint64_t o = (uint64_t)(r * L + l);
      ushort4 q;
      q.x = round_grad(wj * g.x, sr, key, o);
      q.y = round_grad(wj * g.y, sr, key, o + 1);
      q.z = round_grad(wj * g.z, sr, key, o + 2);
      q.w = round_grad(wj * g.w, sr, key, o + 3);
      *(ushort4*)(dy_b + r * L + l) = q;
      if constexpr (Q8) {
        const float4 dv = make_float4(wj * g.x, wj * g.y, wj * g.z, wj * g.w);
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(dv.x), fabsf(dv.y)), fmaxf(fabsf(dv.z), fabsf(dv.w))));
        uchar4 q8;
        q8.x = f32_to_e5m2(dv.x * s5, sr, key8, o);
        q8.y = f32_to_e5m2(dv.y * s5, sr, key8, o + 1);
        q8.z = f32_to_e5m2(dv.z * s5, sr, key8, o + 2);
        q8.w = f32_to_e5m2(dv.w * s5, sr, key8, o + 3);
        *(uchar4*)(dy8 + r * L + l) = q8;
      }
    }
  }
  // fixed-order reduction: wave tree, then the 4 wave sums in order
  const int lane = tid & 63, wave = tid >> 6;
  if constexpr (Q8) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    if (lane == 0 && amax > 0.f) atomicMax(grad_amax, __float_as_uint(amax));
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (j >= k) break;
    float v = part[j];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    if (lane == 0) red[j][wave] = v;
  }
  __syncthreads();
  if (tid < k) dw[t * k + tid] = ((red[tid][0] + red[tid][1]) + red[tid][2]) + red[tid][3];
}

hipError_t launch_combine_bwd(const float* dc, const float* y_rows, const float* topk_w,
                              const int32_t* assign_row, int64_t T, int L, int k, int sr,
                              uint32_t key, uint16_t* dy_b, float* dw, hipStream_t s) {
  hipLaunchKernelGGL(combine_bwd_kernel<false>, dim3((unsigned)T), dim3(256), 0, s, dc, y_rows,
                     topk_w, assign_row, T, L, k, sr, key, dy_b, dw, (uint8_t*)nullptr,
                     (const float*)nullptr, 0u, (uint32_t*)nullptr);
  return hipGetLastError();
}

hipError_t launch_combine_bwd_q8(const float* dc, const float* y_rows, const float* topk_w,
                                 const int32_t* assign_row, int64_t T, int L, int k, int sr,
                                 uint32_t key, uint16_t* dy_b, float* dw, uint8_t* dy8,
                                 const float* grad_scale, uint32_t key8, uint32_t* grad_amax,
                                 hipStream_t s) {
  hipLaunchKernelGGL(combine_bwd_kernel<true>, dim3((unsigned)T), dim3(256), 0, s, dc, y_rows,
                     topk_w, assign_row, T, L, k, sr, key, dy_b, dw, dy8, grad_scale, key8,
                     grad_amax);
  return hipGetLastError();
}

// dz[t] = sum_{j=0..k-1} dzp[assign_row[t, j]]   (FP32, j ascending), cast
// to bf16 for the GEMMs.  One workgroup per token.
__global__ __launch_bounds__(256) void gather_sum_kernel(const float* __restrict__ dzp,
                                                         const int32_t* __restrict__ assign_row,
                                                         int64_t T, int L, int k, int sr,
                                                         uint32_t key,
                                                         uint16_t* __restrict__ dz_b) {
  const int64_t t = blockIdx.x;
  __shared__ int rows[16];
  if (threadIdx.x < k) {
    const int r = assign_row[t * k + threadIdx.x];
    rows[threadIdx.x] = (r >= 0 && (int64_t)r < T * k) ? r : 0;
  }
  __syncthreads();
  for (int l = threadIdx.x * 4; l < L; l += blockDim.x * 4) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; ++j) {
      const float4 v = *(const float4*)(dzp + (int64_t)rows[j] * L + l);
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
    const uint64_t o = (uint64_t)(t * L + l);
    ushort4 q;
    q.x = round_grad(acc.x, sr, key, o);
    q.y = round_grad(acc.y, sr, key, o + 1);
    q.z = round_grad(acc.z, sr, key, o + 2);
    q.w = round_grad(acc.w, sr, key, o + 3);
    *(ushort4*)(dz_b + t * L + l) = q;
  }
}

hipError_t launch_gather_sum(const float* dzp, const int32_t* assign_row, int64_t T, int L, int k,
                             int sr, uint32_t key, uint16_t* dz_b, hipStream_t s) {
  hipLaunchKernelGGL(gather_sum_kernel, dim3((unsigned)T), dim3(256), 0, s, dzp, assign_row, T, L,
                     k, sr, key, dz_b);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// router: gradient of the logits through the softmax, for the gradient dw
// of the selected (not renormalised) probabilities:
//   p = softmax(logits_t),  s = sum_j p[idx_j] dw_j,
//   dl[e] = p[e] ((dw_j if e == idx_j) - s)          (FP32)
// One wave per token, four tokens per workgroup.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void router_bwd_kernel(const float* __restrict__ logits,
                                                         const int32_t* __restrict__ idx,
                                                         const float* __restrict__ dw, int64_t T,
                                                         int E, int k, float* __restrict__ dl) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* lt = logits + t * E;
  float m = -INFINITY;
  for (int e = lane; e < E; e += 64) m = fmaxf(m, lt[e]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  float sum = 0.f;
  for (int e = lane; e < E; e += 64) sum += __expf(lt[e] - m);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
  const float inv = 1.0f / sum;
  // s = sum_j p[idx_j] dw_j, the same value in every lane (fixed order j)
  float sdot = 0.f;
  for (int j = 0; j < k; ++j) {
    int e = idx[t * k + j];
    if (e < 0 || e >= E) e = 0;
    sdot += __expf(lt[e] - m) * inv * dw[t * k + j];
  }
  for (int e = lane; e < E; e += 64) {
    float dp = 0.f;
    for (int j = 0; j < k; ++j)
      if (idx[t * k + j] == e) dp = dw[t * k + j];
    const float p = __expf(lt[e] - m) * inv;
    dl[t * E + e] = p * (dp - sdot);
  }
}

hipError_t launch_router_bwd(const float* logits, const int32_t* idx, const float* dw, int64_t T,
                             int E, int k, float* dl, hipStream_t s) {
  hipLaunchKernelGGL(router_bwd_kernel, dim3((unsigned)ceil_div(T, 4)), dim3(256), 0, s, logits,
                     idx, dw, T, E, k, dl);
  return hipGetLastError();
}

// FP32 GEMM on the vector ALUs (the router is FP32 on the pages):
//   C[m, n] (+)= sum_k A(m, k) B(k, n),  A(m, k) = A[m sam + k sak],
//   B(k, n) = B[k ldb + n] (TB = float or bf16 bits).
// 64 x 64 tiles, K steps of 16, 4 x 4 outputs per thread; each output is
// written by one thread (no atomics, fixed order).  Split K: workgroup z
// covers K range [z k_chunk, (z + 1) k_chunk) and writes its partial result
// to C + z c_split (a fixed-order sum of the partials follows).
template <typename TB, bool A_MCONTIG>
__global__ __launch_bounds__(256) void f32_gemm_kernel(const float* __restrict__ A, int64_t sam,
                                                       int64_t sak, const TB* __restrict__ B,
                                                       int64_t ldb, int64_t M, int64_t N,
                                                       int64_t K, float* __restrict__ C,
                                                       int64_t ldc, int accumulate,
                                                       int64_t k_chunk, int64_t c_split) {
  __shared__ float As[16][64 + 4];
  __shared__ float Bs[16][64 + 4];
  const int tid = threadIdx.x;
  const int64_t m0 = (int64_t)blockIdx.y * 64, n0 = (int64_t)blockIdx.x * 64;
  const int ty = tid >> 4, tx = tid & 15;
  float acc[4][4] = {};
  const int64_t kb0 = (int64_t)blockIdx.z * k_chunk;
  const int64_t kend = kb0 + k_chunk < K ? kb0 + k_chunk : K;
  C += (int64_t)blockIdx.z * c_split;
  for (int64_t k0 = kb0; k0 < kend; k0 += 16) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = tid + 256 * q;
      int mm, kk;
      if (A_MCONTIG) { mm = e & 63; kk = e >> 6; }
      else { kk = e & 15; mm = e >> 4; }
      const int64_t gm = m0 + mm, gk = k0 + kk;
      As[kk][mm] = (gm < M && gk < kend) ? A[gm * sam + gk * sak] : 0.f;
      const int nn = e & 63, kb = e >> 6;
      const int64_t gn = n0 + nn, gkb = k0 + kb;
      float bv = 0.f;
      if (gn < N && gkb < kend) {
        if constexpr (sizeof(TB) == 2) bv = bf16_to_f32(B[gkb * ldb + gn]);
        else bv = B[gkb * ldb + gn];
      }
      Bs[kb][nn] = bv;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t gm = m0 + ty * 4 + i;
    if (gm >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t gn = n0 + tx * 4 + j;
      if (gn >= N) continue;
      float* p = C + gm * ldc + gn;
      *p = accumulate ? *p + acc[i][j] : acc[i][j];
    }
  }
}

// dx += dl W_r  (M = T, N = d, K = E; dl [T, E], W_r [E, d] fp32)
hipError_t launch_router_dx(const float* dl, const float* w_router, int64_t T, int d, int E,
                            float* dx, hipStream_t s) {
  hipLaunchKernelGGL((f32_gemm_kernel<float, false>),
                     dim3((unsigned)ceil_div(d, 64), (unsigned)ceil_div(T, 64)), dim3(256), 0, s,
                     dl, (int64_t)E, (int64_t)1, w_router, (int64_t)d, T, (int64_t)d, (int64_t)E,
                     dx, (int64_t)d, 1, (int64_t)E, (int64_t)0);
  return hipGetLastError();
}

// dW_r = dl^T x  (M = E, N = d, K = T; x bf16 [T, d]).  K (the tokens) is
// split into chunks of ROUTER_DW_CHUNK tokens whose partial sums are added in chunk
// order by a second kernel.
constexpr int64_t ROUTER_DW_CHUNK = 1024;
int64_t router_dw_partial_floats(int64_t T, int d, int E) {
  return ceil_div(T, ROUTER_DW_CHUNK) * (int64_t)E * d;
}
__global__ __launch_bounds__(256) void sum_partials_kernel(const float* __restrict__ part,
                                                           int64_t nsplit, int64_t n,
                                                           float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float acc = 0.f;
  for (int64_t z = 0; z < nsplit; ++z) acc += part[z * n + i];
  out[i] = acc;
}
hipError_t launch_router_dw(const float* dl, const uint16_t* x, int64_t T, int d, int E,
                            float* part, float* dw_router, hipStream_t s) {
  const int64_t nsplit = ceil_div(T, ROUTER_DW_CHUNK);
  const int64_t n = (int64_t)E * d;
  hipLaunchKernelGGL((f32_gemm_kernel<uint16_t, true>),
                     dim3((unsigned)ceil_div(d, 64), (unsigned)ceil_div(E, 64), (unsigned)nsplit),
                     dim3(256), 0, s, dl, (int64_t)1, (int64_t)E, x, (int64_t)d, (int64_t)E,
                     (int64_t)d, T, part, (int64_t)d, 0, ROUTER_DW_CHUNK, n);
  hipLaunchKernelGGL(sum_partials_kernel, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, s, part,
                     nsplit, n, dw_router);
  return hipGetLastError();
}

// db[e] = sum_t dl[t, e]: per-chunk partial sums (256 tokens each), then the
// partials in chunk order.
constexpr int DB_CHUNK = 256;
__global__ __launch_bounds__(256) void colsum_part_kernel(const float* __restrict__ dl, int64_t T,
                                                          int E, float* __restrict__ part) {
  const int64_t t0 = (int64_t)blockIdx.x * DB_CHUNK;
  const int64_t t1 = t0 + DB_CHUNK < T ? t0 + DB_CHUNK : T;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    float acc = 0.f;
    for (int64_t t = t0; t < t1; ++t) acc += dl[t * E + e];
    part[(int64_t)blockIdx.x * E + e] = acc;
  }
}
__global__ __launch_bounds__(256) void colsum_final_kernel(const float* __restrict__ part,
                                                           int64_t nchunk, int E,
                                                           float* __restrict__ db) {
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    float acc = 0.f;
    for (int64_t c = 0; c < nchunk; ++c) acc += part[c * E + e];
    db[e] = acc;
  }
}
int64_t router_db_partial_floats(int64_t T, int E) { return ceil_div(T, DB_CHUNK) * E; }
hipError_t launch_router_db(const float* dl, int64_t T, int E, float* part, float* db,
                            hipStream_t s) {
  const int64_t nchunk = ceil_div(T, DB_CHUNK);
  hipLaunchKernelGGL(colsum_part_kernel, dim3((unsigned)nchunk), dim3(256), 0, s, dl, T, E, part);
  hipLaunchKernelGGL(colsum_final_kernel, dim3(1), dim3(256), 0, s, part, nchunk, E, db);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// bf16 MFMA GEMMs of the backward (all C = A B^T with K-contiguous operands)
// ---------------------------------------------------------------------------

// dense: C[M, N] fp32 = A[M, K] B[N, K]^T
hipError_t launch_dense_f32(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                            int64_t K, int64_t M, int N, float* C, int64_t ldc, hipStream_t s) {
  GemmArgs a = {};
  a.seg[0].A = A; a.seg[0].lda = lda; a.seg[0].B = B; a.seg[0].ldb = ldb; a.seg[0].K = (int)K;
  a.nseg = 1;
  a.N = N;
  a.C = C;
  a.ldc = ldc;
  return dense_gemm_auto<EPI_F32, 1>(a, M, s);
}

hipError_t launch_dense_f32_add2(const uint16_t* A1, int64_t lda1, const uint16_t* B1,
                                 int64_t ldb1, int64_t K1, const uint16_t* A2, int64_t lda2,
                                 const uint16_t* B2, int64_t ldb2, int64_t K2, int64_t M, int N,
                                 float* C, int64_t ldc, hipStream_t s) {
  GemmArgs a = {};
  a.seg[0].A = A1; a.seg[0].lda = lda1; a.seg[0].B = B1; a.seg[0].ldb = ldb1; a.seg[0].K = (int)K1;
  a.seg[1].A = A2; a.seg[1].lda = lda2; a.seg[1].B = B2; a.seg[1].ldb = ldb2; a.seg[1].K = (int)K2;
  a.nseg = 2;
  a.N = N;
  a.C = C;
  a.ldc = ldc;
  return dense_gemm_auto<EPI_F32_ADD, 2>(a, M, s);
}

// per-expert weight gradient: C_e[M, N] = A[:, K_e] B[:, K_e]^T, K_e expert
// e's padded column range kpre[e] .. kpre[e + 1] of A [M, lda] and B [N, ldb]
hipError_t launch_kgrouped_f32(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                               const int32_t* kpre, int E, int M, int N, float* C,
                               int64_t c_expert_stride, hipStream_t s, bool accumulate) {
  using Cfg = TileBig;
  GemmArgs a = {};
  a.seg[0].A = A; a.seg[0].lda = lda; a.seg[0].B = B; a.seg[0].ldb = ldb; a.seg[0].K = 0;
  a.nseg = 1;
  a.M = M;
  a.N = N;
  a.E = E;
  a.kpre = kpre;
  a.C = C;
  a.ldc = N;
  a.c_expert_stride = c_expert_stride;
  a.m_tiles = (int)ceil_div(M, Cfg::bm);
  a.n_tiles = (int)ceil_div(N, Cfg::bn);
  if (accumulate)
    return launch_gemm<Cfg, false, false, EPI_F32_ADD, 1, F8_NONE, true>(
        a, (int64_t)E * a.m_tiles * a.n_tiles, s);
  return launch_gemm<Cfg, false, false, EPI_F32, 1, F8_NONE, true>(
      a, (int64_t)E * a.m_tiles * a.n_tiles, s);
}

}  // namespace moe
