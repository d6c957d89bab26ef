// Weighted combine in FP32 and the up-projection back to the hidden width
// ("The Training and RL Infrastructure Behind MAI-Thinking-1", section 2:
// the MoE combine and the residual stream are FP32; accumulations in a fixed
// order instead of atomics.  "MAI-Base-2: Microsoft's 2.8T base model...",
// section "The model": projected back up after the experts; the shared
// expert is added).
#include "launch.hpp"
#include "gemm.hpp"

namespace moe {

template <int EPI, int NSEG>
hipError_t dense_gemm_auto(GemmArgs a, int64_t M, hipStream_t s);   // expert.hip

// c[t, :] = sum_{j=0..k-1} w[t, j] * y[assign_row[t, j], :]   (fp32, j ascending)
// A gather (each output row read from its k expert rows), so no atomics and a
// fixed summation order.  One workgroup per token; 4 floats per thread step.
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y,
                                                      const float* __restrict__ w,
                                                      const int32_t* __restrict__ assign_row,
                                                      int64_t T, int L, int k,
                                                      uint16_t* __restrict__ c) {
  const int64_t t = blockIdx.x;
  __shared__ int rows[16];
  __shared__ float ws[16];
  if (threadIdx.x < k) {
    const int r = assign_row[t * k + threadIdx.x];
    rows[threadIdx.x] = (r >= 0 && (int64_t)r < T * k) ? r : 0;   // malformed -> row 0
    ws[threadIdx.x] = w[t * k + threadIdx.x];
  }
  __syncthreads();
  for (int l = threadIdx.x * 4; l < L; l += blockDim.x * 4) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; ++j) {
      const float4 v = *(const float4*)(y + (int64_t)rows[j] * L + l);
      const float wj = ws[j];
      acc.x += wj * v.x;
      acc.y += wj * v.y;
      acc.z += wj * v.z;
      acc.w += wj * v.w;
    }
    ushort4 o;
    o.x = f32_to_bf16_rne(acc.x);
    o.y = f32_to_bf16_rne(acc.y);
    o.z = f32_to_bf16_rne(acc.z);
    o.w = f32_to_bf16_rne(acc.w);
    *(ushort4*)(c + t * L + l) = o;
  }
}

hipError_t launch_combine(const float* y_rows, const float* topk_w, const int32_t* assign_row,
                          int64_t T, int L, int k, uint16_t* c, hipStream_t s) {
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)T), dim3(256), 0, s, y_rows, topk_w,
                     assign_row, T, L, k, c);
  return hipGetLastError();
}

hipError_t launch_latent_up(const uint16_t* c, const uint16_t* w_up, const uint16_t* hs,
                            const uint16_t* wsd, int64_t T, int d, int L, int Fs, float* out,
                            hipStream_t s) {
  GemmArgs a = {};
  a.seg[0].A = c; a.seg[0].lda = L; a.seg[0].B = w_up; a.seg[0].ldb = L; a.seg[0].K = L;
  a.nseg = 1;
  if (Fs > 0) {
    a.seg[1].A = hs; a.seg[1].lda = Fs; a.seg[1].B = wsd; a.seg[1].ldb = Fs; a.seg[1].K = Fs;
    a.nseg = 2;
  }
  a.N = d;
  a.C = out;
  a.ldc = d;
  if (Fs > 0) return dense_gemm_auto<EPI_F32, 2>(a, T, s);
  return dense_gemm_auto<EPI_F32, 1>(a, T, s);
}

}  // namespace moe
