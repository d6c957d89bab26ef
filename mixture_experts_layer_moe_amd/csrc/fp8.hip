// FP8 E4M3 support kernels: per-tensor absolute maximum of bf16 tensors,
// quantization with per-tensor scales, and the delayed-scaling update
// ("The Training and RL Infrastructure Behind MAI-Thinking-1", section 2,
// "Pre-training and mid-training precision": FP8 E4M3 forward GEMMs, delayed
// scaling over a 1,024-step amax history).
//
// Maxima are taken with integer atomic max on the bit patterns of
// non-negative floats, which order like unsigned integers: the result does
// not depend on the order of the updates.
#include <algorithm>

#include "launch.hpp"

namespace moe {

namespace {

constexpr float kE4M3Max = 448.0f;

__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  a = fminf(fmaxf(a, -kE4M3Max), kE4M3Max);
  b = fminf(fmaxf(b, -kE4M3Max), kE4M3Max);
  c = fminf(fmaxf(c, -kE4M3Max), kE4M3Max);
  d = fminf(fmaxf(d, -kE4M3Max), kE4M3Max);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// grid (blocks per tensor, tensors): 8 bf16 per thread per step
__global__ __launch_bounds__(256) void amax_bf16_kernel(const uint4* __restrict__ src,
                                                        int64_t n8, uint32_t* __restrict__ amax) {
  const uint4* p = src + (int64_t)blockIdx.y * n8;
  float m = 0.f;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (int64_t)gridDim.x * 256) {
    const uint4 v = p[i];
    m = fmaxf(m, fmaxf(fmaxf(fabsf(lo_bf16(v.x)), fabsf(hi_bf16(v.x))),
                       fmaxf(fabsf(lo_bf16(v.y)), fabsf(hi_bf16(v.y)))));
    m = fmaxf(m, fmaxf(fmaxf(fabsf(lo_bf16(v.z)), fabsf(hi_bf16(v.z))),
                       fmaxf(fabsf(lo_bf16(v.w)), fabsf(hi_bf16(v.w)))));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((threadIdx.x & 63) == 0 && m > 0.f) atomicMax(&amax[blockIdx.y], __float_as_uint(m));
}

__global__ __launch_bounds__(256) void quantize_e4m3_kernel(const uint4* __restrict__ src,
                                                            int64_t n8,
                                                            const float* __restrict__ scale,
                                                            uint2* __restrict__ dst) {
  const int64_t off = (int64_t)blockIdx.y * n8;
  const float sc = scale[blockIdx.y];
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (int64_t)gridDim.x * 256) {
    const uint4 v = src[off + i];
    uint2 q;
    q.x = e4m3x4(lo_bf16(v.x) * sc, hi_bf16(v.x) * sc, lo_bf16(v.y) * sc, hi_bf16(v.y) * sc);
    q.y = e4m3x4(lo_bf16(v.z) * sc, hi_bf16(v.z) * sc, lo_bf16(v.w) * sc, hi_bf16(v.w) * sc);
    dst[off + i] = q;
  }
}

__global__ __launch_bounds__(256) void zero_u32_kernel(uint32_t* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    p[i] = 0u;
}

// one thread per tensor: record the step's amax in its history slot, then the
// scale for the next step is 448 / (largest value in the history), 1 if the
// history is all zeros
__global__ __launch_bounds__(256) void scale_update_kernel(float* __restrict__ history,
                                                           const float* __restrict__ amax,
                                                           int64_t n, int H, int slot,
                                                           float* __restrict__ scale) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= n) return;
  float* h = history + t * H;
  h[slot] = amax[t];
  float m = 0.f;
  for (int i = 0; i < H; ++i) m = fmaxf(m, h[i]);
  scale[t] = m > 0.f ? kE4M3Max / m : 1.0f;
}

int blocks_for(int64_t n8) {
  const int64_t want = ceil_div(n8, 256);
  const int64_t cap = 4 * (int64_t)device_cu_count();
  return (int)(want < cap ? (want > 0 ? want : 1) : cap);
}

}  // namespace

hipError_t launch_zero_u32(uint32_t* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_u32_kernel, dim3((unsigned)std::min<int64_t>(ceil_div(n, 256), 1024)),
                     dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_amax_bf16(const uint16_t* src, int64_t ntensor, int64_t numel, uint32_t* amax,
                            hipStream_t s) {
  hipError_t e = launch_zero_u32(amax, ntensor, s);
  if (e != hipSuccess || numel == 0) return e;
  const int64_t n8 = numel / 8;
  const int bx = std::max(1, blocks_for(n8) / (int)std::min<int64_t>(ntensor, 64));
  hipLaunchKernelGGL(amax_bf16_kernel, dim3((unsigned)bx, (unsigned)ntensor), dim3(256), 0, s,
                     (const uint4*)src, n8, amax);
  return hipGetLastError();
}

hipError_t launch_quantize_e4m3(const uint16_t* src, int64_t ntensor, int64_t numel,
                                const float* scale, uint8_t* dst, hipStream_t s) {
  if (numel == 0) return hipSuccess;
  const int64_t n8 = numel / 8;
  const int bx = std::max(1, blocks_for(n8) / (int)std::min<int64_t>(ntensor, 64));
  hipLaunchKernelGGL(quantize_e4m3_kernel, dim3((unsigned)bx, (unsigned)ntensor), dim3(256), 0, s,
                     (const uint4*)src, n8, scale, (uint2*)dst);
  return hipGetLastError();
}

hipError_t launch_scale_update(float* history, const float* amax, int64_t n, int H, int slot,
                               float* scale, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(scale_update_kernel, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, s,
                     history, amax, n, H, slot, scale);
  return hipGetLastError();
}

}  // namespace moe
