// Device side of the seeded synthetic-input generator (not part of the layer):
// out[i] = table[hash(key, start + i) >> 16], the same function as
// moe_synth/gen.py evaluates with numpy.  hash = two rounds of the lowbias32
// integer mixer (Chris Wellons, "Prospecting for Hash Functions", 2018) over
// the low and high 32-bit words of the element index.
#include <hip/hip_runtime.h>
#include <stdint.h>

__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7FEB352Du;
  x ^= x >> 15;
  x *= 0x846CA68Bu;
  x ^= x >> 16;
  return x;
}

__global__ void synth_fill_kernel(uint16_t* __restrict__ out, int64_t n, int64_t start,
                                  uint32_t k0, uint32_t k1, const uint16_t* __restrict__ table) {
  const int64_t i0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (i0 >= n) return;
  uint16_t v[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const uint64_t idx = (uint64_t)(start + i0 + q);
    uint32_t h = mix32((uint32_t)idx ^ k0);
    h = mix32(h ^ (uint32_t)(idx >> 32) ^ k1);
    v[q] = table[h >> 16];
  }
  if (i0 + 8 <= n && ((uintptr_t)(out + i0) & 15) == 0) {
    uint4 p;
    p.x = v[0] | ((uint32_t)v[1] << 16);
    p.y = v[2] | ((uint32_t)v[3] << 16);
    p.z = v[4] | ((uint32_t)v[5] << 16);
    p.w = v[6] | ((uint32_t)v[7] << 16);
    *(uint4*)(out + i0) = p;
  } else {
    for (int q = 0; q < 8 && i0 + q < n; ++q) out[i0 + q] = v[q];
  }
}

extern "C" int synth_fill_bf16(uint16_t* out, int64_t n, int64_t start, uint32_t k0, uint32_t k1,
                               const uint16_t* table, void* stream) {
  if (n <= 0) return 0;
  const int64_t threads = (n + 7) / 8;
  const int64_t blocks = (threads + 255) / 256;
  hipLaunchKernelGGL(synth_fill_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                     out, n, start, k0, k1, table);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// Plain device copy of n 16-byte words in one dispatch, used only to calibrate
// HBM byte counters (a kernel with known traffic: 16*n bytes read, 16*n written).
__global__ void synth_calib_copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                        int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

extern "C" int synth_calib_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  if (bytes <= 0 || (bytes & 15)) return -1;
  hipLaunchKernelGGL(synth_calib_copy_kernel, dim3(4096), dim3(256), 0, (hipStream_t)stream,
                     (const uint4*)src, (uint4*)dst, bytes / 16);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}
