// Shared device/host definitions of libmoe's HIP kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// Kernel ids of the profiling hook (same numbering as include/moe.h).
enum KernelId {
  K_ROUTER_GEMM = 0, K_ROUTER_TOPK = 1, K_PERMUTE = 2, K_LATENT_DOWN = 3,
  K_GATE_UP = 4, K_EXPERT_DOWN = 5, K_COMBINE = 6, K_LATENT_UP = 7, K_BWD_UP = 8,
  K_BWD_COMBINE = 9, K_BWD_DGRAD = 10, K_BWD_WGRAD = 11, K_BWD_LATENT = 12, K_BWD_ROUTER = 13,
  K_BWD_SHARED = 14, K_COUNT = 15
};

// Records the caller's start/stop events (if registered on this thread)
// around a group of launches.
struct EventScope {
  hipStream_t s;
  int id;
  EventScope(int id_, hipStream_t s_);
  ~EventScope();
};

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// The lowbias32 integer mixer (C. Wellons, hash prospector): two
// xorshift-multiply rounds and a final xorshift.  Host and device.
__host__ __device__ constexpr uint32_t lowbias32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// Key of random stream `stream` under `seed` for stochastic rounding.
__host__ __device__ constexpr uint32_t sr_stream_key(uint32_t seed, uint32_t stream) {
  return lowbias32(seed + 0x9E3779B9u * stream);
}

// fp32 -> bf16 bits by stochastic rounding: a uniform 16-bit integer r
// (counter-based: element index idx of the stream with key `key`) is added
// to the bit pattern and the low 16 bits dropped, so the magnitude rounds up
// with probability equal to the discarded fraction (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_sr(float f, uint32_t key, uint64_t idx) {
  uint32_t h = lowbias32((uint32_t)idx ^ key);
  h = lowbias32(h ^ (uint32_t)(idx >> 32));
  return (uint16_t)((__float_as_uint(f) + (h >> 16)) >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// FP8 E5M2 (OCP: exponent bias 15, 2 fraction bits, subnormals spaced 2^-16
// below 2^-14, largest finite 57344) of a gradient value v that is already
// scaled.  The magnitude saturates at 57344 (the hardware conversion does
// not).  Nearest (sr == 0): the hardware conversion, ties to even.
// Stochastic: at or above 2^-14 the top 21 bits of the stream's hash of
// element idx are added to the fp32 bit pattern of the magnitude and the low
// 21 bits dropped (round up with probability equal to the discarded
// fraction; the result is exactly an E5M2 value, so the conversion that
// follows is exact); below 2^-14 to nearest.  The hash is the one of
// f32_to_bf16_sr.
__device__ __forceinline__ uint8_t f32_to_e5m2(float v, int sr, uint32_t key, uint64_t idx) {
  constexpr float E5M2_MAX = 57344.0f;
  float a = fminf(fabsf(v), E5M2_MAX);
  if (sr && a >= 0x1p-14f) {
    uint32_t h = lowbias32((uint32_t)idx ^ key);
    h = lowbias32(h ^ (uint32_t)(idx >> 32));
    a = __uint_as_float((__float_as_uint(a) + (h >> 11)) & 0xFFE00000u);
  }
  return (uint8_t)(__builtin_amdgcn_cvt_pk_bf8_f32(copysignf(a, v), 0.0f, 0, false) & 0xff);
}

// Largest finite E5M2 value over the largest E4M3 value: a gradient whose
// scale s follows the E4M3 convention (s = 448 / amax) enters E5M2 scaled by
// 128 s (exact: a power of two times s).
constexpr float E5M2_OVER_E4M3 = 128.0f;

__host__ __device__ constexpr int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Upper bound of sum_e ceil(M_e / BM) over any routing of `rows` rows to E
// experts (each non-empty expert adds at most one partial tile).
inline int64_t grouped_mtile_bound(int64_t rows, int E, int BM) {
  const int64_t nonempty = rows < E ? rows : E;
  return (rows + nonempty * (BM - 1)) / BM;
}

}  // namespace moe
