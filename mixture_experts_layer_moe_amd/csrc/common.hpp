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
  K_GATE_UP = 4, K_EXPERT_DOWN = 5, K_COMBINE = 6, K_LATENT_UP = 7, K_COUNT = 8
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

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

__host__ __device__ constexpr int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Upper bound of sum_e ceil(M_e / BM) over any routing of `rows` rows to E
// experts (each non-empty expert adds at most one partial tile).
inline int64_t grouped_mtile_bound(int64_t rows, int E, int BM) {
  const int64_t nonempty = rows < E ? rows : E;
  return (rows + nonempty * (BM - 1)) / BM;
}

}  // namespace moe
