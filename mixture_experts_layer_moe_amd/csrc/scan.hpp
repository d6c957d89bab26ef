// Workgroup-wide exclusive prefix sum of one int per thread (up to 1024
// threads = 16 waves of 64), in a fixed order (deterministic).
#pragma once

#include "common.hpp"

namespace moe {

// Returns the exclusive prefix of `v` over threads 0..threadIdx.x-1 and
// writes the workgroup total to *total.  All threads of the block must call it.
__device__ inline int block_exclusive_scan(int v, int* total) {
  __shared__ int wave_sum[16];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nwaves = (blockDim.x + 63) >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int n = __shfl_up(incl, o);
    if (lane >= o) incl += n;
  }
  if (lane == 63) wave_sum[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    int s = lane < nwaves ? wave_sum[lane] : 0;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const int n = __shfl_up(s, o);
      if (lane >= o) s += n;
    }
    if (lane < nwaves) wave_sum[lane] = s;   // inclusive over waves
  }
  __syncthreads();
  const int before = wave > 0 ? wave_sum[wave - 1] : 0;
  *total = wave_sum[nwaves - 1];
  __syncthreads();   // wave_sum may be reused by a later call
  return before + incl - v;
}

}  // namespace moe
