// Permutation of (token, slot) assignments into expert order: a stable
// counting sort by expert, the "expert encode" step ("The Training and RL
// Infrastructure Behind MAI-Thinking-1", section 3 "Custom kernels"), with the
// token metadata left on the device ("Frontier Pre-training at Microsoft AI",
// "Reducing per-expert overhead").
//
// Deterministic with no order-dependent atomics: each workgroup takes a chunk
// of 256 tokens and builds, in LDS, one 256-bit membership mask per expert
// (bit i set <=> token i of the chunk selected that expert; the OR is
// order-independent).  Popcounts of the masks give the chunk's per-expert
// counts; a single scan workgroup turns the counts into expert offsets and
// per-chunk bases; a token's rank inside its expert is the popcount of the
// mask bits below it, so rows keep ascending token order within an expert.
#include <mutex>

#include "launch.hpp"
#include "scan.hpp"

namespace moe {

__device__ inline void build_masks(const int32_t* __restrict__ idx, int64_t T, int k, int E,
                                   uint32_t* mask) {
  const int tid = threadIdx.x;
  for (int i = tid; i < E * 8; i += PERM_CHUNK) mask[i] = 0u;
  __syncthreads();
  const int64_t t = (int64_t)blockIdx.x * PERM_CHUNK + tid;
  if (t < T) {
    const uint32_t bit = 1u << (tid & 31);
    for (int j = 0; j < k; ++j) {
      const int e = idx[t * k + j];
      if ((unsigned)e < (unsigned)E) atomicOr(&mask[e * 8 + (tid >> 5)], bit);
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(PERM_CHUNK) void perm_count_kernel(const int32_t* __restrict__ idx,
                                                                int64_t T, int k, int E,
                                                                int32_t* __restrict__ chunk_counts) {
  extern __shared__ uint32_t mask[];
  build_masks(idx, T, k, E, mask);
  int32_t* out = chunk_counts + (int64_t)blockIdx.x * E;
  for (int e = threadIdx.x; e < E; e += PERM_CHUNK) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < 8; ++w) c += __popc(mask[e * 8 + w]);
    out[e] = c;
  }
}

__global__ __launch_bounds__(1024) void perm_scan_kernel(const int32_t* __restrict__ chunk_counts,
                                                         int64_t nchunks, int E,
                                                         int32_t* __restrict__ counts,
                                                         int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ chunk_base) {
  const int e = threadIdx.x;
  int tot = 0;
  if (e < E) {
#pragma unroll 8
    for (int64_t ch = 0; ch < nchunks; ++ch) tot += chunk_counts[ch * E + e];
  }
  int total;
  const int excl = block_exclusive_scan(tot, &total);
  if (e < E) {
    counts[e] = tot;
    offsets[e] = excl;
    int run = excl;
#pragma unroll 8
    for (int64_t ch = 0; ch < nchunks; ++ch) {
      chunk_base[ch * E + e] = run;
      run += chunk_counts[ch * E + e];
    }
  }
  if (e == 0) offsets[E] = total;
}

__global__ __launch_bounds__(PERM_CHUNK) void perm_scatter_kernel(
    const int32_t* __restrict__ idx, int64_t T, int k, int E,
    const int32_t* __restrict__ chunk_base, int32_t* __restrict__ assign_row,
    int32_t* __restrict__ row_token) {
  extern __shared__ uint32_t mask[];
  build_masks(idx, T, k, E, mask);
  const int tid = threadIdx.x;
  const int64_t t = (int64_t)blockIdx.x * PERM_CHUNK + tid;
  if (t >= T) return;
  const int32_t* base = chunk_base + (int64_t)blockIdx.x * E;
  const int w = tid >> 5;
  const uint32_t below = (1u << (tid & 31)) - 1u;
  for (int j = 0; j < k; ++j) {
    const int e = idx[t * k + j];
    if ((unsigned)e >= (unsigned)E) continue;   // malformed input: leave the slot unset
    const uint32_t* m = mask + e * 8;
    int rank = __popc(m[w] & below);
    for (int q = 0; q < w; ++q) rank += __popc(m[q]);
    const int row = base[e] + rank;
    if ((int64_t)row >= T * k) continue;        // only reachable with repeated experts
    assign_row[t * k + j] = row;
    row_token[row] = (int32_t)t;
  }
}

hipError_t launch_permute(const int32_t* topk_idx, int64_t T, int k, int E, int32_t* counts,
                          int32_t* offsets, int32_t* row_token, int32_t* assign_row,
                          int32_t* chunk_counts, int32_t* chunk_base, hipStream_t s) {
  const int64_t nchunks = ceil_div(T, PERM_CHUNK);
  const size_t lds = (size_t)E * 8 * sizeof(uint32_t);
  hipLaunchKernelGGL(perm_count_kernel, dim3((unsigned)nchunks), dim3(PERM_CHUNK), lds, s,
                     topk_idx, T, k, E, chunk_counts);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(perm_scan_kernel, dim3(1), dim3(1024), 0, s, chunk_counts, nchunks, E,
                     counts, offsets, chunk_base);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(perm_scatter_kernel, dim3((unsigned)nchunks), dim3(PERM_CHUNK), lds, s,
                     topk_idx, T, k, E, chunk_base, assign_row, row_token);
  return hipGetLastError();
}

__global__ void perm_empty_kernel(int E, int32_t* __restrict__ counts,
                                  int32_t* __restrict__ offsets) {
  for (int e = threadIdx.x; e <= E; e += blockDim.x) {
    if (e < E) counts[e] = 0;
    offsets[e] = 0;
  }
}

hipError_t launch_permute_empty(int E, int32_t* counts, int32_t* offsets, hipStream_t s) {
  hipLaunchKernelGGL(perm_empty_kernel, dim3(1), dim3(1024), 0, s, E, counts, offsets);
  return hipGetLastError();
}

// Library-owned scratch of the permutation for callers that cannot allocate
// (moe_permute_noalloc): the per-chunk expert counts and bases, PERM_SCRATCH_INTS
// int32 values (8 MiB) per GPU, held until the process ends.  In host code
// `scratch` names a host-side stand-in, not device memory: the kernels get the
// device address from hipGetSymbolAddress, taken once per device with that
// device current.  Every value the kernels read is written earlier in the
// same call (chunk counts by the count kernel, bases by the scan), so nothing
// needs clearing; calls that overlap on one GPU share the array and race.
static __device__ __align__(256) int32_t scratch[PERM_SCRATCH_INTS];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
int32_t* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t permute_scratch(int32_t** out) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    g_scratch_ptr[dev] = (int32_t*)p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

int64_t permute_scratch_ints(int64_t T, int E) { return 2 * ceil_div(T, PERM_CHUNK) * (int64_t)E; }

hipError_t launch_permute_noalloc(const int32_t* topk_idx, int64_t T, int k, int E,
                                  int32_t* counts, int32_t* offsets, int32_t* row_token,
                                  int32_t* assign_row, hipStream_t s) {
  if (permute_scratch_ints(T, E) > PERM_SCRATCH_INTS) return hipErrorInvalidValue;
  int32_t* ptr = nullptr;
  const hipError_t err = permute_scratch(&ptr);
  if (err != hipSuccess) return err;
  const int64_t half = ceil_div(T, PERM_CHUNK) * (int64_t)E;
  return launch_permute(topk_idx, T, k, E, counts, offsets, row_token, assign_row, ptr,
                        ptr + half, s);
}

}  // namespace moe
