// Host-side launchers of libmoe's kernels (internal; the public C ABI is
// include/moe.h).  Every launcher only enqueues on `s` and returns the HIP
// error of its launches.
#pragma once

#include "common.hpp"

namespace moe {

// route.hip
// K chunks of the routing GEMM (a function of the shapes only): 1, or 2-4
// when its 128 x 256 tiles alone would leave MI355X's CUs idle; the GEMM then
// writes router_ksplit partial logit arrays [T, E] (no bias) that the top-k
// kernel sums.
int router_ksplit(int64_t T, int E);
// logits: router_ksplit(T, E) arrays of T * E floats, back to back.  With one
// chunk the logits (with bias) are final; with several, partials.
hipError_t launch_router_gemm(const uint16_t* x, const float* w_router, const float* bias,
                              int64_t T, int d, int E, uint16_t* w3, float* logits,
                              hipStream_t s);
// Softmax over all E logits and top-k.  logits: nsplit partial arrays of T * E
// floats (summed in order, then lbias added when given; logits_out, when
// given, receives the sums).  sel_bias (nullable): per-expert bias added to
// the selection values only.  prob_sum (nullable): per-expert sum of
// probabilities over all tokens (prob_part: topk_partial_floats(T, E) floats
// of scratch for the deterministic fixed-order reduction).
int64_t topk_chunks(int64_t T);
int64_t topk_partial_floats(int64_t T, int E);
hipError_t launch_softmax_topk(const float* logits, int nsplit, const float* lbias,
                               float* logits_out, const float* sel_bias, int64_t T, int E, int k,
                               int32_t* topk_idx, float* topk_w, float* prob_part,
                               float* prob_sum, hipStream_t s);

// permute.hip
constexpr int PERM_CHUNK = 256;   // tokens per permutation workgroup
hipError_t launch_permute(const int32_t* topk_idx, int64_t T, int k, int E, int32_t* counts,
                          int32_t* offsets, int32_t* row_token, int32_t* assign_row,
                          int32_t* chunk_counts, int32_t* chunk_base, hipStream_t s);
hipError_t launch_permute_empty(int E, int32_t* counts, int32_t* offsets, hipStream_t s);
// The same permutation on library-owned scratch (a static device array of
// PERM_SCRATCH_INTS int32 per GPU; permute_scratch_ints(T, E) of it used):
// allocates nothing.  hipErrorInvalidValue if the shapes need more.
constexpr int64_t PERM_SCRATCH_INTS = int64_t(1) << 21;
int64_t permute_scratch_ints(int64_t T, int E);
hipError_t launch_permute_noalloc(const int32_t* topk_idx, int64_t T, int k, int E,
                                  int32_t* counts, int32_t* offsets, int32_t* row_token,
                                  int32_t* assign_row, hipStream_t s);

// expert.hip
struct ExpertGemmPlan {
  int bm_gate_up;    // M tile of the gate/up grouped GEMM
  int bm_down;       // M tile of the down grouped GEMM
};
ExpertGemmPlan plan_expert_gemms(int64_t rows, int E);
hipError_t launch_latent_down(const uint16_t* x, const uint16_t* w_dn, int64_t T, int d, int L,
                              uint16_t* z, hipStream_t s);
hipError_t launch_shared_gate_up(const uint16_t* x, const uint16_t* wsg, const uint16_t* wsu,
                                 int64_t T, int d, int Fs, uint16_t* hs, hipStream_t s);
hipError_t launch_tile_prefix(const int32_t* offsets, int E, int bm_a, int bm_b, int32_t* pre_a,
                              int32_t* pre_b, int32_t* exp_a, int32_t* exp_b, int32_t* queues,
                              hipStream_t s);
hipError_t launch_gate_up(const uint16_t* z, const int32_t* offsets, const int32_t* row_token,
                          const int32_t* tile_prefix, const int32_t* tile_expert,
                          int32_t* queue, const uint16_t* w_gate, const uint16_t* w_up, int64_t T,
                          int64_t rows, int E, int L, int F, int bm, uint16_t* H, hipStream_t s);
hipError_t launch_expert_down(const uint16_t* H, const int32_t* offsets,
                              const int32_t* tile_prefix, const int32_t* tile_expert,
                              int32_t* queue, const uint16_t* w_down, int64_t rows, int E, int L,
                              int F, int bm, float* Y, hipStream_t s);

// FP8 experts (expert.hip)
hipError_t launch_latent_down_q8(const uint16_t* x, const uint16_t* w_dn, int64_t T, int d,
                                 int L, const float* z_scale, uint32_t* amax, uint8_t* z8,
                                 hipStream_t s);
hipError_t launch_gate_up_fp8(const uint8_t* z8, const int32_t* offsets, const int32_t* row_token,
                              const int32_t* tile_prefix, const int32_t* tile_expert,
                              int32_t* queue, const uint8_t* w_gate, const uint8_t* w_up,
                              const float* z_scale, const float* wg_scale, const float* wu_scale,
                              const float* h_scale, uint32_t* amax, int64_t T, int64_t rows,
                              int E, int L, int F, int bm, uint8_t* H8, hipStream_t s);
hipError_t launch_expert_down_fp8(const uint8_t* H8, const int32_t* offsets,
                                  const int32_t* tile_prefix, const int32_t* tile_expert,
                                  int32_t* queue, const uint8_t* w_down, const float* h_scale,
                                  const float* wd_scale, int64_t rows, int E, int L, int F,
                                  int bm, float* Y, hipStream_t s);

// multi-round dropless schedule (expert.hip)
// h_end (nullable, the backward): the round's rows packed in expert order in
// the round buffer (h_base = exclusive prefix of the rows each expert has this
// round, h_end[e] = h_base[e] + its rows); null: the forward's slot layout
// (group g's rows from row first_expert(g) * C)
hipError_t launch_round_tables(const int32_t* offsets, int E, int G, int C, int round, int bm_a,
                               int bm_b, int32_t* seg_start, int32_t* seg_end, int32_t* h_base,
                               int32_t* pre_a, int32_t* pre_b, int32_t* exp_a, int32_t* exp_b,
                               int32_t* queues, int32_t* rounds_out, hipStream_t s,
                               int32_t* h_end = nullptr);
// one round of the multi-round backward's expert data gradients (expert.hip)
hipError_t launch_round_expert_bwd(const uint16_t* dy_b, const uint16_t* z,
                                   const int32_t* row_token, const int32_t* seg_start,
                                   const int32_t* seg_end, const int32_t* h_base,
                                   const int32_t* pre_a, const int32_t* exp_a,
                                   const int32_t* pre_b, const int32_t* exp_b, int32_t* queues,
                                   const uint16_t* w_gate, const uint16_t* w_up,
                                   const uint16_t* w_gate_t, const uint16_t* w_up_t,
                                   const uint16_t* w_down_t, int64_t T, int64_t rows_bound, int E,
                                   int L, int F, int bm_a, int bm_b, int sr, uint32_t key_dg,
                                   uint32_t key_du, float* dh, uint16_t* dg_b, uint16_t* du_b,
                                   uint16_t* h, float* dzp, hipStream_t s);
hipError_t launch_round_experts(const uint16_t* z, const int32_t* seg_start,
                                const int32_t* seg_end, const int32_t* h_base,
                                const int32_t* row_token, const int32_t* pre_a,
                                const int32_t* exp_a, const int32_t* pre_b, const int32_t* exp_b,
                                int32_t* queues, const uint16_t* w_gate, const uint16_t* w_up,
                                const uint16_t* w_down, int64_t T, int64_t rows_bound, int E,
                                int L, int F, int bm_a, int bm_b, uint16_t* Hr, float* Y,
                                hipStream_t s);

int device_cu_count();

// backward (expert.hip): dh, the gate/up recomputation with the SwiGLU backward in
// its epilogue, the latent gradient of the routed rows
hipError_t launch_expert_dh(const uint16_t* dy_b, const int32_t* offsets,
                            const int32_t* tile_prefix, const int32_t* tile_expert,
                            int32_t* queue, const uint16_t* w_down_t, int64_t rows, int E, int L,
                            int F, int bm, float* dh, hipStream_t s);
hipError_t launch_gate_up_bwd(const uint16_t* z, const int32_t* offsets, const int32_t* row_token,
                              const int32_t* tile_prefix, const int32_t* tile_expert,
                              int32_t* queue, const uint16_t* w_gate, const uint16_t* w_up,
                              const float* dh, int64_t T, int64_t rows, int E, int L, int F, int bm,
                              int sr, uint32_t key_dg, uint32_t key_du, uint16_t* dg_b,
                              uint16_t* du_b, uint16_t* h, hipStream_t s);
hipError_t launch_dzp(const uint16_t* dg_b, const uint16_t* du_b, const int32_t* offsets,
                      const int32_t* tile_prefix, const int32_t* tile_expert, int32_t* queue,
                      const uint16_t* w_gate_t, const uint16_t* w_up_t, int64_t rows, int E,
                      int L, int F, int bm, float* dzp, hipStream_t s);

// backward with FP8 data gradients (expert.hip)
hipError_t launch_gate_up_bwd_q8(const uint16_t* z, const int32_t* offsets,
                                 const int32_t* row_token, const int32_t* tile_prefix,
                                 const int32_t* tile_expert, int32_t* queue,
                                 const uint16_t* w_gate, const uint16_t* w_up, const float* dh,
                                 int64_t T, int64_t rows, int E, int L, int F, int bm, int sr,
                                 uint32_t key_dg, uint32_t key_du, uint32_t key_dg8,
                                 uint32_t key_du8, const float* grad_scale, uint32_t* grad_amax,
                                 uint16_t* dg_b, uint16_t* du_b, uint16_t* h, uint8_t* dg8,
                                 uint8_t* du8, hipStream_t s);
hipError_t launch_expert_dh_fp8(const uint8_t* dy8, const int32_t* offsets,
                                const int32_t* tile_prefix, const int32_t* tile_expert,
                                int32_t* queue, const uint8_t* w_down_t8, const float* dy_scale,
                                const float* wd_scale, int64_t rows, int E, int L, int F, int bm,
                                float* dh, hipStream_t s);
hipError_t launch_dzp_fp8(const uint8_t* dg8, const uint8_t* du8, const int32_t* offsets,
                          const int32_t* tile_prefix, const int32_t* tile_expert, int32_t* queue,
                          const uint8_t* w_gate_t8, const uint8_t* w_up_t8,
                          const float* dg_scale, const float* du_scale, const float* wg_scale,
                          const float* wu_scale, int64_t rows, int E, int L, int F, int bm,
                          float* dzp, hipStream_t s);

// shared expert backward (expert.hip): the gate/up recompute with the SwiGLU
// backward in its epilogue
hipError_t launch_shared_gate_up_bwd(const uint16_t* x, const uint16_t* wsg, const uint16_t* wsu,
                                     const float* dhs, int64_t T, int d, int Fs, int sr,
                                     uint32_t key_dg, uint32_t key_du, uint16_t* dgs_b,
                                     uint16_t* dus_b, uint16_t* hs_b, hipStream_t s);

// backward.hip
// C[M, N] += A1 B1^T + A2 B2^T (fp32 C; bf16 operands, K-contiguous)
hipError_t launch_dense_f32_add2(const uint16_t* A1, int64_t lda1, const uint16_t* B1,
                                 int64_t ldb1, int64_t K1, const uint16_t* A2, int64_t lda2,
                                 const uint16_t* B2, int64_t ldb2, int64_t K2, int64_t M, int N,
                                 float* C, int64_t ldc, hipStream_t s);
hipError_t launch_cvt_e5m2(const float* src, int64_t n, const float* scale, int sr, uint32_t key,
                           uint8_t* dst, hipStream_t s);
hipError_t launch_combine_bwd_q8(const float* dc, const float* y_rows, const float* topk_w,
                                 const int32_t* assign_row, int64_t T, int L, int k, int sr,
                                 uint32_t key, uint16_t* dy_b, float* dw, uint8_t* dy8,
                                 const float* grad_scale, uint32_t key8, uint32_t* grad_amax,
                                 hipStream_t s);
hipError_t launch_cvt_grad(const float* src, int64_t n, int sr, uint32_t key, uint16_t* dst,
                           hipStream_t s);
hipError_t launch_kpad_prefix(const int32_t* offsets, int E, int32_t* kpre, hipStream_t s,
                              const int32_t* ends = nullptr);
hipError_t launch_transpose_dense(const uint16_t* src, int64_t nrows, int C, uint16_t* dst,
                                  int64_t ldd, int batch, int64_t src_batch, int64_t dst_batch,
                                  hipStream_t s);
hipError_t launch_transpose_grouped(const uint16_t* src, const int32_t* gather, int64_t gather_rows,
                                    int C, const int32_t* offsets, const int32_t* kpre, int E,
                                    uint16_t* dst, int64_t ldd, hipStream_t s,
                                    const int32_t* ends = nullptr);
hipError_t launch_combine_bwd(const float* dc, const float* y_rows, const float* topk_w,
                              const int32_t* assign_row, int64_t T, int L, int k, int sr,
                              uint32_t key, uint16_t* dy_b, float* dw, hipStream_t s);
hipError_t launch_gather_sum(const float* dzp, const int32_t* assign_row, int64_t T, int L, int k,
                             int sr, uint32_t key, uint16_t* dz_b, hipStream_t s);
hipError_t launch_router_bwd(const float* logits, const int32_t* idx, const float* dw, int64_t T,
                             int E, int k, float* dl, hipStream_t s);
hipError_t launch_router_dx(const float* dl, const float* w_router, int64_t T, int d, int E,
                            float* dx, hipStream_t s);
int64_t router_dw_partial_floats(int64_t T, int d, int E);
hipError_t launch_router_dw(const float* dl, const uint16_t* x, int64_t T, int d, int E,
                            float* part, float* dw_router, hipStream_t s);
int64_t router_db_partial_floats(int64_t T, int E);
hipError_t launch_router_db(const float* dl, int64_t T, int E, float* part, float* db,
                            hipStream_t s);
hipError_t launch_dense_f32(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                            int64_t K, int64_t M, int N, float* C, int64_t ldc, hipStream_t s);
// accumulate: C_e += (tiles of experts with an empty K range are skipped)
hipError_t launch_kgrouped_f32(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                               const int32_t* kpre, int E, int M, int N, float* C,
                               int64_t c_expert_stride, hipStream_t s, bool accumulate = false);

// fp8.hip: per-tensor amax of bf16 tensors (ntensor tensors of numel values,
// numel a multiple of 8; amax holds float bits), E4M3 quantization with one
// scale per tensor, delayed-scaling update, and a zero fill
hipError_t launch_zero_u32(uint32_t* p, int64_t n, hipStream_t s);
hipError_t launch_amax_bf16(const uint16_t* src, int64_t ntensor, int64_t numel, uint32_t* amax,
                            hipStream_t s);
hipError_t launch_quantize_e4m3(const uint16_t* src, int64_t ntensor, int64_t numel,
                                const float* scale, uint8_t* dst, hipStream_t s);
hipError_t launch_scale_update(float* history, const float* amax, int64_t n, int H, int slot,
                               float* scale, hipStream_t s);

// combine.hip
hipError_t launch_combine(const float* y_rows, const float* topk_w, const int32_t* assign_row,
                          int64_t T, int L, int k, uint16_t* c, hipStream_t s);
hipError_t launch_latent_up(const uint16_t* c, const uint16_t* w_up, const uint16_t* hs,
                            const uint16_t* wsd, int64_t T, int d, int L, int Fs, float* out,
                            hipStream_t s);

}  // namespace moe
