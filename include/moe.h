/*
 * libmoe — forward (and backward) pass of the LatentMoE feed-forward layer on one AMD
 * MI355X (gfx950), as a C ABI over hand-written HIP kernels.
 *
 * The layer (pages: "The Training and RL Infrastructure Behind MAI-Thinking-1",
 * section "The model the systems run", model table MoE and Feed-forward rows
 * and the paragraph after it; "MAI-Base-2: Microsoft's 2.8T base model...",
 * section "The model"):
 *
 *   logits = x W_r^T + b            router on the full hidden state, FP32
 *   p      = softmax(logits)        over all E experts
 *   idx,w  = top-k of logits        stable: ties to the lower expert index;
 *                                   w = p at the selected experts, not renormalised
 *   z      = x W_dn^T               shared down-projection to the latent width L
 *   y_r    = W_d,e (silu(W_g,e z_t) * (W_u,e z_t))   per routed (token, expert)
 *   c_t    = sum_j w[t,j] y_{row(t,j)}               fixed order j = 0..k-1, FP32
 *   out    = c W_up^T  [+ shared expert SwiGLU(x) on the full width]   FP32
 *
 * The call sequence of one forward pass is
 *   moe_route -> moe_permute -> moe_latent_ffn_forward -> moe_combine
 * on one stream.  A caller may skip moe_route and supply its own topk_idx /
 * topk_w (router replay; "The Training and RL Infrastructure Behind
 * MAI-Thinking-1", section 3 "From capacity to dropless" and section 4
 * "Closing the learner-inference numerics gap").
 *
 * Conventions for every entry point
 * ---------------------------------
 * - All tensor pointers are DEVICE pointers, contiguous, row-major, 16-byte
 *   aligned.  bf16 tensors are passed as uint16_t (raw bfloat16 bits).
 * - `stream` is a hipStream_t (NULL = the null stream).  Every call only
 *   enqueues work on that stream and returns; nothing is copied to the host,
 *   and per-expert sizes are read on the device only (device-resident token
 *   metadata: "Frontier Pre-training at Microsoft AI", section "Reducing
 *   per-expert overhead").
 * - Ownership: the caller allocates and frees every buffer, including the
 *   workspace `ws` (size from moe_workspace_bytes).  The library never
 *   allocates or frees memory and never synchronises.  Buffer sizes depend
 *   only on the shapes, never on the routing (dropless, fixed memory).
 * - Errors: 0 (MOE_OK) on success, a negative MOE_ERR_* code otherwise.  All
 *   arguments are checked on the host before anything is launched; on an
 *   argument error nothing is enqueued.  T == 0 is a successful no-op.
 *   Faults inside a kernel surface at the caller's next synchronisation, as
 *   for any HIP call.  Non-finite inputs give undefined (but memory-safe)
 *   results.
 * - Determinism: identical inputs on the same device give bitwise-identical
 *   outputs (no floating-point atomics; fixed reduction orders), as the pages
 *   require of MoE top-k and of accumulations ("The Training and RL
 *   Infrastructure Behind MAI-Thinking-1", section 2, "Bitwise determinism").
 * - Limits: 1 <= k <= min(E, 16); E <= 1024; d, L, F, Fs multiples of 64
 *   (Fs may be 0 = no shared expert); T * k < 2^31; T * L * 2 < 2^31 bytes.
 * - Thread safety: calls from several host threads on different streams are
 *   safe.  Library state: the per-thread profiling-event registry, a
 *   per-device cache of the compute-unit count (atomic), and the per-device
 *   scratch address of moe_permute_noalloc (taken under a mutex; calls of
 *   that entry point that overlap on one GPU race, see there).
 */
#ifndef LATENT_MOE_H
#define LATENT_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define MOE_OK               0
#define MOE_ERR_INVALID_ARG (-1)  /* null pointer, negative size, k < 1, k > E   */
#define MOE_ERR_UNSUPPORTED (-2)  /* outside the limits above, misaligned pointer */
#define MOE_ERR_WORKSPACE   (-3)  /* ws_bytes smaller than moe_workspace_bytes()  */
#define MOE_ERR_HIP         (-4)  /* a HIP launch/record call failed             */

/* ---- workspace query ops ----------------------------------------------- */
#define MOE_OP_ROUTE       0
#define MOE_OP_PERMUTE     1
#define MOE_OP_LATENT_FFN  2
#define MOE_OP_COMBINE     3
#define MOE_OP_LATENT_FFN_FP8 4

/*
 * Bytes of device workspace that the entry point `op` needs for these shapes
 * (arguments an op does not use are ignored).  Returns 0 for an unknown op
 * or invalid shapes.
 *   ROUTE      : three bf16 parts of W_r (3*E*d*2) + fp32 logits (T*E*4)
 *                + probability partials ((n + ceil(n/64))*E*4, n = ceil(T/16))
 *   PERMUTE    : per-chunk expert counts and bases (2 * ceil(T/256) * E * 4)
 *   LATENT_FFN : z (T*L*2) + SwiGLU activations H (T*k*F*2) + tile tables
 *                (2 * (E+1) + 2 * ceil-bound of 128-row M tiles + 16, int32)
 *   COMBINE    : combined latent c in bf16 (T*L*2)
 *   LATENT_FFN_FP8 : z in E4M3 (T*L) + H in E4M3 (T*k*F) + the same tile
 *                tables as LATENT_FFN
 */
size_t moe_workspace_bytes(int op, int64_t T, int32_t d, int32_t L, int32_t E,
                           int32_t k, int32_t F, int32_t Fs);

/* Human-readable text of a status code (static storage, never NULL).  For
 * MOE_ERR_HIP it includes the HIP error of the last failure on this thread. */
const char* moe_status_string(int status);

/*
 * Router: softmax gating over all E experts on the full hidden state, top-k.
 * Defined by "The Training and RL Infrastructure Behind MAI-Thinking-1",
 * model table (MoE row: softmax gating, 8 of 512 experts), the paragraph
 * after it (the router sees the full hidden state), section 2 "Pre-training
 * and mid-training precision" (router weights, routing GEMM and logits FP32)
 * and section 2 "Bitwise determinism" (stable top-k).
 *
 *   x          [T, d]  bf16   hidden states (exact bf16 values)
 *   w_router   [E, d]  fp32   router weights
 *   b_router   [E]     fp32   per-expert bias added to the logits before the
 *                             softmax (affects selection and weights); NULL = 0
 *   topk_idx   [T, k]  int32  out: selected experts, by logit descending,
 *                             equal logits -> lower expert index first
 *   topk_w     [T, k]  fp32   out: softmax probability (over all E) of each
 *                             selected expert; not renormalised over the k
 *   logits_out [T, E]  fp32   out, optional (NULL): the FP32 logits
 * The routing GEMM accumulates exact bf16 x bf16 products of x and a three-way
 * bf16 split of W_r (hi + mid + lo == W_r exactly) in fp32.
 */
int moe_route(const uint16_t* x, const float* w_router, const float* b_router,
              int64_t T, int32_t d, int32_t E, int32_t k,
              int32_t* topk_idx, float* topk_w, float* logits_out,
              void* ws, size_t ws_bytes, void* stream);

/*
 * moe_route with two options, for training-style use:
 *
 *   bias_mode  MOE_BIAS_LOGITS    : b_router is part of the logits (moe_route)
 *              MOE_BIAS_SELECTION : b_router only steers which experts are
 *                                   selected; topk_w are the softmax of the
 *                                   unbiased logits (a loss-free balancer,
 *                                   "The Training and RL Infrastructure Behind
 *                                   MAI-Thinking-1", section 3 "From capacity
 *                                   to dropless"); logits_out is unbiased
 *   prob_sum   [E] fp32, optional (NULL): sum over the T tokens of each
 *              expert's router probability.  With the per-expert assignment
 *              counts of moe_permute these are the statistics of a
 *              global-batch load-balancing loss; both are sums, so callers
 *              aggregate micro-batches and workers by adding them (same
 *              section; "Frontier Pre-training at Microsoft AI", "Reducing
 *              per-expert overhead": one batched reduction across layers).
 *              Reduced in a fixed order: deterministic.
 * Other arguments, workspace and errors as for moe_route (an unknown
 * bias_mode is MOE_ERR_INVALID_ARG).
 */
#define MOE_BIAS_LOGITS    0
#define MOE_BIAS_SELECTION 1
int moe_route_ex(const uint16_t* x, const float* w_router, const float* b_router,
                 int32_t bias_mode, int64_t T, int32_t d, int32_t E, int32_t k,
                 int32_t* topk_idx, float* topk_w, float* logits_out, float* prob_sum,
                 void* ws, size_t ws_bytes, void* stream);

/*
 * Permutation of the T*k (token, slot) assignments into expert order: a
 * stable counting sort by expert ("expert encode", "The Training and RL
 * Infrastructure Behind MAI-Thinking-1", section 3 "Custom kernels"; device-
 * resident token metadata, "Frontier Pre-training at Microsoft AI", "Reducing
 * per-expert overhead").  Integer-exact and deterministic.
 *
 *   topk_idx        [T, k]  int32  in: expert of each (t, j); the k experts of
 *                                  one token must be distinct, each in [0, E)
 *   expert_counts   [E]     int32  out: assignments per expert
 *   expert_offsets  [E+1]   int32  out: exclusive prefix sum; [E] = T*k
 *   row_token       [T*k]   int32  out: source token of each expert-ordered
 *                                  row; ascending token order within an expert
 *   assign_row      [T, k]  int32  out: row occupied by assignment (t, j)
 */
int moe_permute(const int32_t* topk_idx, int64_t T, int32_t k, int32_t E,
                int32_t* expert_counts, int32_t* expert_offsets,
                int32_t* row_token, int32_t* assign_row,
                void* ws, size_t ws_bytes, void* stream);

/*
 * moe_permute without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  Same arguments, results and errors as moe_permute,
 * minus ws / ws_bytes: its scratch (the per-chunk expert counts and bases,
 * 2 * ceil(T / 256) * E int32) lives in a library-owned static device array
 * of 2^21 int32 (8 MiB) per GPU, which each GPU the library runs on holds
 * until the process ends.  Shapes that need more (ceil(T / 256) * E > 2^20,
 * e.g. T > 524,288 at E = 512) return MOE_ERR_UNSUPPORTED with nothing
 * enqueued.  Allocates nothing and calls no allocating routine.  Every call
 * on one GPU shares that GPU's array: calls that overlap on one GPU (two
 * streams, two host threads) race and must be serialised by the caller.
 */
int moe_permute_noalloc(const int32_t* topk_idx, int64_t T, int32_t k, int32_t E,
                        int32_t* expert_counts, int32_t* expert_offsets,
                        int32_t* row_token, int32_t* assign_row, void* stream);

/*
 * Latent down-projection and the routed SwiGLU experts as grouped GEMMs
 * (plus, for a Base-2 layer, the shared expert's gate/up half).
 * "The Training and RL Infrastructure Behind MAI-Thinking-1": model table
 * (shared down-projection before dispatch; expert FFN; SwiGLU), section 3
 * "Custom kernels" (grouped GEMMs for MoE); "MAI-Base-2: Microsoft's 2.8T
 * base model...", section "The model" (shared expert not down/up projected).
 *
 *   x               [T, d]        bf16   hidden states
 *   w_lat_down      [L, d]        bf16   W_dn
 *   expert_offsets  [E+1]         int32  from moe_permute
 *   row_token       [T*k]         int32  from moe_permute
 *   w_gate, w_up    [E, F, L]     bf16   W_g, W_u of every routed expert
 *   w_down          [E, L, F]     bf16   W_d of every routed expert
 *   ws_gate, ws_up  [Fs, d]       bf16   shared expert (NULL when Fs == 0)
 *   y_rows          [T*k, L]      fp32   out: expert outputs, expert order
 *   hs              [T, Fs]       bf16   out: shared expert activation
 *                                        silu(x Ws_g^T) * (x Ws_u^T); NULL when Fs == 0
 * z and the SwiGLU activations are bf16 (MFMA operands); accumulation is fp32.
 */
int moe_latent_ffn_forward(const uint16_t* x, const uint16_t* w_lat_down,
                           const int32_t* expert_offsets, const int32_t* row_token,
                           const uint16_t* w_gate, const uint16_t* w_up,
                           const uint16_t* w_down,
                           const uint16_t* ws_gate, const uint16_t* ws_up,
                           int64_t T, int32_t d, int32_t L, int32_t E, int32_t k,
                           int32_t F, int32_t Fs,
                           float* y_rows, uint16_t* hs,
                           void* ws, size_t ws_bytes, void* stream);

/*
 * Weighted combine in FP32 and up-projection back to the hidden width (plus
 * the shared expert's down half).  "The Training and RL Infrastructure
 * Behind MAI-Thinking-1", section 2 (MoE combine and residual stream FP32;
 * fixed-order accumulation instead of atomics); "MAI-Base-2...", section
 * "The model" (projected back up after the experts; shared expert added).
 *
 *   y_rows      [T*k, L]  fp32   from moe_latent_ffn_forward
 *   topk_w      [T, k]    fp32   gate weights
 *   assign_row  [T, k]    int32  from moe_permute
 *   w_lat_up    [d, L]    bf16   W_up
 *   hs          [T, Fs]   bf16   shared activation (NULL when Fs == 0)
 *   ws_down     [d, Fs]   bf16   shared expert W_d (NULL when Fs == 0)
 *   out         [T, d]    fp32   out: bf16(c) W_up^T + hs Ws_d^T
 * c_t = sum_{j=0..k-1} w[t,j] y[assign_row[t,j]] is a gather in fixed j
 * order (fp32), rounded to bf16 only as the up-projection's MFMA operand.
 */
int moe_combine(const float* y_rows, const float* topk_w, const int32_t* assign_row,
                const uint16_t* w_lat_up, const uint16_t* hs, const uint16_t* ws_down,
                int64_t T, int32_t d, int32_t L, int32_t k, int32_t Fs,
                float* out, void* ws, size_t ws_bytes, void* stream);

/* ---- FP8 E4M3 forward expert GEMMs ----------------------------------------
 * "The Training and RL Infrastructure Behind MAI-Thinking-1", section 2,
 * "Pre-training and mid-training precision": the forward GEMMs take FP8 E4M3
 * operands, with delayed scaling over a 1,024-step history of each tensor's
 * absolute maximum.  Format: OCP E4M3FN bytes (bias 7, 3 fraction bits,
 * largest finite 448).  A tensor t with scale s_t enters a GEMM as
 * e4m3(float32(v) * s_t), rounded to nearest even and saturated at +-448;
 * the product of two such operands is divided by both scales.  Scales and
 * maxima are fp32 device values; maxima are non-negative.
 */

/* amax[t] = max |src[t][i]| over i, for ntensor bf16 tensors of numel values
 * each, stored back to back.  numel must be a multiple of 8 and src 16-byte
 * aligned (MOE_ERR_UNSUPPORTED), ntensor <= 65535.  Order-independent,
 * deterministic.  ntensor == 0 is a no-op. */
int moe_fp8_amax(const uint16_t* src, int64_t ntensor, int64_t numel, float* amax,
                 void* stream);

/* dst[t][i] = e4m3(float32(src[t][i]) * scale[t]) (one byte each), for
 * ntensor bf16 tensors of numel values; the weights of the FP8 experts are
 * quantized with this once (e.g. 512 experts of F*L values, scale 448 /
 * amax per expert).  numel a multiple of 8; src and dst 16-byte aligned. */
int moe_fp8_quantize(const uint16_t* src, int64_t ntensor, int64_t numel, const float* scale,
                     uint8_t* dst, void* stream);

/* Delayed scaling, one step for ntensor tensors: history[t][slot] = amax[t],
 * then scale[t] = 448 / max_i history[t][i] (1 if that maximum is 0).
 * history is [ntensor][hist_len] fp32 (hist_len 1,024 on the pages), owned
 * and zero-initialised by the caller; the caller advances slot modulo
 * hist_len.  MOE_ERR_INVALID_ARG for slot outside [0, hist_len). */
int moe_fp8_scale_update(float* history, const float* amax, int64_t ntensor, int32_t hist_len,
                         int32_t slot, float* scale, void* stream);

/*
 * moe_latent_ffn_forward with the routed experts' GEMMs in FP8 E4M3.
 *   w_gate, w_up   : [E, F, L] E4M3 bytes;  w_down : [E, L, F] E4M3 bytes
 *   w_scale        : [3*E] fp32, the quantization scales of W_g[e] (first
 *                    E), W_u[e] (next E), W_d[e] (last E)
 *   act_scale      : [2] fp32, the scales of the latent z and of the SwiGLU
 *                    activation h for this step (from their amax histories)
 *   act_amax (out) : [2] fp32, max |z| and max |h| of this step (of the bf16
 *                    values before quantization), for the histories
 * z = bf16(x W_dn^T) and h = bf16(silu(g) u) are computed as in the bf16
 * path and quantized in the epilogues that produce them; each expert GEMM
 * dequantizes in its epilogue; y_rows is fp32.  The latent down-projection
 * and the shared expert stay bf16.  L and F must be multiples of 128
 * (MOE_ERR_UNSUPPORTED).  Other arguments, limits and errors as for
 * moe_latent_ffn_forward; workspace op MOE_OP_LATENT_FFN_FP8.  Finish with
 * moe_combine as usual.
 */
int moe_latent_ffn_forward_fp8(const uint16_t* x, const uint16_t* w_lat_down,
                               const int32_t* expert_offsets, const int32_t* row_token,
                               const uint8_t* w_gate, const uint8_t* w_up, const uint8_t* w_down,
                               const float* w_scale, const float* act_scale,
                               const uint16_t* ws_gate, const uint16_t* ws_up, int64_t T,
                               int32_t d, int32_t L, int32_t E, int32_t k, int32_t F, int32_t Fs,
                               float* y_rows, uint16_t* hs, float* act_amax, void* ws,
                               size_t ws_bytes, void* stream);

/* ---- multi-round dropless experts (fixed memory) ---------------------------
 * "Frontier Pre-training at Microsoft AI", "Dropless MoE with tunable,
 * fixed-size memory usage" (and the multi-round figure on "MAI-Base-2 ...")
 * moe_latent_ffn_forward with a fixed per-expert token capacity: experts form
 * groups of group_size consecutive experts (the last may be smaller); in
 * every round a group of n experts has n * capacity slots that its experts
 * share (an overloaded expert uses the slots its neighbours leave free);
 * rows that do not fit run in the next round; the round count is global.
 * A group's rows are taken in permutation order (expert, then token), so a
 * round is a contiguous slice of the group's rows.  The SwiGLU activations
 * live in a round buffer of E * capacity rows whatever the routing, instead
 * of T * k rows; each row is computed exactly as by moe_latent_ffn_forward,
 * so y_rows is bitwise the same.  The host enqueues the most rounds any
 * routing can need (max over group sizes n of ceil(T * min(k, n) /
 * (n * capacity))); rounds beyond the routing's own find no rows.
 *   rounds_out (nullable): int32 on the device, the rounds this routing needs
 * Other arguments, limits and errors as for moe_latent_ffn_forward;
 * capacity < 1 or group_size < 1 is MOE_ERR_INVALID_ARG; workspace from
 * moe_workspace_bytes_rounds (z, the round buffer E*capacity*F*2, row and
 * tile tables for one round).  MOE_KERNEL_GATE_UP brackets all rounds.
 */
size_t moe_workspace_bytes_rounds(int64_t T, int32_t d, int32_t L, int32_t E, int32_t k,
                                  int32_t F, int32_t Fs, int32_t capacity, int32_t group_size);
int moe_latent_ffn_forward_rounds(const uint16_t* x, const uint16_t* w_lat_down,
                                  const int32_t* expert_offsets, const int32_t* row_token,
                                  const uint16_t* w_gate, const uint16_t* w_up,
                                  const uint16_t* w_down, const uint16_t* ws_gate,
                                  const uint16_t* ws_up, int64_t T, int32_t d, int32_t L,
                                  int32_t E, int32_t k, int32_t F, int32_t Fs, int32_t capacity,
                                  int32_t group_size, float* y_rows, uint16_t* hs,
                                  int32_t* rounds_out, void* ws, size_t ws_bytes, void* stream);

/* ---- backward pass ---------------------------------------------------------
 * Gradients of the forward pass above for a gradient g_out = dLoss/d out
 * [T, d] fp32 (a Base-2 layer's shared expert: moe_shared_backward below).  Math, per "The Training and RL
 * Infrastructure Behind MAI-Thinking-1", section 2 "Numerics":
 *   dW_up = g^T c,  dc = g W_up                        (g = g_out cast to bf16)
 *   dy_r = w[t,j] dc_t,  dw[t,j] = dc_t . y_r          (combine backward, FP32)
 *   per expert e, rows r:  g = z W_g^T, u = z W_u^T     (recomputed, FP32)
 *     dh = dy W_d,  dg = dh u silu'(g),  du = dh silu(g)
 *     dz_r = dg W_g + du W_u,  dW_d = dy^T h,  dW_g = dg^T z_r,  dW_u = du^T z_r
 *   dz_t = sum_j dz_{row(t,j)} (fixed order),  dx = dz W_dn,  dW_dn = dz^T x
 *   router (FP32): p = softmax(router_logits), dl = p (dp - sum p dp) with dp
 *     = dw at the selected experts, dx += dl W_r, dW_r = dl^T x, db = sum_t dl
 * GEMM operands are bf16 with FP32 accumulation; the gradients g_out, dy, dg,
 * du and dz are cast to bf16 where they become GEMM operands, rounded to
 * nearest even (rounding = MOE_ROUND_NEAREST) or stochastically (rounding =
 * MOE_ROUND_STOCHASTIC: the pages round stochastically wherever a gradient
 * is cast to lower precision).  Stochastic rounding adds a uniform 16-bit
 * integer to the fp32 bit pattern and drops the low 16 bits; the integer of
 * element i (flat row-major index) of stream s (1 g_out, 2 dy with rows in
 * expert order, 3 dg, 4 du, 5 dz) is the top 16 bits of
 *   h = lowbias32(lowbias32((i mod 2^32) ^ key) ^ (i >> 32)),
 *   key = lowbias32(seed + 0x9E3779B9 * s)     (uint32 arithmetic)
 * with lowbias32 the published integer mixer x ^= x >> 16, x *= 0x7feb352d,
 * x ^= x >> 15, x *= 0x846ca68b, x ^= x >> 16.
 *
 * moe_backward_prepare: the transposed weight copies the data-gradient GEMMs
 * read (all bf16, caller-allocated): w_lat_down_t [d, L], w_gate_t and
 * w_up_t [E, L, F], w_down_t [E, F, L], w_lat_up_t [L, d].  Call once per
 * weight update (the pages' backward likewise needs each tensor and its
 * transpose, "The Training and RL Infrastructure Behind MAI-Thinking-1",
 * section 3 "Custom kernels").
 *
 * moe_backward inputs: the forward's x, routing (topk_idx, topk_w,
 * router_logits = moe_route's logits_out [T, E] fp32, bias_mode as given to
 * moe_route_ex: MOE_BIAS_LOGITS or MOE_BIAS_SELECTION), permutation
 * (expert_offsets, row_token, assign_row), the expert rows y_rows [T*k, L]
 * fp32 of moe_latent_ffn_forward, the weights w_lat_down, w_gate, w_up
 * (recomputation) and w_router [E, d] fp32, the prepared transposes, and
 * g_out.  Outputs (fp32, overwritten, caller-allocated): dx [T, d],
 * dw_router [E, d], db_router [E] (nullable; zero in the selection bias
 * mode), dw_lat_down [L, d], dw_gate [E, F, L], dw_up [E, F, L],
 * dw_down [E, L, F], dw_lat_up [d, L], dtopk_w [T, k] (nullable: the
 * gradient of the gate weights).  Workspace: MOE_OP_BACKWARD.  Limits and
 * errors as for the forward, and T * k + 64 * E < 2^22 (the weight-gradient
 * GEMMs address 256-row tiles of the transposed operands with 32-bit
 * offsets); otherwise MOE_ERR_UNSUPPORTED.  The shared expert's gradients
 * come from moe_shared_backward.  Deterministic: every reduction has a fixed
 * order.
 */
/* moe_grad_cast_bf16: dst[i] = src[i] cast to bf16 with the backward's
 * gradient rounding (MOE_ROUND_NEAREST, or MOE_ROUND_STOCHASTIC with the
 * element's integer from stream `stream_id` under `seed`, as above); n a
 * multiple of 4.  The cast the backward applies to g_out (stream 1). */
int moe_grad_cast_bf16(const float* src, int64_t n, int32_t rounding, uint32_t seed,
                       int32_t stream_id, uint16_t* dst, void* stream);
#define MOE_OP_BACKWARD      5
#define MOE_ROUND_NEAREST    0
#define MOE_ROUND_STOCHASTIC 1
int moe_backward_prepare(const uint16_t* w_lat_down, const uint16_t* w_gate,
                         const uint16_t* w_up, const uint16_t* w_down,
                         const uint16_t* w_lat_up, int32_t d, int32_t L, int32_t E, int32_t F,
                         uint16_t* w_lat_down_t, uint16_t* w_gate_t, uint16_t* w_up_t,
                         uint16_t* w_down_t, uint16_t* w_lat_up_t, void* stream);
int moe_backward(const uint16_t* x, const float* w_router, const float* router_logits,
                 int32_t bias_mode, const int32_t* topk_idx, const float* topk_w,
                 const int32_t* expert_offsets, const int32_t* row_token,
                 const int32_t* assign_row, const float* y_rows, const uint16_t* w_lat_down,
                 const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_lat_down_t,
                 const uint16_t* w_gate_t, const uint16_t* w_up_t, const uint16_t* w_down_t,
                 const uint16_t* w_lat_up_t, const float* g_out, int64_t T, int32_t d,
                 int32_t L, int32_t E, int32_t k, int32_t F, int32_t rounding, uint32_t seed,
                 float* dx, float* dw_router, float* db_router, float* dw_lat_down,
                 float* dw_gate, float* dw_up, float* dw_down, float* dw_lat_up, float* dtopk_w,
                 void* ws, size_t ws_bytes, void* stream);

/* ---- backward on the multi-round dropless schedule -----------------------------
 * "Frontier Pre-training at Microsoft AI", "Dropless MoE with tunable,
 * fixed-size memory usage" (the backward recomputes per expert group on the
 * multi-round schedule); "The Training and RL Infrastructure Behind
 * MAI-Thinking-1", section "Memory and dropless MoE" (static-memory dropless
 * mode: recomputation per expert and per round).
 * moe_backward with the routed experts' part on the forward's round schedule
 * (moe_latent_ffn_forward_rounds: groups of group_size experts share
 * group_size * capacity rows per round): in round r the rows that round
 * holds get dh = dy W_d, the recomputed gate/up GEMM with the SwiGLU
 * backward (dg, du, h) and their latent gradient, in buffers of
 * min(T k, E capacity) rows whatever the routing, and add their share of
 * dW_d, dW_g, dW_u (round 0 writes them, later rounds add, in round order:
 * deterministic).  Every row's data gradients are moe_backward's bit for bit
 * (same tiles along K, the same stochastic-rounding element indices), so dx,
 * dW_dn, dW_up, the router's gradients and dtopk_w equal moe_backward's;
 * the expert weight gradients equal them up to the fp32 summation order
 * (their K sums split at round boundaries).  The host enqueues the most
 * rounds any routing can need (as the forward does); surplus rounds find no
 * rows.  bf16 data gradients only.  Arguments as for moe_backward plus
 * capacity, group_size (>= 1, MOE_ERR_INVALID_ARG otherwise); workspace
 * moe_workspace_bytes_backward_rounds.  MOE_KERNEL_BWD_DGRAD brackets every
 * round (MOE_KERNEL_BWD_WGRAD is not recorded).
 */
size_t moe_workspace_bytes_backward_rounds(int64_t T, int32_t d, int32_t L, int32_t E, int32_t k,
                                           int32_t F, int32_t capacity, int32_t group_size);
int moe_backward_rounds(const uint16_t* x, const float* w_router, const float* router_logits,
                        int32_t bias_mode, const int32_t* topk_idx, const float* topk_w,
                        const int32_t* expert_offsets, const int32_t* row_token,
                        const int32_t* assign_row, const float* y_rows,
                        const uint16_t* w_lat_down, const uint16_t* w_gate, const uint16_t* w_up,
                        const uint16_t* w_lat_down_t, const uint16_t* w_gate_t,
                        const uint16_t* w_up_t, const uint16_t* w_down_t,
                        const uint16_t* w_lat_up_t, const float* g_out, int64_t T, int32_t d,
                        int32_t L, int32_t E, int32_t k, int32_t F, int32_t capacity,
                        int32_t group_size, int32_t rounding, uint32_t seed, float* dx,
                        float* dw_router, float* db_router, float* dw_lat_down, float* dw_gate,
                        float* dw_up, float* dw_down, float* dw_lat_up, float* dtopk_w, void* ws,
                        size_t ws_bytes, void* stream);

/* ---- backward of the shared expert (Base-2) -----------------------------------
 * "MAI-Base-2: Microsoft's 2.8T base model...", section "The model": one
 * shared expert that every token passes through, a SwiGLU FFN on the full
 * hidden state (not down/up projected), added to the layer output.  With
 * gs = x Ws_g^T, us = x Ws_u^T, hs = bf16(silu(gs) us) (the forward's hs)
 * and g = g_out cast to bf16 exactly as moe_backward casts it (stream 1):
 *   dWs_d = g^T hs,  dhs = g Ws_d,  dgs = dhs us silu'(gs),  dus = dhs silu(gs)
 *   dx   += dgs Ws_g + dus Ws_u,   dWs_g = dgs^T x,   dWs_u = dus^T x
 * dgs and dus are cast to bf16 where they become GEMM operands (nearest, or
 * stochastic with streams 9 and 10, element index t * Fs + f); dhs and the
 * accumulations are FP32; gs, us and hs are recomputed (the forward's
 * values bit for bit).  The shared expert stays bf16 in moe_backward_fp8's
 * setting too.
 *
 * moe_backward_prepare_shared: the transposed bf16 copies the data-gradient
 * GEMMs read: ws_gate_t, ws_up_t [d, Fs] (of Ws_g, Ws_u [Fs, d]) and
 * ws_down_t [Fs, d] (of Ws_d [d, Fs]); call once per weight update.
 *
 * moe_shared_backward: inputs x [T, d] bf16, g_out [T, d] fp32, the forward
 * weights ws_gate, ws_up [Fs, d] and the prepared transposes.  Outputs (fp32,
 * caller-allocated): dx [T, d] is ACCUMULATED (dx += the shared expert's
 * part; run it after moe_backward, which overwrites dx), dws_gate,
 * dws_up [Fs, d] and dws_down [d, Fs] are overwritten.  Workspace:
 * MOE_OP_SHARED_BACKWARD (T, d and Fs used).  Errors as for the forward
 * (Fs must be a positive multiple of 64).  Deterministic.
 */
#define MOE_OP_SHARED_BACKWARD 7
int moe_backward_prepare_shared(const uint16_t* ws_gate, const uint16_t* ws_up,
                                const uint16_t* ws_down, int32_t d, int32_t Fs,
                                uint16_t* ws_gate_t, uint16_t* ws_up_t, uint16_t* ws_down_t,
                                void* stream);
int moe_shared_backward(const uint16_t* x, const float* g_out, const uint16_t* ws_gate,
                        const uint16_t* ws_up, const uint16_t* ws_gate_t,
                        const uint16_t* ws_up_t, const uint16_t* ws_down_t, int64_t T,
                        int32_t d, int32_t Fs, int32_t rounding, uint32_t seed, float* dx,
                        float* dws_gate, float* dws_up, float* dws_down, void* ws,
                        size_t ws_bytes, void* stream);

/* ---- backward with FP8 data gradients ----------------------------------------
 * "The Training and RL Infrastructure Behind MAI-Thinking-1", section 2
 * "Numerics", "Pre-training and mid-training precision" (GEMM table: the
 * backward's data-gradient GEMMs in FP8 E5M2; delayed scaling over a
 * 1,024-step amax history; stochastic rounding of every gradient downcast)
 * and section 3 "Custom kernels" ("FP8 and MoE GEMMs").
 *
 * E5M2 (OCP): exponent bias 15, 2 fraction bits, subnormals spaced 2^-16
 * below 2^-14, largest finite 57344; casts saturate at +-57344.  A gradient
 * tensor's scale s follows the E4M3 convention of the forward (s = 448 /
 * max of its amax history, moe_fp8_scale_update); its E5M2 operand is
 * e5m2(float32(v) * (128 s)) (57344 / 448 = 128).  Rounding: to nearest even
 * (MOE_ROUND_NEAREST), or stochastic (MOE_ROUND_STOCHASTIC): for a magnitude
 * at or above 2^-14, the top 21 bits of the stream's hash h (as for the
 * bf16 casts above) are added to the fp32 bit pattern of the magnitude and
 * the low 21 bits dropped; below 2^-14 to nearest even.  Streams: 6 dy, 7
 * dg, 8 du (element index as for streams 2, 3, 4).
 */

/* moe_grad_cast_e5m2: dst[i] = e5m2(src[i] * 128 scale[0]) (one byte each),
 * rounded with `rounding` (stochastic: stream `stream_id` under `seed`); the
 * cast the FP8 backward applies to dy, dg and du.  n a multiple of 4; src
 * 16-byte and dst 4-byte aligned (MOE_ERR_UNSUPPORTED); scale is a device
 * fp32. */
int moe_grad_cast_e5m2(const float* src, int64_t n, const float* scale, int32_t rounding,
                       uint32_t seed, int32_t stream_id, uint8_t* dst, void* stream);

/* moe_backward_fp8: moe_backward with the routed experts' two data-gradient
 * GEMMs in FP8, the gradient operand in E5M2 and the weight in E4M3 (the
 * forward's quantization, one scale per expert matrix):
 *   dh   = (q_dy Q(W_d[e])) / (128 s_dy s_Wd[e])
 *   dz_r = (q_dg Q(W_g[e])) / (128 s_dg s_Wg[e]) + (q_du Q(W_u[e])) / (128 s_du s_Wu[e])
 * with q_t the E5M2 operand of gradient t.  The combine backward writes dy
 * in bf16 (the weight-gradient GEMMs, BF16 on the pages) and in E5M2; the
 * gate/up recompute writes dg and du likewise.  Arguments as for
 * moe_backward, except:
 *   w_gate_t8, w_up_t8 : [E, L, F] E4M3 bytes, Q(W_g[e])^T, Q(W_u[e])^T
 *   w_down_t8          : [E, F, L] E4M3 bytes, Q(W_d[e])^T
 *                        (e.g. moe_fp8_quantize of moe_backward_prepare's
 *                        bf16 transposes with the forward's w_scale:
 *                        quantizing commutes with transposing)
 *   w_scale            : [3E] fp32, the scales of W_g[e], W_u[e], W_d[e] (as
 *                        for moe_latent_ffn_forward_fp8)
 *   grad_scale         : [3] fp32, s_dy, s_dg, s_du for this step (from their
 *                        amax histories)
 *   grad_amax (out)    : [3] fp32, max |dy|, max |dg|, max |du| of this step
 *                        (fp32 values before scaling), for the histories
 * The recompute of g, u and h stays bf16 (the forward's values).  L and F
 * must be multiples of 128 (MOE_ERR_UNSUPPORTED).  Workspace:
 * MOE_OP_BACKWARD_FP8.  Deterministic (the maxima are order-independent). */
#define MOE_OP_BACKWARD_FP8  6
int moe_backward_fp8(const uint16_t* x, const float* w_router, const float* router_logits,
                     int32_t bias_mode, const int32_t* topk_idx, const float* topk_w,
                     const int32_t* expert_offsets, const int32_t* row_token,
                     const int32_t* assign_row, const float* y_rows, const uint16_t* w_lat_down,
                     const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_lat_down_t,
                     const uint8_t* w_gate_t8, const uint8_t* w_up_t8, const uint8_t* w_down_t8,
                     const float* w_scale, const uint16_t* w_lat_up_t, const float* g_out,
                     const float* grad_scale, int64_t T, int32_t d, int32_t L, int32_t E,
                     int32_t k, int32_t F, int32_t rounding, uint32_t seed, float* dx,
                     float* dw_router, float* db_router, float* dw_lat_down, float* dw_gate,
                     float* dw_up, float* dw_down, float* dw_lat_up, float* dtopk_w,
                     float* grad_amax, void* ws, size_t ws_bytes, void* stream);

/* ---- profiling hook ------------------------------------------------------
 * Register two hipEvent_t (created by the caller) that the library records on
 * the call's stream immediately before and after every launch of `kernel`
 * made by THIS host thread, until replaced; NULL, NULL clears.  Lets a caller
 * time one kernel of the sequence with events on the stream it runs on.
 * Returns MOE_ERR_INVALID_ARG for an unknown kernel id. */
#define MOE_KERNEL_ROUTER_GEMM   0   /* routing GEMM (split-bf16 MFMA)          */
#define MOE_KERNEL_ROUTER_TOPK   1   /* softmax + top-k                         */
#define MOE_KERNEL_PERMUTE       2   /* histogram/scan/scatter (first..last)    */
#define MOE_KERNEL_LATENT_DOWN   3   /* z = x W_dn^T (+ shared gate/up)         */
#define MOE_KERNEL_GATE_UP       4   /* grouped gate/up GEMM + SwiGLU           */
#define MOE_KERNEL_EXPERT_DOWN   5   /* grouped expert down GEMM                */
#define MOE_KERNEL_COMBINE       6   /* weighted gather-combine                 */
#define MOE_KERNEL_LATENT_UP     7   /* out = c W_up^T (+ shared down)          */
#define MOE_KERNEL_BWD_UP        8   /* backward: g cast, dW_up, dc             */
#define MOE_KERNEL_BWD_COMBINE   9   /* backward: combine (dy rows, dw)         */
#define MOE_KERNEL_BWD_DGRAD    10   /* backward: gate/up recompute, dh + SwiGLU
                                        backward, expert rows' latent gradient  */
#define MOE_KERNEL_BWD_WGRAD    11   /* backward: padded transposes, dW_d/g/u   */
#define MOE_KERNEL_BWD_LATENT   12   /* backward: gather dz, dx, dW_dn          */
#define MOE_KERNEL_BWD_ROUTER   13   /* backward: softmax backward, router GEMMs */
#define MOE_KERNEL_BWD_SHARED   14   /* moe_shared_backward: the whole call      */
#define MOE_KERNEL_COUNT        15
int moe_set_kernel_events(int kernel, void* start_event, void* stop_event);

#ifdef __cplusplus
}  /* extern "C" */
#endif

#endif  /* LATENT_MOE_H */
