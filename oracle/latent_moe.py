"""CPU oracle of the LatentMoE layer forward pass (numpy, float64).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (no kernels, headers, tables or helpers) and imports nothing from it,
nor from the synthetic-input package: every function takes plain arrays.

What it computes, and where the pages state it
----------------------------------------------
"The Training and RL Infrastructure Behind MAI-Thinking-1" (MAI-Base-1):
* section "The model the systems run", model table, MoE row: LatentMoE, a
  shared down-projection to the latent width before dispatch, 8 of 512 experts
  with softmax gating, expert FFN; Feed-forward row: SwiGLU.
* same section, paragraph after the table: the router sees the full hidden
  state while the experts work on the compressed latent.
* section 2 "Numerics", "Pre-training and mid-training precision": router
  logits, router weights, the routing GEMM and the MoE combine are FP32; the
  residual stream is FP32; weights and activations default to BF16.
* section 2, "Bitwise determinism": MoE top-k uses a stable sort, so ties break
  the same way every run; fixed-order accumulation instead of atomics.
* section 3, "Sharding and parallelism", "From capacity to dropless": dropless
  routing (no capacity, no dropped tokens); a global-batch load-balancing
  loss aggregated across workers and micro-batches; a loss-free balancer.
"MAI-Base-2: Microsoft's 2.8T base model..." (MAI-Base-2), section "The
model": 7 of 512 routed experts plus one shared expert every token passes
through; MoE down-projection dimension; the shared expert is not down/up
projected; tokens are projected down before dispatch and back up afterwards.

Readings where the pages are silent (each is listed in the design notes):
softmax over all E experts before top-k, selected probabilities used without
renormalisation; router bias added to the logits before the softmax; top-k
selection on the FP32 logits, ties to the lower expert index, slots ordered by
logit descending; rows of one expert in ascending token order; SwiGLU is
W_d (silu(W_g z) * (W_u z)) with silu(v) = v * sigmoid(v) and no biases; the
latent projections are plain linear maps; the combine is done in the latent
space (linear, so equal to combining after the up-projection); the shared
expert's output is added with weight 1; no extra scaling of the routed output;
the load-balancing statistics are per-expert sums (assignment counts and router
probabilities), additive across micro-batches and workers; the loss-free
balancer is a per-expert bias that steers selection only.

Precision modes
---------------
``exact``         : nothing is rounded after the inputs (float64 throughout).
``bf16_operands`` : every GEMM operand is BF16, as the pages make weights and
                    activations BF16: the latent z, the SwiGLU activation h,
                    the combined latent c and the shared expert's h are
                    rounded to bf16 (round to nearest, ties to even) where they
                    enter their next GEMM.  Expert outputs y, the combine and
                    the layer output stay float64 (the pages keep the combine
                    and the residual stream FP32).
``fp8_operands``  : as ``bf16_operands``, and the routed experts' GEMMs take
                    FP8 E4M3 operands ("The Training and RL Infrastructure
                    Behind MAI-Thinking-1", section 2, "Pre-training and
                    mid-training precision": forward GEMMs in FP8 E4M3 with
                    delayed per-tensor scaling).  Every operand tensor t has a
                    scale s_t; its values enter the GEMM as
                    e4m3(float32(v) * s_t) and the product is divided by the
                    two scales.  Tensors: the bf16 latent z, the bf16 SwiGLU
                    activation h, and each expert's W_g, W_u, W_d.  Readings:
                    the conversion rounds to nearest, ties to even, and
                    saturates at +-448; the latent projections, the shared
                    expert and the router are not FP8 in this build (the
                    router is FP32 on the pages).

Parity pins: see ``tests/test_oracle.py`` (closed forms, brute force over all
experts, invariants, special cases).  No function here is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

MODES = ("exact", "bf16_operands", "fp8_operands")
E4M3_MAX = 448.0


# ---------------------------------------------------------------------------
# rounding
# ---------------------------------------------------------------------------

def round_bf16(v: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value (8-bit significand,
    ties to even), returned as float64.  Written from the definition: scale the
    significand to [128, 256), round half to even, scale back."""
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)                 # v = m * 2**e, 0.5 <= |m| < 1
    r = np.rint(np.ldexp(m, 8))        # np.rint rounds half to even
    return np.ldexp(r, e - 8)


def _maybe_bf16(v, mode):
    if mode not in MODES:
        raise ValueError(f"unknown mode {mode!r}")
    return v if mode == "exact" else round_bf16(v)


def round_e4m3(v: np.ndarray) -> np.ndarray:
    """Round float64 values to FP8 E4M3 (OCP "E4M3FN": 4 exponent bits with
    bias 7, 3 fraction bits, subnormals below 2**-6, largest finite 448),
    round to nearest with ties to even, saturating: magnitudes above 448
    become 448.  Written from the format: the spacing of representable values
    is 2**(e - 3) in the binade [2**e, 2**(e+1)) for e >= -6, and 2**-9 below
    2**-6."""
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), E4M3_MAX)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    quantum = np.exp2(np.maximum(e, -6.0) - 3.0)
    r = np.minimum(np.rint(a / quantum) * quantum, E4M3_MAX)   # np.rint: half to even
    return np.copysign(r, v)


def quantize_e4m3(v, scale) -> np.ndarray:
    """FP8 operand of a tensor with scale s: e4m3(float32(v) * float32(s)),
    the product taken in float32 as the kernels take it.  Returned as the
    float64 values of the E4M3 codes."""
    p = np.asarray(v, np.float32) * np.float32(scale)
    return round_e4m3(p.astype(np.float64))


def fp8_matmul(a, b, scale_a, scale_b):
    """a b^T with both operands in FP8: (Q(a, s_a) Q(b, s_b)^T) / (s_a s_b)."""
    qa = quantize_e4m3(a, scale_a)
    qb = quantize_e4m3(b, scale_b)
    return (qa @ qb.T) / (float(np.float32(scale_a)) * float(np.float32(scale_b)))


def fp8_scale_from_history(history) -> np.ndarray:
    """Delayed scaling: the scale of a tensor is 448 / (largest absolute value
    in its amax history), in float32; 1 when the history holds only zeros.
    ``history`` is [..., H]; returns the scales of the leading axes."""
    h = np.asarray(history, np.float32)
    m = h.max(axis=-1)
    with np.errstate(divide="ignore"):
        s = np.where(m > 0, np.float32(E4M3_MAX) / np.where(m > 0, m, np.float32(1)),
                     np.float32(1))
    return s.astype(np.float32)


# ---------------------------------------------------------------------------
# A1: router (softmax gating over all experts, stable top-k)
# ---------------------------------------------------------------------------

def router_logits(x, w_router, b_router=None):
    """Router logits l = x W_r^T + b on the full hidden state (float64)."""
    logits = np.asarray(x, np.float64) @ np.asarray(w_router, np.float64).T
    if b_router is not None:
        logits = logits + np.asarray(b_router, np.float64)[None, :]
    return logits


def softmax(logits):
    """Softmax over the expert axis, max-subtracted."""
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m)
    return e / e.sum(axis=1, keepdims=True)


def topk_stable(scores, k):
    """Indices of the k largest scores per row, largest first; equal scores
    keep ascending expert index (a stable sort of -score)."""
    order = np.argsort(-np.asarray(scores), axis=1, kind="stable")
    return order[:, :k]


BIAS_MODES = ("logits", "selection")


def route(x, w_router, b_router, k, bias_mode="logits"):
    """Softmax gating with top-k.

    bias_mode "logits": the bias is part of the logits (selection and weights).
    bias_mode "selection": the bias only steers which experts are selected (a
    loss-free balancer); the weights are the softmax of the unbiased logits.

    Returns dict: logits (float64 selection logits, bias included),
    logits_f32 (float32, the precision the selection is taken in), probs
    (float64 softmax over all experts of the weight logits), topk_idx [T,k]
    int32, topk_w [T,k] float64 (probabilities of the selected experts, not
    renormalised)."""
    if bias_mode not in BIAS_MODES:
        raise ValueError(f"unknown bias mode {bias_mode!r}")
    logits = router_logits(x, w_router, b_router)
    logits_f32 = logits.astype(np.float32)
    if bias_mode == "selection" and b_router is not None:
        probs = softmax(router_logits(x, w_router, None))
    else:
        probs = softmax(logits)
    idx = topk_stable(logits_f32, k).astype(np.int32)
    w = np.take_along_axis(probs, idx.astype(np.int64), axis=1)
    return {"logits": logits, "logits_f32": logits_f32, "probs": probs,
            "topk_idx": idx, "topk_w": w}


def lbl_stats(probs, topk_idx, E):
    """Per-expert statistics of a global-batch load-balancing loss, as sums
    so that micro-batches and workers aggregate by addition: the number of
    (token, slot) assignments routed to each expert and the sum over tokens
    of each expert's router probability."""
    counts = np.bincount(np.asarray(topk_idx, np.int64).ravel(), minlength=E)
    return {"counts": counts, "prob_sum": np.asarray(probs, np.float64).sum(axis=0)}


# ---------------------------------------------------------------------------
# A2: permutation of (token, slot) assignments into expert order
# ---------------------------------------------------------------------------

def permute(topk_idx, E):
    """Stable counting sort of the assignments (t, j) by expert.

    Returns expert_counts[E], expert_offsets[E+1] (exclusive prefix sum,
    offsets[E] = T*k), row_token[T*k] (source token of each expert-ordered
    row; ascending token order inside an expert) and assign_row[T,k] (the row
    that assignment (t, j) occupies).  All int64."""
    idx = np.asarray(topk_idx, dtype=np.int64)
    T, k = idx.shape
    counts = np.bincount(idx.ravel(), minlength=E).astype(np.int64)
    offsets = np.zeros(E + 1, np.int64)
    offsets[1:] = np.cumsum(counts)
    row_token = np.empty(T * k, np.int64)
    assign_row = np.empty((T, k), np.int64)
    for e in range(E):
        toks, slots = np.nonzero(idx == e)     # row-major scan: ascending t
        rows = offsets[e] + np.arange(toks.size)
        row_token[rows] = toks
        assign_row[toks, slots] = rows
    return {"expert_counts": counts, "expert_offsets": offsets,
            "row_token": row_token, "assign_row": assign_row}


# ---------------------------------------------------------------------------
# A3, A5, A6: latent down-projection and the SwiGLU experts
# ---------------------------------------------------------------------------

def silu(v):
    """silu(v) = v * sigmoid(v)."""
    v = np.asarray(v, np.float64)
    with np.errstate(over="ignore"):
        return v / (1.0 + np.exp(-v))


def latent_down(x, w_dn, mode="exact"):
    """z = x W_dn^T: the shared projection of every token to the latent width."""
    return _maybe_bf16(np.asarray(x, np.float64) @ np.asarray(w_dn, np.float64).T, mode)


def swiglu_activation(z_rows, w_gate, w_up, mode="exact", fp8=None):
    """h = silu(z W_g^T) * (z W_u^T), as it enters the down projection (bf16 in
    the bf16_operands and fp8_operands modes)."""
    if mode == "fp8_operands":
        s_z, s_g, s_u, _, _ = fp8
        g = fp8_matmul(z_rows, w_gate, s_z, s_g)
        u = fp8_matmul(z_rows, w_up, s_z, s_u)
        return round_bf16(silu(g) * u)
    g = z_rows @ np.asarray(w_gate, np.float64).T
    u = z_rows @ np.asarray(w_up, np.float64).T
    return _maybe_bf16(silu(g) * u, mode)


def swiglu_expert(z_rows, w_gate, w_up, w_down, mode="exact", fp8=None):
    """y = (silu(z W_g^T) * (z W_u^T)) W_d^T for the rows routed to one expert.
    fp8_operands mode: ``fp8`` = (s_z, s_gate, s_up, s_h, s_down), the scales
    of the latent, of this expert's three weights and of the activation h."""
    h = swiglu_activation(z_rows, w_gate, w_up, mode, fp8)
    if mode == "fp8_operands":
        return fp8_matmul(h, w_down, fp8[3], fp8[4])
    return h @ np.asarray(w_down, np.float64).T


def expert_fp8_scales(fp8, e):
    """(s_z, s_gate, s_up, s_h, s_down) of expert e from a scale dict with keys
    z, h (floats) and w_gate, w_up, w_down (per expert)."""
    if fp8 is None:
        return None
    return (fp8["z"], fp8["w_gate"][e], fp8["w_up"][e], fp8["h"], fp8["w_down"][e])


def expert_rows(z, perm, experts, mode="exact", expert_fn=None, fp8=None):
    """Expert outputs y[T*k, L] in expert order: for every expert e, the rows
    offsets[e] .. offsets[e+1] are its tokens' latents through its FFN.
    ``experts[e]`` yields (W_gate[e], W_up[e], W_down[e]); ``expert_fn`` may
    replace the SwiGLU (used by the identity-expert pin)."""
    offsets = perm["expert_offsets"]
    row_token = perm["row_token"]
    E = offsets.size - 1
    y = np.zeros((row_token.size, z.shape[1]), np.float64)
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a == b:
            continue
        zr = z[row_token[a:b]]
        y[a:b] = expert_fn(e, zr) if expert_fn is not None else \
            swiglu_expert(zr, *experts[e], mode=mode, fp8=expert_fp8_scales(fp8, e))
    return y


def round_schedule(expert_offsets, capacity, group_size):
    """Multi-round dropless schedule with a fixed per-expert token capacity
    ("Frontier Pre-training at Microsoft AI", "Dropless MoE with tunable,
    fixed-size memory usage"; "MAI-Base-2 ...", the multi-round dropless
    figure): experts form groups of ``group_size`` consecutive experts (the
    last group may be smaller); in every round a group of n experts has
    n * capacity slots, which its experts share (an overloaded expert uses
    the slots its quieter neighbours leave free); rows overflowing a round go
    to the next; the round count is global (the largest any group needs).

    Reading: a group's rows are taken in expert order, then token order (the
    permutation's row order), so round r of group g is the slice
    [start_g + r * cap_g, start_g + (r + 1) * cap_g) of its row range.  The
    round's activation buffer has E * capacity rows; group g's slots start at
    row first_expert(g) * capacity.

    Returns (rounds, plan) with plan[r] = list over experts e of
    (row_begin, row_end, buffer_row_of_row_begin); empty ranges have
    row_begin == row_end."""
    off = np.asarray(expert_offsets, np.int64)
    E = off.size - 1
    groups = [(g0, min(g0 + group_size, E)) for g0 in range(0, E, group_size)]
    rounds = 0
    for g0, g1 in groups:
        load = int(off[g1] - off[g0])
        rounds = max(rounds, -(-load // ((g1 - g0) * capacity)))
    plan = []
    for r in range(rounds):
        rr = []
        for g0, g1 in groups:
            cap = (g1 - g0) * capacity
            w0 = min(int(off[g0]) + r * cap, int(off[g1]))      # the group's window
            w1 = min(int(off[g1]), w0 + cap)
            for e in range(g0, g1):
                b = min(max(int(off[e]), w0), int(off[e + 1]))   # the expert's rows in it
                en = max(min(int(off[e + 1]), w1), b)
                rr.append((b, en, g0 * capacity + min(max(b - w0, 0), cap)))
        plan.append(rr)
    return rounds, plan


# ---------------------------------------------------------------------------
# A7, A8, A9: combine, up-projection, shared expert
# ---------------------------------------------------------------------------

def combine(y_rows, topk_w, assign_row):
    """c[t] = sum over j = 0..k-1 (ascending) of w[t, j] * y[assign_row[t, j]]."""
    T, k = assign_row.shape
    c = np.zeros((T, y_rows.shape[1]), np.float64)
    for j in range(k):
        c += np.asarray(topk_w, np.float64)[:, j:j + 1] * y_rows[assign_row[:, j]]
    return c


def latent_up(c, w_lat_up, mode="exact"):
    """out = c W_up^T: projection of the combined latent back to the hidden width."""
    return _maybe_bf16(c, mode) @ np.asarray(w_lat_up, np.float64).T


def shared_expert(x, ws_gate, ws_up, ws_down, mode="exact"):
    """Base-2 shared expert: SwiGLU on the full hidden state, no latent projection."""
    x = np.asarray(x, np.float64)
    g = x @ np.asarray(ws_gate, np.float64).T
    u = x @ np.asarray(ws_up, np.float64).T
    h = _maybe_bf16(silu(g) * u, mode)
    return h @ np.asarray(ws_down, np.float64).T


# ---------------------------------------------------------------------------
# whole layer
# ---------------------------------------------------------------------------

def forward(x, w_router, b_router, k, w_dn, experts, w_lat_up, shared=None,
            mode="exact", routing=None, expert_fn=None, fp8=None):
    """LatentMoE forward: route -> permute -> z = x W_dn^T -> experts on the
    latent -> weighted combine -> up-projection (+ shared expert).

    ``experts[e]`` -> (W_gate[e], W_up[e], W_down[e]); ``shared`` is None or
    (Ws_gate, Ws_up, Ws_down); ``routing`` optionally replaces the router with
    given (topk_idx, topk_w); ``fp8`` holds the FP8 scales for the
    fp8_operands mode (see ``expert_fp8_scales``).  Returns a dict of every
    stage's result."""
    x = np.asarray(x, np.float64)
    E = int(np.asarray(w_router).shape[0]) if w_router is not None else len(experts)
    if routing is None:
        r = route(x, w_router, b_router, k)
    else:
        r = {"topk_idx": np.asarray(routing[0], np.int32),
             "topk_w": np.asarray(routing[1], np.float64)}
    p = permute(r["topk_idx"], E)
    z = latent_down(x, w_dn, mode)
    y = expert_rows(z, p, experts, mode, expert_fn, fp8)
    c = combine(y, r["topk_w"], p["assign_row"])
    out = latent_up(c, w_lat_up, mode)
    if shared is not None:
        out = out + shared_expert(x, *shared, mode=mode)
    res = dict(r)
    res.update(p)
    res.update({"z": z, "y_rows": y, "c": c, "out": out})
    return res


def forward_tokens(x_rows, topk_idx, topk_w, w_dn, experts, w_lat_up, shared=None,
                   mode="exact", fp8=None):
    """Per-token definition of the layer output, with no permutation: for each
    token t, out[t] = (sum_j w[t,j] * expert_{idx[t,j]}(z_t)) W_up^T (+ shared).
    Used for sampled tokens of shapes too large for ``forward``."""
    x_rows = np.asarray(x_rows, np.float64)
    z = latent_down(x_rows, w_dn, mode)
    c = np.zeros_like(z)
    for t in range(x_rows.shape[0]):
        for j in range(topk_idx.shape[1]):
            e = int(topk_idx[t, j])
            c[t] += float(topk_w[t, j]) * swiglu_expert(
                z[t:t + 1], *experts[e], mode=mode, fp8=expert_fp8_scales(fp8, e))[0]
    out = latent_up(c, w_lat_up, mode)
    if shared is not None:
        out = out + shared_expert(x_rows, *shared, mode=mode)
    return {"z": z, "c": c, "out": out}


def forward_dense_bruteforce(x, w_router, b_router, k, w_dn, experts, w_lat_up,
                             shared=None, mode="exact", expert_fn=None, fp8=None):
    """Brute force: evaluate every expert on every token, then keep the top-k
    by a mask (no permutation, no gather).  For tiny inputs only."""
    x = np.asarray(x, np.float64)
    r = route(x, w_router, b_router, k)
    T = x.shape[0]
    E = int(np.asarray(w_router).shape[0])
    mask = np.zeros((T, E), np.float64)
    for t in range(T):
        for j in range(k):
            mask[t, r["topk_idx"][t, j]] = 1.0
    z = latent_down(x, w_dn, mode)
    c = np.zeros_like(z)
    for e in range(E):
        ye = expert_fn(e, z) if expert_fn is not None else \
            swiglu_expert(z, *experts[e], mode=mode, fp8=expert_fp8_scales(fp8, e))
        c += (mask[:, e] * r["probs"][:, e])[:, None] * ye
    out = latent_up(c, w_lat_up, mode)
    if shared is not None:
        out = out + shared_expert(x, *shared, mode=mode)
    return {"out": out, "c": c, "topk_idx": r["topk_idx"], "probs": r["probs"]}
