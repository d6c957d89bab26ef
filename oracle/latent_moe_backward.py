"""CPU oracle of the LatentMoE layer backward pass (numpy, float64).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only ``tests/`` and ``bench.py``'s ``cpu_baseline`` leg
use it.  It shares no code with the HIP library and imports nothing from it or
from the synthetic-input package; it builds on the forward oracle in
``latent_moe.py``.

What it computes
----------------
The gradients of the forward pass in ``latent_moe.py`` for a given gradient of
the layer output, g_out = dLoss/d out ([T, d]):

* the routed experts, per expert e and its rows r (token t = row_token[r]):
  with g = z_t W_g^T, u = z_t W_u^T, h = silu(g) u, y = h W_d^T:
  dh = dy W_d, dg = dh u silu'(g), du = dh silu(g), dz_t += dg W_g + du W_u,
  dW_d += dy^T h, dW_g += dg^T z_t, dW_u += du^T z_t, where
  silu'(v) = s (1 + v (1 - s)) with s = sigmoid(v);
* the weighted combine c_t = sum_j w_tj y_r(t,j): dy_r = w_tj dc_t and
  dw_tj = dc_t . y_r (the combine is FP32 on the pages);
* the projections: out = c W_up^T gives dc = g_out W_up, dW_up = g_out^T c;
  z = x W_dn^T gives dx = dz W_dn, dW_dn = dz^T x;
* the Base-2 shared expert (SwiGLU on x, added to out with weight 1): with
  gs = x Ws_g^T, us = x Ws_u^T, hs = silu(gs) us, s = hs Ws_d^T:
  dWs_d = g_out^T hs, dhs = g_out Ws_d, dgs = dhs us silu'(gs),
  dus = dhs silu(gs), dx += dgs Ws_g + dus Ws_u, dWs_g = dgs^T x,
  dWs_u = dus^T x;
* the router: w_tj = p_t[idx_tj] with p = softmax(l), l = x W_r^T + b, the
  selection itself piecewise constant (no gradient), the weights not
  renormalised: dp_te = dw_tj where e = idx_tj (0 elsewhere),
  dl_te = p_te (dp_te - sum_e' p_te' dp_te'), dx += dl W_r, dW_r = dl^T x,
  db = sum_t dl_t.  In the "selection" bias mode the bias only steers
  selection and gets no gradient; p is the softmax of the unbiased logits.

Precision of the backward on the pages ("The Training and RL Infrastructure
Behind MAI-Thinking-1", section 2 "Numerics", "Pre-training and mid-training
precision"): weight-gradient GEMMs in BF16 with FP32 accumulation, the router
and the MoE combine in FP32, and stochastic rounding wherever a gradient is
cast from higher to lower precision.  The data-gradient GEMMs are FP8 E5M2
there, with delayed scaling ("FP8 and MoE GEMMs"); ``grad_fp8`` selects that
for the routed experts' two data-gradient GEMMs (below); without it they run
on the bf16 operands.

Modes
-----
``exact``          nothing rounded after the inputs; the forward is recomputed
                   in exact mode.
``bf16_operands``  the forward as in its bf16_operands mode (z, h, c rounded
                   to bf16 with round-to-nearest-even where they feed a GEMM),
                   and the gradients rounded to bf16 where they become GEMM
                   operands: g_out, dy, dg, du, dz and the shared expert's
                   dgs and dus, by ``rounding``:
                   "rne" (nearest, ties to even) or "sr" (stochastic rounding
                   with the counter-based generator below).  dh, dz rows, the
                   combine gradient and everything on the router side stay
                   float64 (FP32 on the GPU).

FP8 data gradients (``grad_fp8``, bf16_operands mode only).  The pages give
the format (E5M2) and delayed scaling; the operand pairing is the plainest
reading of an FP8 GEMM: both operands FP8, the gradient in E5M2 and the
weight in E4M3 quantized as the forward quantizes it (one scale per expert
matrix, 448 / its amax).  For each of dy, dg, du (per tensor, scale s from
the caller's amax history, s = 448 / max history as for the forward; the
E5M2 operand takes 128 s = 57344 / max, E5M2's largest finite value over the
maximum) the operand is q = e5m2(float32(float32(v) * float32(128 s))), and
    dh    = (q_dy Q(W_d[e])) / (128 s_dy  s_Wd[e])
    dz_r  = (q_dg Q(W_g[e])) / (128 s_dg  s_Wg[e]) + (q_du Q(W_u[e])) / (128 s_du  s_Wu[e])
with Q the forward's E4M3 quantization.  The bf16 copies of dy, dg, du still
feed the weight-gradient GEMMs (BF16 on the pages).  The step's maxima
max |dy|, max |dg|, max |du| (before scaling) are returned for the history.
E5M2 (OCP): 5 exponent bits with bias 15, 2 fraction bits, subnormals below
2^-14 spaced 2^-16, largest finite 57344; values saturate at +-57344.
Rounding to E5M2: "rne" to nearest, ties to even; "sr" (the pages'
stochastic rounding of a gradient cast): for a magnitude a >= 2^-14 with
float32 bits u, the result is the float32 with bits (u + r) with the low 21
bits cleared, r = top 21 bits of the stream hash below; below 2^-14 (scaled
values 2^-30 of the tensor's maximum) to nearest even.  Streams 6 dy, 7 dg,
8 du, element index as for the bf16 casts.

Stochastic rounding (reading: the pages name the technique, not the
generator).  A value v is first taken to float32 (the GPU holds it in fp32);
with u its 32 bits and r a uniform 16-bit integer, the bf16 result is the top
16 bits of u + r: the magnitude is rounded up with probability equal to the
discarded fraction, so the rounding is unbiased.  r for element i (flat
row-major index of the tensor) of stream s under seed S is the top 16 bits of
    key = lowbias32((S + 0x9E3779B9 * s) mod 2^32)
    h   = lowbias32(lowbias32((i mod 2^32) xor key) xor (i >> 32))
where lowbias32 is the 32-bit integer mixer published by C. Wellons (hash
prospector): x ^= x >> 16; x *= 0x7feb352d; x ^= x >> 15; x *= 0x846ca68b;
x ^= x >> 16 (all mod 2^32).  Streams: 1 g_out [T, d], 2 dy [T*k, L] (rows in
expert order), 3 dg and 4 du [T*k, F], 5 dz [T, L], 9 dgs and 10 dus [T, Fs]
(the shared expert's gate and up gradients).

Parity pins: ``tests/test_oracle_backward.py`` (central finite differences of
the independently pinned forward oracle, softmax-gradient invariants,
linearity, the rounding's definition and statistics).
"""
from __future__ import annotations

import numpy as np

from . import latent_moe as F

ROUNDINGS = ("rne", "sr")
SR_STREAM = {"g_out": 1, "dy": 2, "dg": 3, "du": 4, "dz": 5, "dgs": 9, "dus": 10}
FP8_STREAM = {"dy": 6, "dg": 7, "du": 8}
E5M2_MAX = 57344.0
E5M2_MIN_NORMAL = 2.0 ** -14
E5M2_OVER_E4M3 = 128.0      # 57344 / 448
_M32 = np.uint64(0xFFFFFFFF)


# ---------------------------------------------------------------------------
# counter-based generator and stochastic rounding
# ---------------------------------------------------------------------------

def lowbias32(x) -> np.ndarray:
    """The lowbias32 integer mixer (uint32 in, uint32 out), from its published
    definition: two xorshift-multiply rounds and a final xorshift."""
    x = np.asarray(x, np.uint64) & _M32
    x ^= x >> np.uint64(16)
    x = (x * np.uint64(0x7FEB352D)) & _M32
    x ^= x >> np.uint64(15)
    x = (x * np.uint64(0x846CA68B)) & _M32
    x ^= x >> np.uint64(16)
    return x.astype(np.uint32)


def sr_hash(seed: int, stream: int, index) -> np.ndarray:
    """The stream's 32-bit hash of elements ``index`` (int64 array), as
    defined in the module notes."""
    key = lowbias32(np.uint64((int(seed) + 0x9E3779B9 * int(stream)) & 0xFFFFFFFF))
    i = np.asarray(index, np.int64).astype(np.uint64)
    h = lowbias32((i & _M32) ^ np.uint64(key))
    return lowbias32(h.astype(np.uint64) ^ (i >> np.uint64(32)))


def sr_bits(seed: int, stream: int, index) -> np.ndarray:
    """Uniform 16-bit integers for elements ``index`` (int64 array) of a
    stream: the top 16 bits of its hash."""
    return (sr_hash(seed, stream, index) >> np.uint32(16)).astype(np.uint32)


def round_bf16_sr(v, seed: int, stream: int, index=None) -> np.ndarray:
    """Stochastic rounding of float values to bf16 (returned as float64): v is
    taken to float32, the stream's 16 random bits are added to its bit
    pattern and the low 16 bits dropped.  Element i is the flat row-major
    index of ``v`` in its tensor: 0 .. v.size - 1, or ``index`` (same shape
    as v) for a part of a larger tensor."""
    v32 = np.ascontiguousarray(np.asarray(v, np.float64).astype(np.float32))
    u = v32.view(np.uint32).astype(np.uint64)
    idx = np.arange(v32.size, dtype=np.int64) if index is None else \
        np.asarray(index, np.int64).ravel()
    r = sr_bits(seed, stream, idx).reshape(v32.shape)
    out = ((u + r.astype(np.uint64)) & np.uint64(0xFFFF0000)).astype(np.uint32)
    return out.view(np.float32).astype(np.float64)


def round_e5m2(v) -> np.ndarray:
    """Round float64 values to E5M2 with ties to even, saturating at
    +-57344.  Written from the format: the spacing of representable values is
    2**(e - 2) in the binade [2**e, 2**(e+1)) for e >= -14, and 2**-16
    below 2**-14."""
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), E5M2_MAX)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    quantum = np.exp2(np.maximum(e, -14.0) - 2.0)
    r = np.minimum(np.rint(a / quantum) * quantum, E5M2_MAX)   # np.rint: half to even
    return np.copysign(r, v)


def round_e5m2_sr(x, seed: int, stream: int, index=None) -> np.ndarray:
    """Stochastic rounding of float32 values x to E5M2 (returned as the
    float64 values of the codes), as defined in the module notes: magnitudes
    saturate at 57344; at or above 2**-14 the stream's top 21 hash bits are
    added to the float32 bit pattern and the low 21 bits dropped; below, to
    nearest even.  Element i is the flat index of x or ``index``."""
    x32 = np.ascontiguousarray(np.asarray(x, np.float32))
    a = np.minimum(np.abs(x32), np.float32(E5M2_MAX))
    u = a.view(np.uint32).astype(np.uint64)
    idx = np.arange(x32.size, dtype=np.int64) if index is None else \
        np.asarray(index, np.int64).ravel()
    r = (sr_hash(seed, stream, idx) >> np.uint32(11)).astype(np.uint64).reshape(x32.shape)
    up = ((u + r) & np.uint64(0xFFE00000)).astype(np.uint32).view(np.float32).astype(np.float64)
    sub = np.rint(a.astype(np.float64) * 2.0 ** 16) / 2.0 ** 16
    out = np.where(a.astype(np.float64) >= E5M2_MIN_NORMAL, up, sub)
    return np.copysign(out, x32.astype(np.float64))


def quantize_grad_e5m2(v, scale, rounding: str, seed: int, name: str, index=None):
    """E5M2 operand of a gradient tensor with (E4M3-convention) scale s:
    the code values of e5m2(float32(float32(v) * float32(128 s))), float64."""
    s5 = np.float32(E5M2_OVER_E4M3) * np.float32(scale)
    x32 = np.asarray(v, np.float64).astype(np.float32) * s5
    if rounding == "rne":
        return round_e5m2(x32.astype(np.float64))
    if rounding == "sr":
        return round_e5m2_sr(x32, seed, FP8_STREAM[name], index)
    raise ValueError(f"unknown rounding {rounding!r}")


def bf16_bits(v) -> np.ndarray:
    """bf16 bit patterns (uint16) of values that are exactly bf16."""
    v32 = np.ascontiguousarray(np.asarray(v, np.float64).astype(np.float32))
    return (v32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _grad_round(v, name, mode, rounding, seed):
    """A gradient cast to bf16 where it becomes a GEMM operand."""
    if mode == "exact":
        return np.asarray(v, np.float64)
    if rounding == "rne":
        return F.round_bf16(v)
    if rounding == "sr":
        return round_bf16_sr(v, seed, SR_STREAM[name])
    raise ValueError(f"unknown rounding {rounding!r}")


# ---------------------------------------------------------------------------
# pieces
# ---------------------------------------------------------------------------

def silu_grad(v):
    """d silu / dv = s (1 + v (1 - s)), s = sigmoid(v)."""
    v = np.asarray(v, np.float64)
    with np.errstate(over="ignore"):
        s = 1.0 / (1.0 + np.exp(-v))
    return s * (1.0 + v * (1.0 - s))


def softmax_backward(p, dp):
    """Gradient of the logits of a softmax p for an upstream gradient dp:
    dl = p (dp - sum(p dp)) per row."""
    p = np.asarray(p, np.float64)
    dp = np.asarray(dp, np.float64)
    return p * (dp - (p * dp).sum(axis=1, keepdims=True))


def combine_backward(dc, y_rows, topk_w, assign_row):
    """Gradient of c_t = sum_j w_tj y_r(t,j): returns (dy_rows, dtopk_w) with
    dy_r = w_tj dc_t and dw_tj = dc_t . y_r."""
    T, k = assign_row.shape
    dy = np.zeros_like(np.asarray(y_rows, np.float64))
    dw = np.zeros((T, k), np.float64)
    for j in range(k):
        r = assign_row[:, j]
        dy[r] = np.asarray(topk_w, np.float64)[:, j:j + 1] * dc
        dw[:, j] = (dc * y_rows[r]).sum(axis=1)
    return dy, dw


def expert_backward(zr, w_gate, w_up, w_down, dy_b, mode, dh=None):
    """First half of one expert's backward on its rows (the part before the
    gate/up gradients are rounded): recomputes g, u and h, and returns them
    with dh = dy W_d (or the given dh), dg = dh u silu'(g), du = dh silu(g)
    and dW_down = dy^T h."""
    wg = np.asarray(w_gate, np.float64)
    wu = np.asarray(w_up, np.float64)
    wd = np.asarray(w_down, np.float64)
    g = zr @ wg.T
    u = zr @ wu.T
    h = F._maybe_bf16(F.silu(g) * u, mode)
    if dh is None:
        dh = dy_b @ wd
    dg = dh * u * silu_grad(g)
    du = dh * F.silu(g)
    return {"g": g, "u": u, "h": h, "dh": dh, "dg": dg, "du": du,
            "dW_down": dy_b.T @ h}


# ---------------------------------------------------------------------------
# whole layer
# ---------------------------------------------------------------------------

def shared_backward(x, ws_gate, ws_up, ws_down, go, mode="exact", rounding="rne", seed=0):
    """Gradients of the Base-2 shared expert s = (silu(x Ws_g^T) (x Ws_u^T))
    Ws_d^T (hs rounded to bf16 in bf16_operands mode, as in the forward) for
    the upstream gradient go (already cast where it feeds the GEMMs): the
    module notes' formulas, dgs and dus cast to bf16 (streams 9, 10) where
    they become GEMM operands."""
    x = np.asarray(x, np.float64)
    wsg, wsu, wsd = (np.asarray(m, np.float64) for m in (ws_gate, ws_up, ws_down))
    gs = x @ wsg.T
    us = x @ wsu.T
    hs = F._maybe_bf16(F.silu(gs) * us, mode)
    dhs = go @ wsd
    dgs = dhs * us * silu_grad(gs)
    dus = dhs * F.silu(gs)
    dgs_b = _grad_round(dgs, "dgs", mode, rounding, seed)
    dus_b = _grad_round(dus, "dus", mode, rounding, seed)
    return {"dx_shared": dgs_b @ wsg + dus_b @ wsu, "dWs_gate": dgs_b.T @ x,
            "dWs_up": dus_b.T @ x, "dWs_down": go.T @ hs, "hs_b": hs, "dhs": dhs,
            "dgs_b": dgs_b, "dus_b": dus_b}


def backward(x, w_router, b_router, k, w_dn, experts, w_lat_up, g_out, mode="exact",
             rounding="rne", seed=0, routing=None, bias_mode="logits", grad_fp8=None,
             shared=None):
    """Gradients of the LatentMoE forward for dLoss/d out = g_out; ``shared``
    = (Ws_gate, Ws_up, Ws_down) adds the Base-2 shared expert (its weight
    gradients dWs_gate, dWs_up, dWs_down, and its part of dx).  ``routing`` = (topk_idx, topk_w) replays a routing (the weights'
    gradient still flows through the softmax of this oracle's own logits at
    the replayed indices).  ``grad_fp8`` = {"grad_scale": (s_dy, s_dg, s_du),
    "w_scale": (s_Wg[E], s_Wu[E], s_Wd[E])} runs the experts' data-gradient
    GEMMs in FP8 (module notes).  Returns a dict with dx, dW_router,
    db_router, dW_dn, dW_gate, dW_up, dW_down ([E, ...] arrays), dW_lat_up,
    the gate weight gradient dtopk_w, the router logit gradient dlogits, the
    intermediates (go, dc, dy_b, dzp, dz, dz_b, ...) and, with grad_fp8, the
    maxima "grad_amax" = (max|dy|, max|dg|, max|du|)."""
    if mode not in ("exact", "bf16_operands"):
        raise ValueError(f"backward mode {mode!r} not supported")
    if grad_fp8 is not None and mode != "bf16_operands":
        raise ValueError("FP8 data gradients need the bf16_operands mode")
    if rounding not in ROUNDINGS:
        raise ValueError(f"unknown rounding {rounding!r}")
    x = np.asarray(x, np.float64)
    E = int(np.asarray(w_router).shape[0])
    r = F.route(x, w_router, b_router, k, bias_mode=bias_mode)
    if routing is not None:
        idx = np.asarray(routing[0], np.int32)
        w = np.asarray(routing[1], np.float64)
    else:
        idx, w = r["topk_idx"], r["topk_w"]
    p = F.permute(idx, E)
    off, row_token, assign_row = p["expert_offsets"], p["row_token"], p["assign_row"]
    z = F.latent_down(x, w_dn, mode)
    zp = z[row_token]
    R = row_token.size
    L = z.shape[1]
    Fw = np.asarray(experts[0][0]).shape[0] if E > 0 else 0
    # forward recomputation of the expert rows and the combine
    y = np.zeros((R, L), np.float64)
    hs = np.zeros((R, Fw), np.float64)
    for e in range(E):
        a, b = int(off[e]), int(off[e + 1])
        if a == b:
            continue
        hs[a:b] = F.swiglu_activation(zp[a:b], experts[e][0], experts[e][1], mode)
        y[a:b] = hs[a:b] @ np.asarray(experts[e][2], np.float64).T
    c = F.combine(y, w, assign_row)
    c_b = F._maybe_bf16(c, mode)
    # up-projection
    wup = np.asarray(w_lat_up, np.float64)
    go = _grad_round(g_out, "g_out", mode, rounding, seed)
    dW_lat_up = go.T @ c_b
    dc = go @ wup
    # combine
    dy, dtopk_w = combine_backward(dc, y, w, assign_row)
    dy_b = _grad_round(dy, "dy", mode, rounding, seed)
    if grad_fp8 is not None:
        s_dy, s_dg, s_du = (np.float32(s) for s in grad_fp8["grad_scale"])
        s_wg, s_wu, s_wd = (np.asarray(s, np.float32) for s in grad_fp8["w_scale"])
        q_dy = quantize_grad_e5m2(dy, s_dy, rounding, seed, "dy")
        f5 = float(np.float32(E5M2_OVER_E4M3))
    # experts
    dh = np.zeros((R, Fw), np.float64)
    dg = np.zeros((R, Fw), np.float64)
    du = np.zeros((R, Fw), np.float64)
    dW_gate = np.zeros((E, Fw, L), np.float64)
    dW_up = np.zeros((E, Fw, L), np.float64)
    dW_down = np.zeros((E, L, Fw), np.float64)
    for e in range(E):
        a, b = int(off[e]), int(off[e + 1])
        if a == b:
            continue
        dh_e = None
        if grad_fp8 is not None:
            # W_d[e] is [L, F]: dh = q_dy Q(W_d[e]) over L
            dh_e = (q_dy[a:b] @ F.quantize_e4m3(experts[e][2], s_wd[e])) / \
                (f5 * float(s_dy) * float(s_wd[e]))
        res = expert_backward(zp[a:b], *experts[e], dy_b[a:b], mode, dh=dh_e)
        dh[a:b], dg[a:b], du[a:b] = res["dh"], res["dg"], res["du"]
        dW_down[e] = res["dW_down"]
    dg_b = _grad_round(dg, "dg", mode, rounding, seed)
    du_b = _grad_round(du, "du", mode, rounding, seed)
    if grad_fp8 is not None:
        q_dg = quantize_grad_e5m2(dg, s_dg, rounding, seed, "dg")
        q_du = quantize_grad_e5m2(du, s_du, rounding, seed, "du")
    dzp = np.zeros((R, L), np.float64)
    for e in range(E):
        a, b = int(off[e]), int(off[e + 1])
        if a == b:
            continue
        wg = np.asarray(experts[e][0], np.float64)
        wu = np.asarray(experts[e][1], np.float64)
        if grad_fp8 is not None:
            dzp[a:b] = (q_dg[a:b] @ F.quantize_e4m3(wg, s_wg[e])) / \
                (f5 * float(s_dg) * float(s_wg[e])) + \
                (q_du[a:b] @ F.quantize_e4m3(wu, s_wu[e])) / (f5 * float(s_du) * float(s_wu[e]))
        else:
            dzp[a:b] = dg_b[a:b] @ wg + du_b[a:b] @ wu
        dW_gate[e] = dg_b[a:b].T @ zp[a:b]
        dW_up[e] = du_b[a:b].T @ zp[a:b]
    # gather the rows' latent gradients back to their tokens, fixed slot order
    T = x.shape[0]
    dz = np.zeros((T, L), np.float64)
    for j in range(k):
        dz += dzp[assign_row[:, j]]
    dz_b = _grad_round(dz, "dz", mode, rounding, seed)
    wdn = np.asarray(w_dn, np.float64)
    dx = dz_b @ wdn
    dW_dn = dz_b.T @ x
    # router (FP32 on the pages): gradient through the selected probabilities
    probs = r["probs"]
    dp = np.zeros((T, E), np.float64)
    for j in range(k):
        dp[np.arange(T), idx[:, j].astype(np.int64)] += dtopk_w[:, j]
    dl = softmax_backward(probs, dp)
    wr = np.asarray(w_router, np.float64)
    dx_router = dl @ wr
    dW_router = dl.T @ x
    if b_router is None:
        db = None
    elif bias_mode == "selection":
        db = np.zeros(E, np.float64)
    else:
        db = dl.sum(axis=0)
    extra = {}
    dx_shared = 0.0
    if shared is not None:
        sb = shared_backward(x, *shared, go, mode=mode, rounding=rounding, seed=seed)
        dx_shared = sb["dx_shared"]
        extra.update(sb)
    if grad_fp8 is not None:
        extra["grad_amax"] = tuple(float(np.abs(t).max()) if t.size else 0.0 for t in (dy, dg, du))
    return {**extra, "dx": dx + dx_router + dx_shared, "dx_latent": dx, "dx_router": dx_router,
            "dW_router": dW_router, "db_router": db, "dW_dn": dW_dn, "dW_gate": dW_gate,
            "dW_up": dW_up, "dW_down": dW_down, "dW_lat_up": dW_lat_up, "dtopk_w": dtopk_w,
            "dlogits": dl, "probs": probs, "go": go, "dc": dc, "dy_b": dy_b, "dh": dh,
            "dg_b": dg_b, "du_b": du_b, "dzp": dzp, "dz": dz, "dz_b": dz_b,
            "c_b": c_b, "y_rows": y, "h": hs, "topk_idx": idx, "topk_w": w,
            "expert_offsets": off, "row_token": row_token, "assign_row": assign_row}
