"""LatentMoE forward (and backward) passes through libmoe's entry points.

``LatentMoEBuffers`` allocates (with torch, once) every output and workspace
buffer a forward pass of a given shape needs; ``forward`` then only enqueues
moe_route -> moe_permute -> moe_latent_ffn_forward -> moe_combine on one
stream.  Buffer sizes depend only on the shapes (fixed memory, dropless).
"""
from __future__ import annotations

import dataclasses

import torch

from . import _lib


@dataclasses.dataclass
class LatentMoEWeights:
    w_router: torch.Tensor            # [E, d] fp32
    b_router: torch.Tensor | None     # [E] fp32
    w_lat_down: torch.Tensor          # [L, d] bf16
    w_gate: torch.Tensor              # [E, F, L] bf16
    w_up: torch.Tensor                # [E, F, L] bf16
    w_down: torch.Tensor              # [E, L, F] bf16
    w_lat_up: torch.Tensor            # [d, L] bf16
    ws_gate: torch.Tensor | None = None   # [Fs, d] bf16
    ws_up: torch.Tensor | None = None     # [Fs, d] bf16
    ws_down: torch.Tensor | None = None   # [d, Fs] bf16

    @property
    def dims(self):
        E, F, L = self.w_gate.shape
        d = self.w_lat_up.shape[0]
        Fs = 0 if self.ws_gate is None else self.ws_gate.shape[0]
        return d, L, E, F, Fs


class LatentMoEBuffers:
    """Outputs and workspace of a forward pass.  keep_logits: also keep the
    router logits [T, E] fp32, which the backward pass needs."""

    def __init__(self, T, d, L, E, k, F, Fs=0, device="cuda", keep_logits=False):
        self.T, self.d, self.L, self.E, self.k, self.F, self.Fs = T, d, L, E, k, F, Fs
        dev = torch.device(device)
        i32, f32 = torch.int32, torch.float32
        self.topk_idx = torch.empty((T, k), dtype=i32, device=dev)
        self.topk_w = torch.empty((T, k), dtype=f32, device=dev)
        self.expert_counts = torch.empty(E, dtype=i32, device=dev)
        self.expert_offsets = torch.empty(E + 1, dtype=i32, device=dev)
        self.row_token = torch.empty(T * k, dtype=i32, device=dev)
        self.assign_row = torch.empty((T, k), dtype=i32, device=dev)
        self.y_rows = torch.empty((T * k, L), dtype=f32, device=dev)
        self.hs = torch.empty((T, Fs), dtype=torch.bfloat16, device=dev) if Fs else None
        self.out = torch.empty((T, d), dtype=f32, device=dev)
        self.logits = torch.empty((T, E), dtype=f32, device=dev) if keep_logits else None
        nb = max(_lib.moe_workspace_bytes(op, T, d, L, E, k, F, Fs) for op in range(5))
        # one workspace reused by the four calls (they run in order on one stream)
        self.ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=dev)


def forward(x, w: LatentMoEWeights, k, buf: LatentMoEBuffers, stream=None, route=True):
    """Enqueue one forward pass; results land in ``buf`` (buf.out is [T, d] fp32).
    With route=False the caller's buf.topk_idx / buf.topk_w are used (router replay)."""
    if route:
        _lib.moe_route(x, w.w_router, w.b_router, k, buf.topk_idx, buf.topk_w,
                       logits_out=buf.logits, ws=buf.ws, stream=stream)
    _lib.moe_permute(buf.topk_idx, buf.E, buf.expert_counts, buf.expert_offsets, buf.row_token,
                     buf.assign_row, buf.ws, stream=stream)
    _lib.moe_latent_ffn_forward(x, w.w_lat_down, buf.expert_offsets, buf.row_token, w.w_gate,
                                w.w_up, w.w_down, w.ws_gate, w.ws_up, k, buf.y_rows, buf.hs,
                                buf.ws, stream=stream)
    _lib.moe_combine(buf.y_rows, buf.topk_w, buf.assign_row, w.w_lat_up, buf.hs, w.ws_down,
                     buf.out, buf.ws, stream=stream)
    return buf.out


# ---------------------------------------------------------------------------
# FP8 E4M3 experts with delayed scaling
# ---------------------------------------------------------------------------

E4M3_MAX = 448.0


@dataclasses.dataclass
class LatentMoEFp8Experts:
    """The routed experts' weights as E4M3 bytes with one scale per expert
    matrix: w_scale = [s(W_g[0..E)), s(W_u[0..E)), s(W_d[0..E))]."""
    w_gate: torch.Tensor      # [E, F, L] uint8
    w_up: torch.Tensor        # [E, F, L] uint8
    w_down: torch.Tensor      # [E, L, F] uint8
    w_scale: torch.Tensor     # [3E] fp32


def quantize_experts(w: LatentMoEWeights, stream=None) -> LatentMoEFp8Experts:
    """Quantize each expert matrix with scale 448 / its own amax (all in libmoe
    kernels: amax, the one-slot scale update, quantization)."""
    E = w.w_gate.shape[0]
    dev = w.w_gate.device
    amax = torch.empty(3 * E, dtype=torch.float32, device=dev)
    scale = torch.empty(3 * E, dtype=torch.float32, device=dev)
    for i, t in enumerate((w.w_gate, w.w_up, w.w_down)):
        _lib.moe_fp8_amax(t, E, amax[i * E:(i + 1) * E], stream=stream)
    hist = torch.zeros((3 * E, 1), dtype=torch.float32, device=dev)
    _lib.moe_fp8_scale_update(hist, amax, 0, scale, stream=stream)
    q = []
    for i, t in enumerate((w.w_gate, w.w_up, w.w_down)):
        dst = torch.empty(t.shape, dtype=torch.uint8, device=dev)
        _lib.moe_fp8_quantize(t, E, scale[i * E:(i + 1) * E], dst, stream=stream)
        q.append(dst)
    return LatentMoEFp8Experts(q[0], q[1], q[2], scale)


class Fp8Scaling:
    """Delayed scaling state of the two activation tensors (z, h): an amax
    history of hist_len steps each, the scales for the next step, and this
    step's amax.  Scales start at 1 until the first step is recorded."""

    def __init__(self, hist_len=1024, device="cuda"):
        dev = torch.device(device)
        self.history = torch.zeros((2, hist_len), dtype=torch.float32, device=dev)
        self.scale = torch.ones(2, dtype=torch.float32, device=dev)
        self.amax = torch.zeros(2, dtype=torch.float32, device=dev)
        self.step = 0

    def update(self, stream=None):
        _lib.moe_fp8_scale_update(self.history, self.amax, self.step % self.history.shape[1],
                                  self.scale, stream=stream)
        self.step += 1


def forward_fp8(x, w: LatentMoEWeights, w8: LatentMoEFp8Experts, k, buf: LatentMoEBuffers,
                scaling: Fp8Scaling, stream=None, route=True, update_scaling=True):
    """One forward pass with FP8 expert GEMMs: the step uses scaling.scale
    (from earlier steps' maxima), records this step's maxima and, with
    update_scaling, folds them into the history for the next step."""
    if route:
        _lib.moe_route(x, w.w_router, w.b_router, k, buf.topk_idx, buf.topk_w, ws=buf.ws,
                       stream=stream)
    _lib.moe_permute(buf.topk_idx, buf.E, buf.expert_counts, buf.expert_offsets, buf.row_token,
                     buf.assign_row, buf.ws, stream=stream)
    _lib.moe_latent_ffn_forward_fp8(x, w.w_lat_down, buf.expert_offsets, buf.row_token, w8.w_gate,
                                    w8.w_up, w8.w_down, w8.w_scale, scaling.scale, w.ws_gate,
                                    w.ws_up, k, buf.y_rows, buf.hs, scaling.amax, buf.ws,
                                    stream=stream)
    _lib.moe_combine(buf.y_rows, buf.topk_w, buf.assign_row, w.w_lat_up, buf.hs, w.ws_down,
                     buf.out, buf.ws, stream=stream)
    if update_scaling:
        scaling.update(stream=stream)
    return buf.out


# ---------------------------------------------------------------------------
# multi-round dropless experts (fixed activation memory)
# ---------------------------------------------------------------------------

def forward_rounds(x, w: LatentMoEWeights, k, buf: LatentMoEBuffers, capacity, group_size,
                   ws_rounds=None, rounds_out=None, stream=None, route=True):
    """One forward pass whose experts run the multi-round schedule with a
    fixed per-expert capacity (borrowing inside groups of group_size
    experts).  ``ws_rounds``: workspace of moe_workspace_bytes_rounds bytes
    (allocated here if None); ``rounds_out``: optional int32 device tensor
    that receives the number of rounds the routing needed."""
    if ws_rounds is None:
        d, L, E, F, Fs = w.dims
        nb = _lib.moe_workspace_bytes_rounds(buf.T, d, L, E, k, F, Fs, capacity, group_size)
        ws_rounds = torch.empty(nb, dtype=torch.uint8, device=x.device)
    if route:
        _lib.moe_route(x, w.w_router, w.b_router, k, buf.topk_idx, buf.topk_w, ws=buf.ws,
                       stream=stream)
    _lib.moe_permute(buf.topk_idx, buf.E, buf.expert_counts, buf.expert_offsets, buf.row_token,
                     buf.assign_row, buf.ws, stream=stream)
    _lib.moe_latent_ffn_forward_rounds(x, w.w_lat_down, buf.expert_offsets, buf.row_token,
                                       w.w_gate, w.w_up, w.w_down, w.ws_gate, w.ws_up, k, capacity,
                                       group_size, buf.y_rows, buf.hs, rounds_out, ws_rounds,
                                       stream=stream)
    _lib.moe_combine(buf.y_rows, buf.topk_w, buf.assign_row, w.w_lat_up, buf.hs, w.ws_down,
                     buf.out, buf.ws, stream=stream)
    return buf.out


# ---------------------------------------------------------------------------
# backward pass
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class LatentMoETransposed:
    """Transposed bf16 weight copies of the backward's data-gradient GEMMs
    (and of the shared expert's, for a layer that has one)."""
    w_lat_down_t: torch.Tensor   # [d, L]
    w_gate_t: torch.Tensor       # [E, L, F]
    w_up_t: torch.Tensor         # [E, L, F]
    w_down_t: torch.Tensor       # [E, F, L]
    w_lat_up_t: torch.Tensor     # [L, d]
    ws_gate_t: torch.Tensor | None = None   # [d, Fs]
    ws_up_t: torch.Tensor | None = None     # [d, Fs]
    ws_down_t: torch.Tensor | None = None   # [Fs, d]


def backward_prepare(w: LatentMoEWeights, stream=None) -> LatentMoETransposed:
    d, L, E, F, _ = w.dims
    dev = w.w_gate.device
    bf = torch.bfloat16
    t = LatentMoETransposed(torch.empty((d, L), dtype=bf, device=dev),
                            torch.empty((E, L, F), dtype=bf, device=dev),
                            torch.empty((E, L, F), dtype=bf, device=dev),
                            torch.empty((E, F, L), dtype=bf, device=dev),
                            torch.empty((L, d), dtype=bf, device=dev))
    _lib.moe_backward_prepare(w.w_lat_down, w.w_gate, w.w_up, w.w_down, w.w_lat_up,
                              t.w_lat_down_t, t.w_gate_t, t.w_up_t, t.w_down_t, t.w_lat_up_t,
                              stream=stream)
    if w.ws_gate is not None:
        Fs = w.ws_gate.shape[0]
        t.ws_gate_t = torch.empty((d, Fs), dtype=bf, device=dev)
        t.ws_up_t = torch.empty((d, Fs), dtype=bf, device=dev)
        t.ws_down_t = torch.empty((Fs, d), dtype=bf, device=dev)
        _lib.moe_backward_prepare_shared(w.ws_gate, w.ws_up, w.ws_down, t.ws_gate_t, t.ws_up_t,
                                         t.ws_down_t, stream=stream)
    return t


class LatentMoEGrads:
    """fp32 gradients of every parameter and of x, the gate weights' gradient,
    and the backward's workspace (Fs > 0: also the shared expert's weight
    gradients and its workspace)."""

    def __init__(self, T, d, L, E, k, F, device="cuda", bias=True, fp8=False, Fs=0,
                 workspace=True):
        dev = torch.device(device)
        f32 = torch.float32
        self.dx = torch.empty((T, d), dtype=f32, device=dev)
        self.dw_router = torch.empty((E, d), dtype=f32, device=dev)
        self.db_router = torch.empty(E, dtype=f32, device=dev) if bias else None
        self.dw_lat_down = torch.empty((L, d), dtype=f32, device=dev)
        self.dw_gate = torch.empty((E, F, L), dtype=f32, device=dev)
        self.dw_up = torch.empty((E, F, L), dtype=f32, device=dev)
        self.dw_down = torch.empty((E, L, F), dtype=f32, device=dev)
        self.dw_lat_up = torch.empty((d, L), dtype=f32, device=dev)
        self.dtopk_w = torch.empty((T, k), dtype=f32, device=dev)
        op = _lib.MOE_OP_BACKWARD_FP8 if fp8 else _lib.MOE_OP_BACKWARD
        nb = _lib.moe_workspace_bytes(op, T, d, L, E, k, F, 0)
        self.dws_gate = self.dws_up = self.dws_down = None
        if Fs:
            self.dws_gate = torch.empty((Fs, d), dtype=f32, device=dev)
            self.dws_up = torch.empty((Fs, d), dtype=f32, device=dev)
            self.dws_down = torch.empty((d, Fs), dtype=f32, device=dev)
            # one workspace for both calls (they run in order on one stream)
            nb = max(nb, _lib.moe_workspace_bytes(_lib.MOE_OP_SHARED_BACKWARD, T, d, L, E, k, F, Fs))
        # workspace=False: no workspace (backward_rounds brings its own)
        self.ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=dev) if workspace else None


def backward(x, w: LatentMoEWeights, wt: LatentMoETransposed, buf: LatentMoEBuffers, g_out,
             grads: LatentMoEGrads, rounding=_lib.MOE_ROUND_STOCHASTIC, seed=0,
             bias_mode=_lib.MOE_BIAS_LOGITS, stream=None):
    """Enqueue the backward pass of the forward held in ``buf`` (run with
    keep_logits=True) for dLoss/d out = g_out [T, d] fp32."""
    if buf.logits is None:
        raise ValueError("the forward buffers must keep the router logits (keep_logits=True)")
    _lib.moe_backward(x, w.w_router, buf.logits, bias_mode, buf.topk_idx, buf.topk_w,
                      buf.expert_offsets, buf.row_token, buf.assign_row, buf.y_rows, w.w_lat_down,
                      w.w_gate, w.w_up, wt.w_lat_down_t, wt.w_gate_t, wt.w_up_t, wt.w_down_t,
                      wt.w_lat_up_t, g_out, rounding, seed, grads.dx, grads.dw_router,
                      grads.db_router, grads.dw_lat_down, grads.dw_gate, grads.dw_up,
                      grads.dw_down, grads.dw_lat_up, grads.dtopk_w, grads.ws, stream=stream)
    _shared_backward(x, w, wt, g_out, grads, rounding, seed, stream)
    return grads


def backward_rounds(x, w: LatentMoEWeights, wt: LatentMoETransposed, buf: LatentMoEBuffers, g_out,
                    grads: LatentMoEGrads, capacity, group_size, ws_rounds=None,
                    rounding=_lib.MOE_ROUND_STOCHASTIC, seed=0, bias_mode=_lib.MOE_BIAS_LOGITS,
                    stream=None):
    """The backward pass with the routed experts on the multi-round schedule
    (fixed per-expert capacity per round, shared inside groups of group_size
    experts): the experts' activation buffers hold one round's rows.
    ``ws_rounds``: workspace of moe_workspace_bytes_backward_rounds bytes (and
    of the shared expert's backward, for a layer that has one), allocated
    here if None; grads' own workspace is not used."""
    if buf.logits is None:
        raise ValueError("the forward buffers must keep the router logits (keep_logits=True)")
    d, L, E, F, Fs = w.dims
    if ws_rounds is None:
        nb = _lib.moe_workspace_bytes_backward_rounds(buf.T, d, L, E, buf.k, F, capacity,
                                                      group_size)
        if Fs:
            nb = max(nb, _lib.moe_workspace_bytes(_lib.MOE_OP_SHARED_BACKWARD, buf.T, d, L, E,
                                                  buf.k, F, Fs))
        ws_rounds = torch.empty(max(nb, 256), dtype=torch.uint8, device=x.device)
    _lib.moe_backward_rounds(x, w.w_router, buf.logits, bias_mode, buf.topk_idx, buf.topk_w,
                             buf.expert_offsets, buf.row_token, buf.assign_row, buf.y_rows,
                             w.w_lat_down, w.w_gate, w.w_up, wt.w_lat_down_t, wt.w_gate_t,
                             wt.w_up_t, wt.w_down_t, wt.w_lat_up_t, g_out, capacity, group_size,
                             rounding, seed, grads.dx, grads.dw_router, grads.db_router,
                             grads.dw_lat_down, grads.dw_gate, grads.dw_up, grads.dw_down,
                             grads.dw_lat_up, grads.dtopk_w, ws_rounds, stream=stream)
    if w.ws_gate is not None:
        _lib.moe_shared_backward(x, g_out, w.ws_gate, w.ws_up, wt.ws_gate_t, wt.ws_up_t,
                                 wt.ws_down_t, rounding, seed, grads.dx, grads.dws_gate,
                                 grads.dws_up, grads.dws_down, ws_rounds, stream=stream)
    return grads


def _shared_backward(x, w, wt, g_out, grads, rounding, seed, stream):
    """The shared expert's gradients (a layer with one), after moe_backward
    (which overwrites dx; this adds the shared expert's part)."""
    if w.ws_gate is None:
        return
    if wt.ws_gate_t is None or grads.dws_gate is None:
        raise ValueError("a layer with a shared expert needs backward_prepare's shared transposes "
                         "and LatentMoEGrads(..., Fs=Fs)")
    _lib.moe_shared_backward(x, g_out, w.ws_gate, w.ws_up, wt.ws_gate_t, wt.ws_up_t, wt.ws_down_t,
                             rounding, seed, grads.dx, grads.dws_gate, grads.dws_up,
                             grads.dws_down, grads.ws, stream=stream)


# ---------------------------------------------------------------------------
# backward pass with FP8 data gradients (E5M2 gradients x E4M3 weights)
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class LatentMoEFp8Transposed:
    """E4M3 transposes of the routed experts' weights for the FP8 data-gradient
    GEMMs, quantized with the forward's per-expert scales w_scale."""
    w_gate_t8: torch.Tensor   # [E, L, F] uint8
    w_up_t8: torch.Tensor     # [E, L, F] uint8
    w_down_t8: torch.Tensor   # [E, F, L] uint8
    w_scale: torch.Tensor     # [3E] fp32: W_g, W_u, W_d


def quantize_transposed(wt: LatentMoETransposed, w8: LatentMoEFp8Experts,
                        stream=None) -> LatentMoEFp8Transposed:
    """Quantize the bf16 transposes with the forward's scales (quantizing
    commutes with transposing, so these are the forward's E4M3 weights,
    transposed)."""
    E = wt.w_gate_t.shape[0]
    q = []
    for i, t in enumerate((wt.w_gate_t, wt.w_up_t, wt.w_down_t)):
        dst = torch.empty(t.shape, dtype=torch.uint8, device=t.device)
        _lib.moe_fp8_quantize(t, E, w8.w_scale[i * E:(i + 1) * E], dst, stream=stream)
        q.append(dst)
    return LatentMoEFp8Transposed(q[0], q[1], q[2], w8.w_scale)


class Fp8GradScaling:
    """Delayed scaling state of the three FP8 gradient tensors (dy, dg, du):
    an amax history of hist_len steps each, the scales for the next step
    (E4M3 convention, 448 / max history; the E5M2 operand takes 128 times
    that), and this step's maxima.  Scales start at 1."""

    def __init__(self, hist_len=1024, device="cuda"):
        dev = torch.device(device)
        self.history = torch.zeros((3, hist_len), dtype=torch.float32, device=dev)
        self.scale = torch.ones(3, dtype=torch.float32, device=dev)
        self.amax = torch.zeros(3, dtype=torch.float32, device=dev)
        self.step = 0

    def update(self, stream=None):
        _lib.moe_fp8_scale_update(self.history, self.amax, self.step % self.history.shape[1],
                                  self.scale, stream=stream)
        self.step += 1


def backward_fp8(x, w: LatentMoEWeights, wt: LatentMoETransposed, wt8: LatentMoEFp8Transposed,
                 buf: LatentMoEBuffers, g_out, grads: LatentMoEGrads, scaling: Fp8GradScaling,
                 rounding=_lib.MOE_ROUND_STOCHASTIC, seed=0, bias_mode=_lib.MOE_BIAS_LOGITS,
                 stream=None, update_scaling=True):
    """The backward pass with the experts' data-gradient GEMMs in FP8 (grads
    built with fp8=True): the step uses scaling.scale, records this step's
    maxima and, with update_scaling, folds them into the history."""
    if buf.logits is None:
        raise ValueError("the forward buffers must keep the router logits (keep_logits=True)")
    _lib.moe_backward_fp8(x, w.w_router, buf.logits, bias_mode, buf.topk_idx, buf.topk_w,
                          buf.expert_offsets, buf.row_token, buf.assign_row, buf.y_rows,
                          w.w_lat_down, w.w_gate, w.w_up, wt.w_lat_down_t, wt8.w_gate_t8,
                          wt8.w_up_t8, wt8.w_down_t8, wt8.w_scale, wt.w_lat_up_t, g_out,
                          scaling.scale, rounding, seed, grads.dx, grads.dw_router,
                          grads.db_router, grads.dw_lat_down, grads.dw_gate, grads.dw_up,
                          grads.dw_down, grads.dw_lat_up, grads.dtopk_w, scaling.amax, grads.ws,
                          stream=stream)
    _shared_backward(x, w, wt, g_out, grads, rounding, seed, stream)
    if update_scaling:
        scaling.update(stream=stream)
    return grads
