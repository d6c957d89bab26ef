"""Thin Python binding of libmoe (ctypes): argument marshalling only.

Every function has the name and meaning of the C entry point in
``include/moe.h``; tensors are torch tensors on the GPU, passed by data
pointer, with shapes read from the tensors.  Every step of the layer runs in
libmoe's HIP kernels; this module computes nothing.  It raises if the library
has not been built (there is no fallback path).
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")
_lib = None

MOE_OK = 0
MOE_BIAS_LOGITS, MOE_BIAS_SELECTION = 0, 1
MOE_OP_ROUTE, MOE_OP_PERMUTE, MOE_OP_LATENT_FFN, MOE_OP_COMBINE = 0, 1, 2, 3
MOE_OP_LATENT_FFN_FP8 = 4
MOE_OP_BACKWARD = 5
MOE_OP_BACKWARD_FP8 = 6
MOE_OP_SHARED_BACKWARD = 7
MOE_ROUND_NEAREST, MOE_ROUND_STOCHASTIC = 0, 1
KERNELS = {"router_gemm": 0, "router_topk": 1, "permute": 2, "latent_down": 3, "gate_up": 4,
           "expert_down": 5, "combine": 6, "latent_up": 7, "bwd_up": 8, "bwd_combine": 9,
           "bwd_dgrad": 10, "bwd_wgrad": 11, "bwd_latent": 12, "bwd_router": 13,
           "bwd_shared": 14}

_vp, _i64, _i32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t


class MoEError(RuntimeError):
    def __init__(self, fn, code):
        super().__init__(f"{fn} failed with status {code}: {moe_status_string(code)}")
        self.code = code


def load():
    """Load libmoe.so (built in-tree); raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is not built: run `python -m mixture_experts_layer_moe_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    lib.moe_workspace_bytes.restype = _sz
    lib.moe_workspace_bytes.argtypes = [ctypes.c_int, _i64, _i32, _i32, _i32, _i32, _i32, _i32]
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_status_string.argtypes = [ctypes.c_int]
    lib.moe_route.restype = ctypes.c_int
    lib.moe_route.argtypes = [_vp, _vp, _vp, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _sz, _vp]
    lib.moe_route_ex.restype = ctypes.c_int
    lib.moe_route_ex.argtypes = [_vp, _vp, _vp, _i32, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _vp,
                                 _vp, _sz, _vp]
    lib.moe_permute.restype = ctypes.c_int
    lib.moe_permute.argtypes = [_vp, _i64, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
    lib.moe_permute_noalloc.restype = ctypes.c_int
    lib.moe_permute_noalloc.argtypes = [_vp, _i64, _i32, _i32, _vp, _vp, _vp, _vp, _vp]
    lib.moe_latent_ffn_forward.restype = ctypes.c_int
    lib.moe_latent_ffn_forward.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64,
                                           _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _sz,
                                           _vp]
    lib.moe_combine.restype = ctypes.c_int
    lib.moe_combine.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32, _vp,
                                _vp, _sz, _vp]
    lib.moe_fp8_amax.restype = ctypes.c_int
    lib.moe_fp8_amax.argtypes = [_vp, _i64, _i64, _vp, _vp]
    lib.moe_fp8_quantize.restype = ctypes.c_int
    lib.moe_fp8_quantize.argtypes = [_vp, _i64, _i64, _vp, _vp, _vp]
    lib.moe_fp8_scale_update.restype = ctypes.c_int
    lib.moe_fp8_scale_update.argtypes = [_vp, _vp, _i64, _i32, _i32, _vp, _vp]
    lib.moe_latent_ffn_forward_fp8.restype = ctypes.c_int
    lib.moe_latent_ffn_forward_fp8.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                               _vp, _i64, _i32, _i32, _i32, _i32, _i32, _i32,
                                               _vp, _vp, _vp, _vp, _sz, _vp]
    lib.moe_workspace_bytes_rounds.restype = _sz
    lib.moe_workspace_bytes_rounds.argtypes = [_i64, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                               _i32]
    lib.moe_latent_ffn_forward_rounds.restype = ctypes.c_int
    lib.moe_latent_ffn_forward_rounds.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                                  _i64, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                                  _i32, _vp, _vp, _vp, _vp, _sz, _vp]
    lib.moe_grad_cast_bf16.restype = ctypes.c_int
    lib.moe_grad_cast_bf16.argtypes = [_vp, _i64, _i32, ctypes.c_uint32, _i32, _vp, _vp]
    lib.moe_backward_prepare.restype = ctypes.c_int
    lib.moe_backward_prepare.argtypes = [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp,
                                         _vp, _vp, _vp, _vp, _vp]
    lib.moe_backward.restype = ctypes.c_int
    lib.moe_backward.argtypes = ([_vp, _vp, _vp, _i32] + [_vp] * 15 + [_i64, _i32, _i32, _i32,
                                  _i32, _i32, _i32, ctypes.c_uint32] + [_vp] * 10 + [_sz, _vp])
    lib.moe_grad_cast_e5m2.restype = ctypes.c_int
    lib.moe_grad_cast_e5m2.argtypes = [_vp, _i64, _vp, _i32, ctypes.c_uint32, _i32, _vp, _vp]
    lib.moe_backward_fp8.restype = ctypes.c_int
    lib.moe_backward_fp8.argtypes = ([_vp, _vp, _vp, _i32] + [_vp] * 17 + [_i64, _i32, _i32, _i32,
                                      _i32, _i32, _i32, ctypes.c_uint32] + [_vp] * 11 +
                                     [_sz, _vp])
    lib.moe_workspace_bytes_backward_rounds.restype = _sz
    lib.moe_workspace_bytes_backward_rounds.argtypes = [_i64, _i32, _i32, _i32, _i32, _i32, _i32,
                                                        _i32]
    lib.moe_backward_rounds.restype = ctypes.c_int
    lib.moe_backward_rounds.argtypes = ([_vp, _vp, _vp, _i32] + [_vp] * 15 +
                                        [_i64, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                         ctypes.c_uint32] + [_vp] * 10 + [_sz, _vp])
    lib.moe_backward_prepare_shared.restype = ctypes.c_int
    lib.moe_backward_prepare_shared.argtypes = [_vp, _vp, _vp, _i32, _i32, _vp, _vp, _vp, _vp]
    lib.moe_shared_backward.restype = ctypes.c_int
    lib.moe_shared_backward.argtypes = ([_vp] * 7 + [_i64, _i32, _i32, _i32, ctypes.c_uint32] +
                                        [_vp] * 5 + [_sz, _vp])
    lib.moe_set_kernel_events.restype = ctypes.c_int
    lib.moe_set_kernel_events.argtypes = [ctypes.c_int, _vp, _vp]
    _lib = lib
    return lib


def _ptr(t):
    """Device address of a tensor argument (evaluated after every shape check
    of the call, right before the C entry point runs)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"tensor arguments must be GPU tensors, got one on {t.device}")
    return t.data_ptr()


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(fn, code):
    if code != MOE_OK:
        raise MoEError(fn, code)


def _need(t, name, dtype, ndim=None, shape=None):
    """Checks a tensor argument: dtype, contiguity, dims, shape (a tuple of
    ints, None = any extent).  The C ABI receives only pointers and sizes and
    cannot check extents itself, and a buffer shorter than the sizes imply
    would be read or written out of bounds.  That every tensor lives on the
    GPU is checked by _ptr, after all shape checks of a call."""
    if t is None:
        return
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if shape is not None:
        if t.dim() != len(shape) or any(w is not None and int(w) != g
                                        for g, w in zip(t.shape, shape)):
            want = tuple("*" if w is None else int(w) for w in shape)
            raise ValueError(f"{name} must have shape {want}, got {tuple(t.shape)}")


def _numel(t, name, n):
    """A flat buffer argument must hold exactly n values."""
    if t is not None and t.numel() != int(n):
        raise ValueError(f"{name} must hold {int(n)} values, got {t.numel()}")


def _dims2(t, name):
    if t is None or t.dim() != 2:
        raise ValueError(f"{name} must be a 2-D tensor, got "
                         f"{None if t is None else tuple(t.shape)}")
    return int(t.shape[0]), int(t.shape[1])


def _dims3(t, name):
    if t is None or t.dim() != 3:
        raise ValueError(f"{name} must be a 3-D tensor, got "
                         f"{None if t is None else tuple(t.shape)}")
    return int(t.shape[0]), int(t.shape[1]), int(t.shape[2])


def moe_workspace_bytes(op, T, d, L, E, k, F, Fs=0):
    return int(load().moe_workspace_bytes(op, T, d, L, E, k, F, Fs))


def moe_status_string(code):
    return load().moe_status_string(code).decode()


def moe_set_kernel_events(kernel, start_event, stop_event):
    """Register raw hipEvent_t handles (ints) recorded around `kernel` (name or id)."""
    kid = KERNELS[kernel] if isinstance(kernel, str) else int(kernel)
    _check("moe_set_kernel_events", load().moe_set_kernel_events(kid, start_event, stop_event))


def _route_args(x, w_router, b_router, k, topk_idx, topk_w, logits_out):
    T, d = _dims2(x, "x")
    E = _dims2(w_router, "w_router")[0]
    _need(x, "x", torch.bfloat16, shape=(T, d))
    _need(w_router, "w_router", torch.float32, shape=(E, d))
    _need(b_router, "b_router", torch.float32, shape=(E,))
    _need(topk_idx, "topk_idx", torch.int32, shape=(T, k))
    _need(topk_w, "topk_w", torch.float32, shape=(T, k))
    _need(logits_out, "logits_out", torch.float32, shape=(T, E))
    return T, d, E


def moe_route(x, w_router, b_router, k, topk_idx, topk_w, logits_out=None, ws=None, stream=None):
    T, d, E = _route_args(x, w_router, b_router, k, topk_idx, topk_w, logits_out)
    _need(ws, "ws", torch.uint8, 1)
    _check("moe_route", load().moe_route(_ptr(x), _ptr(w_router), _ptr(b_router), T, d, E, k,
                                         _ptr(topk_idx), _ptr(topk_w), _ptr(logits_out), _ptr(ws),
                                         _nbytes(ws), _stream(stream)))


def moe_route_ex(x, w_router, b_router, bias_mode, k, topk_idx, topk_w, logits_out=None,
                 prob_sum=None, ws=None, stream=None):
    T, d, E = _route_args(x, w_router, b_router, k, topk_idx, topk_w, logits_out)
    _need(prob_sum, "prob_sum", torch.float32, shape=(E,))
    _need(ws, "ws", torch.uint8, 1)
    _check("moe_route_ex", load().moe_route_ex(
        _ptr(x), _ptr(w_router), _ptr(b_router), int(bias_mode), T, d, E, k, _ptr(topk_idx),
        _ptr(topk_w), _ptr(logits_out), _ptr(prob_sum), _ptr(ws), _nbytes(ws), _stream(stream)))


def moe_permute(topk_idx, E, expert_counts, expert_offsets, row_token, assign_row, ws,
                stream=None):
    T, k = _dims2(topk_idx, "topk_idx")
    E = int(E)
    _need(topk_idx, "topk_idx", torch.int32, shape=(T, k))
    for n, t, cnt in (("expert_counts", expert_counts, E), ("expert_offsets", expert_offsets, E + 1),
                      ("row_token", row_token, T * k), ("assign_row", assign_row, T * k)):
        _numel(t, n, cnt)
        _need(t, n, torch.int32)
    _need(ws, "ws", torch.uint8, 1)
    _check("moe_permute", load().moe_permute(_ptr(topk_idx), T, k, E, _ptr(expert_counts),
                                             _ptr(expert_offsets), _ptr(row_token),
                                             _ptr(assign_row), _ptr(ws), _nbytes(ws),
                                             _stream(stream)))


def moe_permute_noalloc(topk_idx, E, expert_counts, expert_offsets, row_token, assign_row,
                        stream=None):
    """moe_permute on the library's own static scratch (no workspace)."""
    T, k = _dims2(topk_idx, "topk_idx")
    E = int(E)
    _need(topk_idx, "topk_idx", torch.int32, shape=(T, k))
    for n, t, cnt in (("expert_counts", expert_counts, E), ("expert_offsets", expert_offsets, E + 1),
                      ("row_token", row_token, T * k), ("assign_row", assign_row, T * k)):
        _numel(t, n, cnt)
        _need(t, n, torch.int32)
    _check("moe_permute_noalloc", load().moe_permute_noalloc(
        _ptr(topk_idx), T, k, E, _ptr(expert_counts), _ptr(expert_offsets), _ptr(row_token),
        _ptr(assign_row), _stream(stream)))


def _ffn_args(x, w_lat_down, expert_offsets, row_token, w_gate, w_up, w_down, ws_gate, ws_up, k,
              y_rows, hs, wdtype):
    """Shapes of the latent-FFN entry points: T, d from x, L from W_dn, E, F
    from W_g, Fs from Ws_g; every other buffer must agree."""
    T, d = _dims2(x, "x")
    L = _dims2(w_lat_down, "w_lat_down")[0]
    E, F, _ = _dims3(w_gate, "w_gate")
    Fs = 0 if ws_gate is None else _dims2(ws_gate, "ws_gate")[0]
    _need(x, "x", torch.bfloat16, shape=(T, d))
    _need(w_lat_down, "w_lat_down", torch.bfloat16, shape=(L, d))
    _need(w_gate, "w_gate", wdtype, shape=(E, F, L))
    _need(w_up, "w_up", wdtype, shape=(E, F, L))
    _need(w_down, "w_down", wdtype, shape=(E, L, F))
    if (ws_up is None) != (ws_gate is None) or (Fs > 0 and hs is None):
        raise ValueError("ws_gate, ws_up and hs are given together (a shared expert) or not at all")
    _need(ws_gate, "ws_gate", torch.bfloat16, shape=(Fs, d))
    _need(ws_up, "ws_up", torch.bfloat16, shape=(Fs, d))
    _need(hs, "hs", torch.bfloat16, shape=(T, Fs))
    _numel(expert_offsets, "expert_offsets", E + 1)
    _need(expert_offsets, "expert_offsets", torch.int32, 1)
    _numel(row_token, "row_token", T * int(k))
    _need(row_token, "row_token", torch.int32, 1)
    _need(y_rows, "y_rows", torch.float32, shape=(T * int(k), L))
    return T, d, L, E, F, Fs


def moe_latent_ffn_forward(x, w_lat_down, expert_offsets, row_token, w_gate, w_up, w_down,
                           ws_gate, ws_up, k, y_rows, hs, ws, stream=None):
    T, d, L, E, F, Fs = _ffn_args(x, w_lat_down, expert_offsets, row_token, w_gate, w_up, w_down,
                                  ws_gate, ws_up, k, y_rows, hs, torch.bfloat16)
    _need(ws, "ws", torch.uint8, 1)
    _check("moe_latent_ffn_forward", load().moe_latent_ffn_forward(
        _ptr(x), _ptr(w_lat_down), _ptr(expert_offsets), _ptr(row_token), _ptr(w_gate),
        _ptr(w_up), _ptr(w_down), _ptr(ws_gate), _ptr(ws_up), T, d, L, E, k, F, Fs, _ptr(y_rows),
        _ptr(hs), _ptr(ws), _nbytes(ws), _stream(stream)))


def moe_combine(y_rows, topk_w, assign_row, w_lat_up, hs, ws_down, out, ws, stream=None):
    T, k = _dims2(topk_w, "topk_w")
    d, L = _dims2(w_lat_up, "w_lat_up")
    Fs = 0 if ws_down is None else _dims2(ws_down, "ws_down")[1]
    if (hs is None) != (ws_down is None):
        raise ValueError("hs and ws_down are given together (a shared expert) or not at all")
    _need(y_rows, "y_rows", torch.float32, shape=(T * k, L))
    _need(topk_w, "topk_w", torch.float32, shape=(T, k))
    _need(assign_row, "assign_row", torch.int32, shape=(T, k))
    _need(w_lat_up, "w_lat_up", torch.bfloat16, shape=(d, L))
    _need(hs, "hs", torch.bfloat16, shape=(T, Fs))
    _need(ws_down, "ws_down", torch.bfloat16, shape=(d, Fs))
    _need(out, "out", torch.float32, shape=(T, d))
    _need(ws, "ws", torch.uint8, 1)
    _check("moe_combine", load().moe_combine(_ptr(y_rows), _ptr(topk_w), _ptr(assign_row),
                                             _ptr(w_lat_up), _ptr(hs), _ptr(ws_down), T, d, L, k,
                                             Fs, _ptr(out), _ptr(ws), _nbytes(ws),
                                             _stream(stream)))


def moe_fp8_amax(src, ntensor, amax, stream=None):
    """amax[t] = max |src_t| for ntensor equal bf16 tensors stored back to back in src."""
    ntensor = int(ntensor)
    if ntensor < 0 or (ntensor and src.numel() % ntensor):
        raise ValueError(f"src ({src.numel()} values) does not split into {ntensor} tensors")
    _need(src, "src", torch.bfloat16)
    _need(amax, "amax", torch.float32, shape=(ntensor,))
    _check("moe_fp8_amax", load().moe_fp8_amax(_ptr(src), ntensor, src.numel() // max(ntensor, 1),
                                               _ptr(amax), _stream(stream)))


def moe_fp8_quantize(src, ntensor, scale, dst, stream=None):
    """dst = e4m3(src_t * scale[t]) bytes (uint8) for ntensor equal bf16 tensors."""
    ntensor = int(ntensor)
    if ntensor < 0 or (ntensor and src.numel() % ntensor):
        raise ValueError(f"src ({src.numel()} values) does not split into {ntensor} tensors")
    _need(src, "src", torch.bfloat16)
    _need(scale, "scale", torch.float32, shape=(ntensor,))
    _numel(dst, "dst", src.numel())
    _need(dst, "dst", torch.uint8)
    _check("moe_fp8_quantize", load().moe_fp8_quantize(
        _ptr(src), ntensor, src.numel() // max(ntensor, 1), _ptr(scale), _ptr(dst),
        _stream(stream)))


def moe_fp8_scale_update(history, amax, slot, scale, stream=None):
    """history [n, H] fp32: history[:, slot] = amax; scale = 448 / max over the history."""
    n, H = _dims2(history, "history")
    _need(history, "history", torch.float32, shape=(n, H))
    _need(amax, "amax", torch.float32, shape=(n,))
    _need(scale, "scale", torch.float32, shape=(n,))
    _check("moe_fp8_scale_update", load().moe_fp8_scale_update(
        _ptr(history), _ptr(amax), n, H, int(slot), _ptr(scale), _stream(stream)))


def moe_latent_ffn_forward_fp8(x, w_lat_down, expert_offsets, row_token, w_gate, w_up, w_down,
                               w_scale, act_scale, ws_gate, ws_up, k, y_rows, hs, act_amax, ws,
                               stream=None):
    T, d, L, E, F, Fs = _ffn_args(x, w_lat_down, expert_offsets, row_token, w_gate, w_up, w_down,
                                  ws_gate, ws_up, k, y_rows, hs, torch.uint8)
    _need(w_scale, "w_scale", torch.float32, shape=(3 * E,))
    _need(act_scale, "act_scale", torch.float32, shape=(2,))
    _need(act_amax, "act_amax", torch.float32, shape=(2,))
    _need(ws, "ws", torch.uint8, 1)
    _check("moe_latent_ffn_forward_fp8", load().moe_latent_ffn_forward_fp8(
        _ptr(x), _ptr(w_lat_down), _ptr(expert_offsets), _ptr(row_token), _ptr(w_gate),
        _ptr(w_up), _ptr(w_down), _ptr(w_scale), _ptr(act_scale), _ptr(ws_gate), _ptr(ws_up), T,
        d, L, E, k, F, Fs, _ptr(y_rows), _ptr(hs), _ptr(act_amax), _ptr(ws), _nbytes(ws),
        _stream(stream)))


def moe_workspace_bytes_rounds(T, d, L, E, k, F, Fs, capacity, group_size):
    return int(load().moe_workspace_bytes_rounds(T, d, L, E, k, F, Fs, capacity, group_size))


def moe_latent_ffn_forward_rounds(x, w_lat_down, expert_offsets, row_token, w_gate, w_up, w_down,
                                  ws_gate, ws_up, k, capacity, group_size, y_rows, hs, rounds_out,
                                  ws, stream=None):
    T, d, L, E, F, Fs = _ffn_args(x, w_lat_down, expert_offsets, row_token, w_gate, w_up, w_down,
                                  ws_gate, ws_up, k, y_rows, hs, torch.bfloat16)
    if rounds_out is not None and rounds_out.numel() < 1:
        raise ValueError("rounds_out must hold one value")
    _need(rounds_out, "rounds_out", torch.int32)
    _need(ws, "ws", torch.uint8, 1)
    _check("moe_latent_ffn_forward_rounds", load().moe_latent_ffn_forward_rounds(
        _ptr(x), _ptr(w_lat_down), _ptr(expert_offsets), _ptr(row_token), _ptr(w_gate),
        _ptr(w_up), _ptr(w_down), _ptr(ws_gate), _ptr(ws_up), T, d, L, E, k, F, Fs,
        int(capacity), int(group_size), _ptr(y_rows), _ptr(hs), _ptr(rounds_out), _ptr(ws),
        _nbytes(ws), _stream(stream)))


def moe_backward_prepare(w_lat_down, w_gate, w_up, w_down, w_lat_up, w_lat_down_t, w_gate_t,
                         w_up_t, w_down_t, w_lat_up_t, stream=None):
    E, F, L = _dims3(w_gate, "w_gate")
    d = _dims2(w_lat_up, "w_lat_up")[0]
    for n, t, shp in (("w_lat_down", w_lat_down, (L, d)), ("w_gate", w_gate, (E, F, L)),
                      ("w_up", w_up, (E, F, L)), ("w_down", w_down, (E, L, F)),
                      ("w_lat_up", w_lat_up, (d, L)), ("w_lat_down_t", w_lat_down_t, (d, L)),
                      ("w_gate_t", w_gate_t, (E, L, F)), ("w_up_t", w_up_t, (E, L, F)),
                      ("w_down_t", w_down_t, (E, F, L)), ("w_lat_up_t", w_lat_up_t, (L, d))):
        if t is None:
            raise ValueError(f"{n} is required")
        _need(t, n, torch.bfloat16, shape=shp)
    _check("moe_backward_prepare", load().moe_backward_prepare(
        _ptr(w_lat_down), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(w_lat_up), d, L, E, F,
        _ptr(w_lat_down_t), _ptr(w_gate_t), _ptr(w_up_t), _ptr(w_down_t), _ptr(w_lat_up_t),
        _stream(stream)))


def _bwd_args(x, w_router, router_logits, topk_idx, topk_w, expert_offsets, row_token,
              assign_row, y_rows, w_lat_down, w_gate, w_up, w_lat_down_t, w_lat_up_t, g_out, dx,
              dw_router, db_router, dw_lat_down, dw_gate, dw_up, dw_down, dw_lat_up, dtopk_w):
    """Shapes of the backward entry points: T, d from x, E, F, L from W_g, k
    from topk_idx; every other buffer must agree."""
    T, d = _dims2(x, "x")
    E, F, L = _dims3(w_gate, "w_gate")
    k = _dims2(topk_idx, "topk_idx")[1]
    _need(x, "x", torch.bfloat16, shape=(T, d))
    f32 = (("w_router", w_router, (E, d)), ("router_logits", router_logits, (T, E)),
           ("topk_w", topk_w, (T, k)), ("y_rows", y_rows, (T * k, L)), ("g_out", g_out, (T, d)),
           ("dx", dx, (T, d)), ("dw_router", dw_router, (E, d)), ("db_router", db_router, (E,)),
           ("dw_lat_down", dw_lat_down, (L, d)), ("dw_gate", dw_gate, (E, F, L)),
           ("dw_up", dw_up, (E, F, L)), ("dw_down", dw_down, (E, L, F)),
           ("dw_lat_up", dw_lat_up, (d, L)), ("dtopk_w", dtopk_w, (T, k)))
    for n, t, shp in f32:
        _need(t, n, torch.float32, shape=shp)
    _need(topk_idx, "topk_idx", torch.int32, shape=(T, k))
    _need(assign_row, "assign_row", torch.int32, shape=(T, k))
    _numel(expert_offsets, "expert_offsets", E + 1)
    _need(expert_offsets, "expert_offsets", torch.int32, 1)
    _numel(row_token, "row_token", T * k)
    _need(row_token, "row_token", torch.int32, 1)
    for n, t, shp in (("w_lat_down", w_lat_down, (L, d)), ("w_gate", w_gate, (E, F, L)),
                      ("w_up", w_up, (E, F, L)), ("w_lat_down_t", w_lat_down_t, (d, L)),
                      ("w_lat_up_t", w_lat_up_t, (L, d))):
        _need(t, n, torch.bfloat16, shape=shp)
    return T, d, L, E, k, F


def moe_backward(x, w_router, router_logits, bias_mode, topk_idx, topk_w, expert_offsets,
                 row_token, assign_row, y_rows, w_lat_down, w_gate, w_up, w_lat_down_t, w_gate_t,
                 w_up_t, w_down_t, w_lat_up_t, g_out, rounding, seed, dx, dw_router, db_router,
                 dw_lat_down, dw_gate, dw_up, dw_down, dw_lat_up, dtopk_w, ws, stream=None):
    T, d, L, E, k, F = _bwd_args(x, w_router, router_logits, topk_idx, topk_w, expert_offsets,
                                 row_token, assign_row, y_rows, w_lat_down, w_gate, w_up,
                                 w_lat_down_t, w_lat_up_t, g_out, dx, dw_router, db_router,
                                 dw_lat_down, dw_gate, dw_up, dw_down, dw_lat_up, dtopk_w)
    for n, t, shp in (("w_gate_t", w_gate_t, (E, L, F)), ("w_up_t", w_up_t, (E, L, F)),
                      ("w_down_t", w_down_t, (E, F, L))):
        _need(t, n, torch.bfloat16, shape=shp)
    _need(ws, "ws", torch.uint8, 1)
    _check("moe_backward", load().moe_backward(
        _ptr(x), _ptr(w_router), _ptr(router_logits), int(bias_mode), _ptr(topk_idx),
        _ptr(topk_w), _ptr(expert_offsets), _ptr(row_token), _ptr(assign_row), _ptr(y_rows),
        _ptr(w_lat_down), _ptr(w_gate), _ptr(w_up), _ptr(w_lat_down_t), _ptr(w_gate_t),
        _ptr(w_up_t), _ptr(w_down_t), _ptr(w_lat_up_t), _ptr(g_out), T, d, L, E, k, F,
        int(rounding), int(seed) & 0xFFFFFFFF, _ptr(dx), _ptr(dw_router), _ptr(db_router),
        _ptr(dw_lat_down), _ptr(dw_gate), _ptr(dw_up), _ptr(dw_down), _ptr(dw_lat_up),
        _ptr(dtopk_w), _ptr(ws), _nbytes(ws), _stream(stream)))


def moe_grad_cast_bf16(src, rounding, seed, stream_id, dst, stream=None):
    _need(src, "src", torch.float32)
    _numel(dst, "dst", src.numel())
    _need(dst, "dst", torch.bfloat16)
    _check("moe_grad_cast_bf16", load().moe_grad_cast_bf16(
        _ptr(src), src.numel(), int(rounding), int(seed) & 0xFFFFFFFF, int(stream_id), _ptr(dst),
        _stream(stream)))


def moe_grad_cast_e5m2(src, scale, rounding, seed, stream_id, dst, stream=None):
    _need(src, "src", torch.float32)
    if scale is None or scale.numel() < 1:
        raise ValueError("scale must hold one value")
    _need(scale, "scale", torch.float32)
    _numel(dst, "dst", src.numel())
    _need(dst, "dst", torch.uint8)
    _check("moe_grad_cast_e5m2", load().moe_grad_cast_e5m2(
        _ptr(src), src.numel(), _ptr(scale), int(rounding), int(seed) & 0xFFFFFFFF,
        int(stream_id), _ptr(dst), _stream(stream)))


def moe_backward_fp8(x, w_router, router_logits, bias_mode, topk_idx, topk_w, expert_offsets,
                     row_token, assign_row, y_rows, w_lat_down, w_gate, w_up, w_lat_down_t,
                     w_gate_t8, w_up_t8, w_down_t8, w_scale, w_lat_up_t, g_out, grad_scale,
                     rounding, seed, dx, dw_router, db_router, dw_lat_down, dw_gate, dw_up,
                     dw_down, dw_lat_up, dtopk_w, grad_amax, ws, stream=None):
    T, d, L, E, k, F = _bwd_args(x, w_router, router_logits, topk_idx, topk_w, expert_offsets,
                                 row_token, assign_row, y_rows, w_lat_down, w_gate, w_up,
                                 w_lat_down_t, w_lat_up_t, g_out, dx, dw_router, db_router,
                                 dw_lat_down, dw_gate, dw_up, dw_down, dw_lat_up, dtopk_w)
    for n, t, shp in (("w_gate_t8", w_gate_t8, (E, L, F)), ("w_up_t8", w_up_t8, (E, L, F)),
                      ("w_down_t8", w_down_t8, (E, F, L))):
        _need(t, n, torch.uint8, shape=shp)
    _need(w_scale, "w_scale", torch.float32, shape=(3 * E,))
    _need(grad_scale, "grad_scale", torch.float32, shape=(3,))
    _need(grad_amax, "grad_amax", torch.float32, shape=(3,))
    _need(ws, "ws", torch.uint8, 1)
    _check("moe_backward_fp8", load().moe_backward_fp8(
        _ptr(x), _ptr(w_router), _ptr(router_logits), int(bias_mode), _ptr(topk_idx),
        _ptr(topk_w), _ptr(expert_offsets), _ptr(row_token), _ptr(assign_row), _ptr(y_rows),
        _ptr(w_lat_down), _ptr(w_gate), _ptr(w_up), _ptr(w_lat_down_t), _ptr(w_gate_t8),
        _ptr(w_up_t8), _ptr(w_down_t8), _ptr(w_scale), _ptr(w_lat_up_t), _ptr(g_out),
        _ptr(grad_scale), T, d, L, E, k, F, int(rounding), int(seed) & 0xFFFFFFFF, _ptr(dx),
        _ptr(dw_router), _ptr(db_router), _ptr(dw_lat_down), _ptr(dw_gate), _ptr(dw_up),
        _ptr(dw_down), _ptr(dw_lat_up), _ptr(dtopk_w), _ptr(grad_amax), _ptr(ws), _nbytes(ws),
        _stream(stream)))


def moe_backward_prepare_shared(ws_gate, ws_up, ws_down, ws_gate_t, ws_up_t, ws_down_t,
                                stream=None):
    """Transposed copies of the shared expert's weights for moe_shared_backward."""
    Fs, d = _dims2(ws_gate, "ws_gate")
    for n, t, shp in (("ws_gate", ws_gate, (Fs, d)), ("ws_up", ws_up, (Fs, d)),
                      ("ws_down", ws_down, (d, Fs)), ("ws_gate_t", ws_gate_t, (d, Fs)),
                      ("ws_up_t", ws_up_t, (d, Fs)), ("ws_down_t", ws_down_t, (Fs, d))):
        if t is None:
            raise ValueError(f"{n} is required")
        _need(t, n, torch.bfloat16, shape=shp)
    _check("moe_backward_prepare_shared", load().moe_backward_prepare_shared(
        _ptr(ws_gate), _ptr(ws_up), _ptr(ws_down), d, Fs, _ptr(ws_gate_t), _ptr(ws_up_t),
        _ptr(ws_down_t), _stream(stream)))


def moe_shared_backward(x, g_out, ws_gate, ws_up, ws_gate_t, ws_up_t, ws_down_t, rounding, seed,
                        dx, dws_gate, dws_up, dws_down, ws, stream=None):
    """Gradients of the shared expert; dx is accumulated into (dx += ...)."""
    T, d = _dims2(x, "x")
    Fs = _dims2(ws_gate, "ws_gate")[0]
    _need(x, "x", torch.bfloat16, shape=(T, d))
    for n, t, shp in (("ws_gate", ws_gate, (Fs, d)), ("ws_up", ws_up, (Fs, d)),
                      ("ws_gate_t", ws_gate_t, (d, Fs)), ("ws_up_t", ws_up_t, (d, Fs)),
                      ("ws_down_t", ws_down_t, (Fs, d))):
        if t is None:
            raise ValueError(f"{n} is required")
        _need(t, n, torch.bfloat16, shape=shp)
    for n, t, shp in (("g_out", g_out, (T, d)), ("dx", dx, (T, d)), ("dws_gate", dws_gate, (Fs, d)),
                      ("dws_up", dws_up, (Fs, d)), ("dws_down", dws_down, (d, Fs))):
        if t is None:
            raise ValueError(f"{n} is required")
        _need(t, n, torch.float32, shape=shp)
    _need(ws, "ws", torch.uint8, 1)
    _check("moe_shared_backward", load().moe_shared_backward(
        _ptr(x), _ptr(g_out), _ptr(ws_gate), _ptr(ws_up), _ptr(ws_gate_t), _ptr(ws_up_t),
        _ptr(ws_down_t), T, d, Fs, int(rounding), int(seed) & 0xFFFFFFFF, _ptr(dx), _ptr(dws_gate),
        _ptr(dws_up), _ptr(dws_down), _ptr(ws), _nbytes(ws), _stream(stream)))


def moe_workspace_bytes_backward_rounds(T, d, L, E, k, F, capacity, group_size):
    return int(load().moe_workspace_bytes_backward_rounds(T, d, L, E, k, F, capacity, group_size))


def moe_backward_rounds(x, w_router, router_logits, bias_mode, topk_idx, topk_w, expert_offsets,
                        row_token, assign_row, y_rows, w_lat_down, w_gate, w_up, w_lat_down_t,
                        w_gate_t, w_up_t, w_down_t, w_lat_up_t, g_out, capacity, group_size,
                        rounding, seed, dx, dw_router, db_router, dw_lat_down, dw_gate, dw_up,
                        dw_down, dw_lat_up, dtopk_w, ws, stream=None):
    T, d, L, E, k, F = _bwd_args(x, w_router, router_logits, topk_idx, topk_w, expert_offsets,
                                 row_token, assign_row, y_rows, w_lat_down, w_gate, w_up,
                                 w_lat_down_t, w_lat_up_t, g_out, dx, dw_router, db_router,
                                 dw_lat_down, dw_gate, dw_up, dw_down, dw_lat_up, dtopk_w)
    for n, t, shp in (("w_gate_t", w_gate_t, (E, L, F)), ("w_up_t", w_up_t, (E, L, F)),
                      ("w_down_t", w_down_t, (E, F, L))):
        _need(t, n, torch.bfloat16, shape=shp)
    _need(ws, "ws", torch.uint8, 1)
    _check("moe_backward_rounds", load().moe_backward_rounds(
        _ptr(x), _ptr(w_router), _ptr(router_logits), int(bias_mode), _ptr(topk_idx),
        _ptr(topk_w), _ptr(expert_offsets), _ptr(row_token), _ptr(assign_row), _ptr(y_rows),
        _ptr(w_lat_down), _ptr(w_gate), _ptr(w_up), _ptr(w_lat_down_t), _ptr(w_gate_t),
        _ptr(w_up_t), _ptr(w_down_t), _ptr(w_lat_up_t), _ptr(g_out), T, d, L, E, k, F,
        int(capacity), int(group_size), int(rounding), int(seed) & 0xFFFFFFFF, _ptr(dx),
        _ptr(dw_router), _ptr(db_router), _ptr(dw_lat_down), _ptr(dw_gate), _ptr(dw_up),
        _ptr(dw_down), _ptr(dw_lat_up), _ptr(dtopk_w), _ptr(ws), _nbytes(ws), _stream(stream)))
