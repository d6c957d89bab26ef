"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every entry point that include/moe.h declares, sizes workspaces as documented
and rejects bad arguments before launching anything."""
import ctypes
import os
import re

import pytest

from mixture_experts_layer_moe_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_\w+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = _lib.load()
    names = declared_functions()
    assert {"moe_route", "moe_route_ex", "moe_permute", "moe_latent_ffn_forward", "moe_combine",
            "moe_workspace_bytes", "moe_status_string", "moe_set_kernel_events", "moe_fp8_amax",
            "moe_fp8_quantize", "moe_fp8_scale_update", "moe_latent_ffn_forward_fp8",
            "moe_workspace_bytes_rounds", "moe_latent_ffn_forward_rounds", "moe_backward_prepare",
            "moe_backward", "moe_grad_cast_bf16"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for code in (0, -1, -2, -3, -4, 7):
        assert isinstance(_lib.moe_status_string(code), str)
    assert "workspace" in _lib.moe_status_string(-3)


def test_workspace_sizes():
    a = lambda v: (v + 255) // 256 * 256  # noqa: E731
    T, d, L, E, k, F = 4096, 6656, 3072, 512, 8, 10240
    n = (T + 3) // 4     # 4-token chunks of the probability partials
    # router: the split weights, then the logits -- at T = 4,096 the routing
    # GEMM's 128 x 256 tiles (32 x 2) are split into 4 K chunks of partial
    # logits -- then the probability partials
    assert _lib.moe_workspace_bytes(0, T, d, L, E, k, F) == \
        a(3 * E * d * 2) + a(4 * T * E * 4) + a((n + (n + 63) // 64) * E * 4)
    T2 = 32768     # 512 tiles of 128 x 256: no split
    n2 = (T2 + 3) // 4
    assert _lib.moe_workspace_bytes(0, T2, d, L, E, k, F) == \
        a(3 * E * d * 2) + a(T2 * E * 4) + a((n2 + (n2 + 63) // 64) * E * 4)
    assert _lib.moe_workspace_bytes(1, T, d, L, E, k, F) == 2 * a(16 * E * 4)
    mt = (T * k + min(E, T * k) * 127) // 128      # M tiles of 128 rows, any routing
    assert _lib.moe_workspace_bytes(2, T, d, L, E, k, F) == \
        a(T * L * 2) + a(T * k * F * 2) + 2 * a((E + 1) * 4) + 2 * a(mt * 4) + a(16 * 4)
    assert _lib.moe_workspace_bytes(3, T, d, L, E, k, F) == a(T * L * 2)
    assert _lib.moe_workspace_bytes(4, T, d, L, E, k, F) == \
        a(T * L) + a(T * k * F) + 2 * a((E + 1) * 4) + 2 * a(mt * 4) + a(16 * 4)
    assert _lib.moe_workspace_bytes(9, T, d, L, E, k, F) == 0
    assert _lib.moe_workspace_bytes(0, -1, d, L, E, k, F) == 0


def test_kernel_event_ids():
    lib = _lib.load()
    assert lib.moe_set_kernel_events(len(_lib.KERNELS), None, None) == -1
    assert lib.moe_set_kernel_events(-1, None, None) == -1
    for kid in _lib.KERNELS.values():
        assert lib.moe_set_kernel_events(kid, None, None) == 0


P = 1 << 20   # a 16-byte aligned fake device address; never dereferenced on these paths


@pytest.mark.parametrize("T,d,E,k,want", [
    (-1, 512, 16, 2, -1), (8, 512, 16, 0, -1), (8, 512, 16, 17, -1), (8, 512, 0, 1, -1),
    (8, 512, 32, 17, -2), (8, 512, 2048, 8, -2), (8, 500, 16, 2, -2), (8, 0, 16, 2, -1),
])
def test_route_rejects_bad_shapes(T, d, E, k, want):
    lib = _lib.load()
    assert lib.moe_route(P, P, None, T, d, E, k, P, P, None, P, 1 << 40, None) == want


def test_route_rejects_null_misaligned_and_small_workspace():
    lib = _lib.load()
    assert lib.moe_route(None, P, None, 8, 512, 16, 2, P, P, None, P, 1 << 40, None) == -1
    assert lib.moe_route(P, P, None, 8, 512, 16, 2, None, P, None, P, 1 << 40, None) == -1
    assert lib.moe_route(P + 2, P, None, 8, 512, 16, 2, P, P, None, P, 1 << 40, None) == -2
    need = _lib.moe_workspace_bytes(0, 8, 512, 0, 16, 2, 0)
    assert lib.moe_route(P, P, None, 8, 512, 16, 2, P, P, None, P, need - 1, None) == -3
    # T == 0 is a no-op success (nothing launched)
    assert lib.moe_route(P, P, None, 0, 512, 16, 2, P, P, None, P, 0, None) == 0


def test_route_ex_rejects_unknown_bias_mode():
    lib = _lib.load()
    lib.moe_route_ex.restype = ctypes.c_int
    lib.moe_route_ex.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                 ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                 ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    assert lib.moe_route_ex(P, P, P, 2, 8, 512, 16, 2, P, P, None, None, P, 1 << 40, None) == -1
    assert lib.moe_route_ex(P, P, P, -1, 8, 512, 16, 2, P, P, None, None, P, 1 << 40, None) == -1
    assert lib.moe_route_ex(P, P, P, 1, 0, 512, 16, 2, P, P, None, None, P, 0, None) == 0


def test_permute_rejects_bad_args():
    lib = _lib.load()
    assert lib.moe_permute(P, 8, 0, 16, P, P, P, P, P, 1 << 30, None) == -1
    assert lib.moe_permute(P, 8, 4, 2, P, P, P, P, P, 1 << 30, None) == -1
    assert lib.moe_permute(P, 8, 2, 2048, P, P, P, P, P, 1 << 30, None) == -2
    assert lib.moe_permute(P, 8, 2, 16, None, P, P, P, P, 1 << 30, None) == -1
    assert lib.moe_permute(P, 8, 2, 16, P, P, P, P, P, 10, None) == -3
    assert lib.moe_permute(P, (1 << 31) // 8, 8, 16, P, P, P, P, P, 1 << 40, None) == -2


def _ffn(lib, T=8, d=512, L=256, E=16, k=2, F=512, Fs=0, x=P, wsb=1 << 40, hs=None, wsg=None):
    return lib.moe_latent_ffn_forward(x, P, P, P, P, P, P, wsg, wsg, T, d, L, E, k, F, Fs, P, hs,
                                      P, wsb, None)


def test_latent_ffn_rejects_bad_args():
    lib = _lib.load()
    assert _ffn(lib, L=200) == -2
    assert _ffn(lib, F=0) == -2
    assert _ffn(lib, Fs=-64) == -1
    assert _ffn(lib, Fs=128) == -1            # shared widths without shared pointers
    assert _ffn(lib, x=None) == -1
    assert _ffn(lib, x=P + 8) == -2
    assert _ffn(lib, wsb=100) == -3
    assert _ffn(lib, T=0) == 0


def test_combine_rejects_bad_args():
    lib = _lib.load()
    assert lib.moe_combine(P, P, P, P, None, None, 8, 512, 256, 0, 0, P, P, 1 << 30, None) == -1
    assert lib.moe_combine(P, P, P, P, None, None, 8, 500, 256, 2, 0, P, P, 1 << 30, None) == -2
    assert lib.moe_combine(P, P, P, P, None, None, 8, 512, 256, 2, 64, P, P, 1 << 30, None) == -1
    assert lib.moe_combine(P, P, P, P, None, None, 8, 512, 256, 2, 0, P, P, 16, None) == -3
    assert lib.moe_combine(None, P, P, P, None, None, 8, 512, 256, 2, 0, P, P, 1 << 30, None) == -1
    assert lib.moe_combine(P, P, P, P, None, None, 0, 512, 256, 2, 0, P, P, 0, None) == 0


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "_LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        _lib.load()


def test_fp8_support_calls_reject_bad_args():
    lib = _lib.load()
    # amax: negative sizes, numel not a multiple of 8, misaligned source
    assert lib.moe_fp8_amax(P, -1, 64, P, None) == -1
    assert lib.moe_fp8_amax(P, 2, 60, P, None) == -2
    assert lib.moe_fp8_amax(P + 2, 2, 64, P, None) == -2
    assert lib.moe_fp8_amax(None, 2, 64, P, None) == -1
    assert lib.moe_fp8_amax(P, 0, 64, P, None) == 0
    # quantize
    assert lib.moe_fp8_quantize(P, 2, 64, None, P, None) == -1
    assert lib.moe_fp8_quantize(P, 2, 64, P, P + 8, None) == -2
    assert lib.moe_fp8_quantize(P, 70000, 64, P, P, None) == -2
    assert lib.moe_fp8_quantize(P, 2, 0, P, P, None) == 0
    # scale update: slot outside the history
    assert lib.moe_fp8_scale_update(P, P, 2, 1024, 1024, P, None) == -1
    assert lib.moe_fp8_scale_update(P, P, 2, 0, 0, P, None) == -1
    assert lib.moe_fp8_scale_update(P, P, 2, 1024, -1, P, None) == -1
    assert lib.moe_fp8_scale_update(P, None, 2, 1024, 3, P, None) == -1
    assert lib.moe_fp8_scale_update(P, P, 0, 1024, 3, P, None) == 0


def _ffn8(lib, T=8, d=512, L=256, E=16, k=2, F=512, Fs=0, wsc=P, amax=P, wsb=1 << 40):
    return lib.moe_latent_ffn_forward_fp8(P, P, P, P, P, P, P, wsc, P, None, None, T, d, L, E, k,
                                          F, Fs, P, None, amax, P, wsb, None)


def test_latent_ffn_fp8_rejects_bad_args():
    lib = _lib.load()
    assert _ffn8(lib, L=192) == -2            # FP8 expert widths are multiples of 128
    assert _ffn8(lib, F=320) == -2
    assert _ffn8(lib, wsc=None) == -1         # weight scales required
    assert _ffn8(lib, amax=None) == -1        # amax output required
    assert _ffn8(lib, k=0) == -1
    need = _lib.moe_workspace_bytes(4, 8, 512, 256, 16, 2, 512)
    assert _ffn8(lib, wsb=need - 1) == -3
    assert _ffn8(lib, T=0) == 0


def test_rounds_workspace_and_bad_args():
    a = lambda v: (v + 255) // 256 * 256  # noqa: E731
    T, d, L, E, k, F, C, G = 4096, 6656, 3072, 512, 8, 10240, 96, 8
    rb = min(T * k, E * C)
    mt = (rb + min(E, rb) * 127) // 128
    assert _lib.moe_workspace_bytes_rounds(T, d, L, E, k, F, 0, C, G) == \
        a(T * L * 2) + a(E * C * F * 2) + 3 * a(E * 4) + 2 * a((E + 1) * 4) + 2 * a(mt * 4) + a(64)
    assert _lib.moe_workspace_bytes_rounds(T, d, L, E, k, F, 0, 0, G) == 0
    lib = _lib.load()

    def call(C=64, G=8, T=8, wsb=1 << 40, E=16, k=2, L=256):
        return lib.moe_latent_ffn_forward_rounds(P, P, P, P, P, P, P, None, None, T, 512, L, E, k,
                                                 512, 0, C, G, P, None, None, P, wsb, None)
    assert call(C=0) == -1
    assert call(G=0) == -1
    assert call(k=0) == -1
    assert call(L=192 + 32) == -2
    assert call(wsb=100) == -3
    assert call(T=0) == 0


def _bwd(lib, T=8, d=512, L=256, E=16, k=2, F=512, rounding=1, bias_mode=0, x=P, dx=P, wsb=1 << 40):
    ptrs = [P] * 15
    outs = [dx, P, None, P, P, P, P, P, None]
    return lib.moe_backward(x, P, P, bias_mode, *ptrs, T, d, L, E, k, F, rounding, 7, *outs, P,
                            wsb, None)


def test_backward_workspace_and_bad_args():
    lib = _lib.load()
    T, d, L, E, k, F = 4096, 6656, 3072, 64, 8, 10240
    assert _lib.moe_workspace_bytes(5, T, d, L, E, k, F) > T * k * F * 4   # dh in fp32
    assert _lib.moe_workspace_bytes(5, T, 0, L, E, k, F) == 0
    assert _bwd(lib, rounding=2) == -1
    assert _bwd(lib, bias_mode=3) == -1
    assert _bwd(lib, k=0) == -1
    assert _bwd(lib, L=200) == -2
    assert _bwd(lib, x=None) == -1
    assert _bwd(lib, dx=None) == -1
    assert _bwd(lib, x=P + 4) == -2
    assert _bwd(lib, wsb=1000) == -3
    assert _bwd(lib, T=0) == 0
    assert _bwd(lib, T=1 << 19, k=8, L=64, d=64, F=64) == -2    # T*k rows beyond 2^22
    # prepare: sizes and pointers are checked before any launch
    assert lib.moe_backward_prepare(P, P, P, P, P, 512, 256, 0, 512, P, P, P, P, P, None) == -1
    assert lib.moe_backward_prepare(P, P, P, P, P, 500, 256, 16, 512, P, P, P, P, P, None) == -2
    assert lib.moe_backward_prepare(P, P, P, None, P, 512, 256, 16, 512, P, P, P, P, P, None) == -1

    assert lib.moe_grad_cast_bf16(P, 64, 2, 0, 1, P, None) == -1
    assert lib.moe_grad_cast_bf16(P, 62, 1, 0, 1, P, None) == -2
    assert lib.moe_grad_cast_bf16(P + 4, 64, 1, 0, 1, P, None) == -2
    assert lib.moe_grad_cast_bf16(None, 64, 1, 0, 1, P, None) == -1
    assert lib.moe_grad_cast_bf16(P, 0, 1, 0, 1, P, None) == 0


def _bwd8(lib, T=8, d=512, L=256, E=16, k=2, F=512, rounding=1, gscale=P, gamax=P, wg8=P,
          wsb=1 << 40):
    # x, w_router, logits, bias_mode, topk_idx, topk_w, offsets, row_token, assign_row, y_rows,
    # w_lat_down, w_gate, w_up, w_lat_down_t, w_gate_t8, w_up_t8, w_down_t8, w_scale,
    # w_lat_up_t, g_out, grad_scale
    ins = [P] * 10 + [wg8, P, P, P, P, P, gscale]
    outs = [P, P, None, P, P, P, P, P, None, gamax]
    return lib.moe_backward_fp8(P, P, P, 0, *ins, T, d, L, E, k, F, rounding, 7, *outs, P, wsb,
                                None)


def test_backward_fp8_workspace_and_bad_args():
    lib = _lib.load()
    T, d, L, E, k, F = 4096, 6656, 3072, 64, 8, 10240
    b16 = _lib.moe_workspace_bytes(5, T, d, L, E, k, F)
    b8 = _lib.moe_workspace_bytes(6, T, d, L, E, k, F)
    # the E5M2 codes of dy [T k, L] and dg, du [T k, F] on top of the bf16 backward's
    assert b8 >= b16 + T * k * (L + 2 * F)
    assert _bwd8(lib, rounding=2) == -1
    assert _bwd8(lib, L=192) == -2          # FP8 widths: multiples of 128
    assert _bwd8(lib, F=320) == -2
    assert _bwd8(lib, gscale=None) == -1
    assert _bwd8(lib, gamax=None) == -1
    assert _bwd8(lib, wg8=None) == -1
    assert _bwd8(lib, wg8=P + 4) == -2
    # a workspace sized for the bf16 backward is too small (the call's own shape)
    small16 = _lib.moe_workspace_bytes(5, 8, 512, 256, 16, 2, 512)
    assert small16 < _lib.moe_workspace_bytes(6, 8, 512, 256, 16, 2, 512)
    assert _bwd8(lib, wsb=small16) == -3
    assert _bwd8(lib, T=0) == 0
    # the E5M2 cast
    assert lib.moe_grad_cast_e5m2(P, 64, P, 2, 0, 6, P, None) == -1
    assert lib.moe_grad_cast_e5m2(P, 62, P, 1, 0, 6, P, None) == -2
    assert lib.moe_grad_cast_e5m2(P + 4, 64, P, 1, 0, 6, P, None) == -2
    assert lib.moe_grad_cast_e5m2(P, 64, P, 1, 0, 6, P + 2, None) == -2
    assert lib.moe_grad_cast_e5m2(P, 64, None, 1, 0, 6, P, None) == -1
    assert lib.moe_grad_cast_e5m2(P, 0, P, 1, 0, 6, P, None) == 0


# ---- the Python binding checks every buffer's extent against the shapes it
# passes to the C ABI (which receives only pointers and sizes), before any
# launch: CPU tensors of the right dtype reach the device check only when
# every extent agrees ----

def _t(shape, dtype):
    import torch
    return torch.zeros(shape, dtype=dtype)


def _ffn_set(T=8, d=64, L=64, E=4, k=2, F=64, Fs=0):
    import torch
    bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32
    a = dict(x=_t((T, d), bf), w_lat_down=_t((L, d), bf), expert_offsets=_t((E + 1,), i32),
             row_token=_t((T * k,), i32), w_gate=_t((E, F, L), bf), w_up=_t((E, F, L), bf),
             w_down=_t((E, L, F), bf), ws_gate=_t((Fs, d), bf) if Fs else None,
             ws_up=_t((Fs, d), bf) if Fs else None, k=k, y_rows=_t((T * k, L), f32),
             hs=_t((T, Fs), bf) if Fs else None, ws=_t((256,), torch.uint8))
    return a


@pytest.mark.parametrize("Fs", [0, 128])
@pytest.mark.parametrize("bad", ["w_up", "w_down", "y_rows", "row_token", "expert_offsets", "hs",
                                 "ws_up", "w_lat_down"])
def test_binding_rejects_mismatched_ffn_buffers(bad, Fs):
    import torch
    a = _ffn_set(Fs=Fs)
    if a.get(bad) is None:
        pytest.skip("buffer absent without a shared expert")
    t = a[bad]
    a[bad] = torch.zeros((t.shape[0] + 1,) + tuple(t.shape[1:]), dtype=t.dtype)
    with pytest.raises(ValueError, match="shape|values"):
        _lib.moe_latent_ffn_forward(**a)
    a = _ffn_set(Fs=Fs)
    with pytest.raises(ValueError, match="GPU tensor"):
        _lib.moe_latent_ffn_forward(**a)


def test_binding_rejects_mismatched_route_permute_combine_buffers():
    import torch
    bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32
    T, d, E, k, L = 8, 64, 4, 2, 64
    good = dict(x=_t((T, d), bf), w_router=_t((E, d), f32), b_router=_t((E,), f32), k=k,
                topk_idx=_t((T, k), i32), topk_w=_t((T, k), f32), logits_out=_t((T, E), f32),
                ws=_t((256,), torch.uint8))
    for bad, shp in (("w_router", (E, d + 64)), ("b_router", (E + 1,)), ("topk_idx", (T, k + 1)),
                     ("topk_w", (T + 1, k)), ("logits_out", (T, E + 1))):
        a = dict(good)
        a[bad] = _t(shp, a[bad].dtype)
        with pytest.raises(ValueError, match="shape"):
            _lib.moe_route(**a)
    with pytest.raises(ValueError, match="GPU tensor"):
        _lib.moe_route(**good)
    pgood = dict(topk_idx=_t((T, k), i32), E=E, expert_counts=_t((E,), i32),
                 expert_offsets=_t((E + 1,), i32), row_token=_t((T * k,), i32),
                 assign_row=_t((T, k), i32), ws=_t((256,), torch.uint8))
    for bad, n in (("expert_counts", E - 1), ("expert_offsets", E), ("row_token", T * k - 1),
                   ("assign_row", T * k + 1)):
        a = dict(pgood)
        a[bad] = _t((n,), i32)
        with pytest.raises(ValueError, match="values"):
            _lib.moe_permute(**a)
    with pytest.raises(ValueError, match="GPU tensor"):
        _lib.moe_permute(**pgood)
    cgood = dict(y_rows=_t((T * k, L), f32), topk_w=_t((T, k), f32), assign_row=_t((T, k), i32),
                 w_lat_up=_t((d, L), bf), hs=None, ws_down=None, out=_t((T, d), f32),
                 ws=_t((256,), torch.uint8))
    for bad, shp in (("y_rows", (T * k - 1, L)), ("assign_row", (T, k - 1)), ("out", (T, d + 1))):
        a = dict(cgood)
        a[bad] = _t(shp, a[bad].dtype)
        with pytest.raises(ValueError, match="shape"):
            _lib.moe_combine(**a)
    a = dict(cgood)
    a["hs"] = _t((T, 64), bf)
    with pytest.raises(ValueError, match="together"):
        _lib.moe_combine(**a)
    with pytest.raises(ValueError, match="GPU tensor"):
        _lib.moe_combine(**cgood)


def test_permute_noalloc_rejects_bad_args():
    lib = _lib.load()
    assert lib.moe_permute_noalloc(P, -1, 2, 16, P, P, P, P, None) == -1
    assert lib.moe_permute_noalloc(P, 8, 0, 16, P, P, P, P, None) == -1
    assert lib.moe_permute_noalloc(P, 8, 17, 16, P, P, P, P, None) == -1
    assert lib.moe_permute_noalloc(P, 8, 17, 32, P, P, P, P, None) == -2
    assert lib.moe_permute_noalloc(P, 8, 2, 16, None, P, P, P, None) == -1
    assert lib.moe_permute_noalloc(None, 8, 2, 16, P, P, P, P, None) == -1
    # the static scratch holds 2^21 int32: 2 * ceil(T / 256) * E beyond that
    assert lib.moe_permute_noalloc(P, 600_000, 1, 512, P, P, P, P, None) == -2


def test_backward_rounds_and_shared_backward_args():
    lib = _lib.load()
    T, d, L, E, k, F = 64, 128, 64, 8, 2, 128
    assert lib.moe_workspace_bytes_backward_rounds(T, d, L, E, k, F, 0, 4) == 0
    assert lib.moe_workspace_bytes_backward_rounds(T, d, L, E, k, F, 16, 0) == 0
    single = lib.moe_workspace_bytes(5, T, d, L, E, k, F, 0)
    # a round holds at most min(T k, E C) rows: the per-round buffers shrink
    # with the capacity, and never exceed the single pass's
    small = lib.moe_workspace_bytes_backward_rounds(T, d, L, E, k, F, 4, 2)
    large = lib.moe_workspace_bytes_backward_rounds(T, d, L, E, k, F, 1000, 2)
    assert 0 < small < large and large >= single
    args = [P] * 18 + [T, d, L, E, k, F]
    tail = [1, 12, P, P, P, P, P, P, P, P, P, P, 1 << 40, None]
    assert lib.moe_backward_rounds(*(args[:3] + [0] + args[3:] + [0, 4] + tail)) == -1
    assert lib.moe_backward_rounds(*(args[:3] + [0] + args[3:] + [16, 0] + tail)) == -1
    # the shared expert's backward
    assert lib.moe_workspace_bytes(7, T, d, 0, 0, 0, 0, 128) > 0
    assert lib.moe_workspace_bytes(7, T, d, 0, 0, 0, 0, 0) == 0
    sargs = [P] * 7
    assert lib.moe_shared_backward(*sargs, T, d, 128, 2, 0, P, P, P, P, P, 1 << 40, None) == -1
    assert lib.moe_shared_backward(*sargs, T, d, 100, 1, 0, P, P, P, P, P, 1 << 40, None) == -2
    assert lib.moe_shared_backward(*sargs, T, d, 128, 1, 0, P, P, P, P, None, 1 << 40, None) == -1
    assert lib.moe_shared_backward(*sargs, T, d, 128, 1, 0, P, P, P, P, P, 16, None) == -3
    assert lib.moe_shared_backward(*sargs, 0, d, 128, 1, 0, P, P, P, P, P, 0, None) == 0
    assert lib.moe_backward_prepare_shared(P, P, P, d, 0, P, P, P, None) == -1
    assert lib.moe_backward_prepare_shared(P, P, None, d, 128, P, P, P, None) == -1
