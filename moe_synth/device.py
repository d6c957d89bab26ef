"""Device side of the seeded input generator: fills torch GPU tensors with the
same bytes that moe_synth.gen produces on the host."""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

from . import gen
from .configs import MoEConfig

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsynth.so")
_lib = None
_tables: dict = {}


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"{_LIB_PATH} is not built: run `python -m moe_synth.build`")
        _lib = ctypes.CDLL(_LIB_PATH)
        _lib.synth_fill_bf16.restype = ctypes.c_int
        _lib.synth_fill_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                         ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p,
                                         ctypes.c_void_p]
        _lib.synth_calib_copy.restype = ctypes.c_int
        _lib.synth_calib_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                          ctypes.c_void_p]
    return _lib


def calibration_copy(src: torch.Tensor, dst: torch.Tensor):
    """One dispatch of a plain copy kernel (synth_calib_copy_kernel) of src into dst,
    for scaling HBM byte counters: reads and writes exactly src's bytes."""
    nbytes = src.numel() * src.element_size()
    assert dst.numel() * dst.element_size() >= nbytes
    rc = _load().synth_calib_copy(src.data_ptr(), dst.data_ptr(), nbytes,
                                  torch.cuda.current_stream(src.device).cuda_stream)
    if rc != 0:
        raise RuntimeError("synth_calib_copy failed")


def _table(sigma, device):
    key = (float(sigma), str(device))
    if key not in _tables:
        t = gen.normal_table_bits(sigma).view(np.int16).copy()
        _tables[key] = torch.from_numpy(t).to(device)
    return _tables[key]


def fill_(out: torch.Tensor, cfg: MoEConfig, name: str, start: int = 0):
    """Fill a contiguous bf16 GPU tensor with elements start.. of tensor `name`."""
    _, sigma = gen.tensor_specs(cfg)[name]
    k0, k1 = gen.tensor_key(cfg.seed, gen.TID[name])
    tab = _table(sigma, out.device)
    rc = _load().synth_fill_bf16(out.data_ptr(), out.numel(), start, k0, k1, tab.data_ptr(),
                                 torch.cuda.current_stream(out.device).cuda_stream)
    if rc != 0:
        raise RuntimeError("synth_fill_bf16 launch failed")
    return out


def device_tensor(cfg: MoEConfig, name: str, device="cuda"):
    shape, _ = gen.tensor_specs(cfg)[name]
    t = torch.empty(shape, dtype=torch.bfloat16, device=device)
    return fill_(t, cfg, name)


def device_inputs(cfg: MoEConfig, device="cuda"):
    """x and every weight of the workload on the GPU (bf16 tensors carry the
    generator's exact bits; router weights/bias fp32)."""
    out = {name: device_tensor(cfg, name, device) for name in gen.tensor_specs(cfg)}
    out["w_router"] = torch.from_numpy(gen.router_weights(cfg)).to(device)
    b = gen.router_bias(cfg)
    out["b_router"] = None if b is None else torch.from_numpy(b).to(device)
    return out
