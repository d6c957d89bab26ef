"""Counter-based synthetic tensors, host side (numpy).

Every bf16 input tensor is defined element by element:

    value[i] = table_sigma[ hash(key(seed, tensor_id), i) >> 16 ]

where ``i`` is the flat row-major element index inside the tensor, ``hash`` is
two rounds of the 32-bit "lowbias32" integer mixer (Chris Wellons, *Prospecting
for Hash Functions*, 2018) over the low and high 32-bit words of ``i``, and
``table_sigma`` is a 65,536-entry inverse-CDF table of N(0, sigma^2) rounded to
bf16: entry j holds bf16(sigma * Phi^-1((j + 0.5) / 65536)).  The GPU fill
kernel (``synth_fill.hip``) evaluates the same function with native uint32
arithmetic, so host and device bytes are identical by construction; a GPU test
checks that on samples.

The fp32 router weights and the Zipf-like router bias are small and are drawn
on the host with numpy's PCG64 and uploaded.
"""
from __future__ import annotations

import concurrent.futures
import functools
import os

import numpy as np
from scipy.special import ndtri

from .configs import MoEConfig

# tensor ids (part of each tensor's hash key)
TID = {
    "x": 1, "w_router": 2, "b_router": 3, "w_dn": 4, "w_gate": 5, "w_up": 6,
    "w_down": 7, "w_lat_up": 8, "ws_gate": 9, "ws_up": 10, "ws_down": 11,
}

_M1 = np.uint32(0x7FEB352D)
_M2 = np.uint32(0x846CA68B)


def mix32(x: np.ndarray) -> np.ndarray:
    """lowbias32 mixer on a uint32 array (wrapping uint32 arithmetic)."""
    x = x.astype(np.uint32, copy=True)
    x ^= x >> np.uint32(16)
    x *= _M1
    x ^= x >> np.uint32(15)
    x *= _M2
    x ^= x >> np.uint32(16)
    return x


def tensor_key(seed: int, tensor_id: int) -> tuple[int, int]:
    """Two 32-bit key words for one tensor of one seeded input set."""
    a = mix32(np.array([(seed * 0x9E3779B9 + 0x632BE5AB) & 0xFFFFFFFF], np.uint32))
    b = mix32(a ^ np.uint32((tensor_id * 0x85EBCA6B) & 0xFFFFFFFF))
    c = mix32(b ^ np.uint32(0x27D4EB2F))
    return int(b[0]), int(c[0])


def hash_counter(start: int, count: int, key: tuple[int, int]) -> np.ndarray:
    """Hash of flat indices start .. start+count-1 (uint32 array)."""
    idx = np.arange(start, start + count, dtype=np.uint64)
    lo = (idx & np.uint64(0xFFFFFFFF)).astype(np.uint32)
    hi = (idx >> np.uint64(32)).astype(np.uint32)
    h = mix32(lo ^ np.uint32(key[0]))
    h = mix32(h ^ hi ^ np.uint32(key[1]))
    return h


def f32_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); returns uint16 bits."""
    b = np.ascontiguousarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return b.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    bits = np.asarray(bits, dtype=np.uint16)
    if bits.size <= _CHUNK:
        return bf16_bits_to_f32(bits).astype(np.float64)
    flat = bits.reshape(-1)
    out = np.empty(flat.size, np.float64)

    def work(i0):
        out[i0:i0 + _CHUNK] = bf16_bits_to_f32(flat[i0:i0 + _CHUNK])

    with concurrent.futures.ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(work, range(0, flat.size, _CHUNK)))
    return out.reshape(bits.shape)


@functools.lru_cache(maxsize=64)
def normal_table_bits(sigma: float) -> np.ndarray:
    """65,536-entry inverse-CDF table of N(0, sigma^2), bf16 bits."""
    j = np.arange(65536, dtype=np.float64)
    q = ndtri((j + 0.5) / 65536.0) * sigma
    t = f32_to_bf16_bits(q.astype(np.float32))
    t.setflags(write=False)
    return t


_CHUNK = 1 << 18


def _threads() -> int:
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:
        return max(1, min(16, os.cpu_count() or 1))


def normal_bf16_bits(key: tuple[int, int], sigma: float, start: int, count: int) -> np.ndarray:
    """bf16 bits of elements start .. start+count-1 of one synthetic tensor.
    Large requests are evaluated in cache-sized chunks on a thread pool (numpy
    releases the GIL inside these loops); the result does not depend on it."""
    table = normal_table_bits(sigma)
    if count <= _CHUNK:
        return table[hash_counter(start, count, key) >> np.uint32(16)]
    out = np.empty(count, np.uint16)

    def work(i0):
        n = min(_CHUNK, count - i0)
        out[i0:i0 + n] = table[hash_counter(start + i0, n, key) >> np.uint32(16)]

    with concurrent.futures.ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(work, range(0, count, _CHUNK)))
    return out


# ---------------------------------------------------------------------------
# per-tensor definitions of one workload
# ---------------------------------------------------------------------------

def tensor_specs(cfg: MoEConfig) -> dict:
    """name -> (shape, sigma) for every bf16 tensor of the layer."""
    T, d, L, E, F, Fs = cfg.T, cfg.d, cfg.L, cfg.E, cfg.F, cfg.Fs
    s = {
        "x": ((T, d), 1.0),
        "w_dn": ((L, d), d ** -0.5),
        "w_gate": ((E, F, L), L ** -0.5),
        "w_up": ((E, F, L), L ** -0.5),
        "w_down": ((E, L, F), F ** -0.5),
        "w_lat_up": ((d, L), L ** -0.5),
    }
    if Fs:
        s["ws_gate"] = ((Fs, d), d ** -0.5)
        s["ws_up"] = ((Fs, d), d ** -0.5)
        s["ws_down"] = ((d, Fs), Fs ** -0.5)
    return s


def host_tensor_bits(cfg: MoEConfig, name: str, index: tuple = ()) -> np.ndarray:
    """bf16 bits of a whole tensor, or of the sub-tensor at a leading ``index``
    (e.g. ``("w_gate", (e,))`` for expert e, ``("x", (t,))`` for token t)."""
    shape, sigma = tensor_specs(cfg)[name]
    key = tensor_key(cfg.seed, TID[name])
    sub = shape[len(index):]
    start = 0
    stride = int(np.prod(shape))
    for i, n in zip(index, shape):
        stride //= n
        start += int(i) * stride
    count = int(np.prod(sub)) if sub else 1
    return normal_bf16_bits(key, sigma, start, count).reshape(sub)


def host_tensor_f64(cfg: MoEConfig, name: str, index: tuple = ()) -> np.ndarray:
    return bf16_bits_to_f64(host_tensor_bits(cfg, name, index))


def host_rows_f64(cfg: MoEConfig, name: str, rows) -> np.ndarray:
    """Selected rows of a 2-D tensor (e.g. some tokens of x) as float64."""
    return np.stack([host_tensor_f64(cfg, name, (int(r),)) for r in rows]) if len(rows) else \
        np.zeros((0,) + tensor_specs(cfg)[name][0][1:])


def router_weights(cfg: MoEConfig) -> np.ndarray:
    """fp32 router weights W_r[E, d] ~ N(0, 1/d)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg.seed, TID["w_router"]])))
    return (rng.standard_normal((cfg.E, cfg.d)) * cfg.d ** -0.5).astype(np.float32)


def router_bias(cfg: MoEConfig) -> np.ndarray | None:
    """fp32 router bias: None for the balanced workloads; for the imbalanced one
    b_e = 2.0 * ln(1 / rank_e^1.2) = -2.4 ln(rank_e) over a seeded ranking."""
    if not cfg.zipf_bias:
        return None
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg.seed, TID["b_router"]])))
    rank = rng.permutation(cfg.E) + 1
    return (-2.4 * np.log(rank.astype(np.float64))).astype(np.float32)


def expert_weights_f64(cfg: MoEConfig, e: int):
    """(W_gate[e], W_up[e], W_down[e]) of one routed expert as float64."""
    return (host_tensor_f64(cfg, "w_gate", (e,)), host_tensor_f64(cfg, "w_up", (e,)),
            host_tensor_f64(cfg, "w_down", (e,)))


class LazyExperts:
    """Indexable view ``experts[e] -> (W_gate[e], W_up[e], W_down[e])`` that
    generates one expert's weights on demand (with a small cache), for shapes
    whose full expert set does not fit in host memory."""

    def __init__(self, cfg: MoEConfig, cache: int = 4):
        self.cfg = cfg
        self._cache: dict = {}
        self._order: list = []
        self._max = cache

    def __len__(self):
        return self.cfg.E

    def __getitem__(self, e):
        e = int(e)
        if e in self._cache:
            return self._cache[e]
        w = expert_weights_f64(self.cfg, e)
        self._cache[e] = w
        self._order.append(e)
        if len(self._order) > self._max:
            del self._cache[self._order.pop(0)]
        return w


def host_inputs_f64(cfg: MoEConfig) -> dict:
    """All inputs of a (small) workload as float64 arrays (bf16 values exactly)."""
    out = {name: host_tensor_f64(cfg, name) for name in tensor_specs(cfg)}
    out["w_router"] = router_weights(cfg).astype(np.float64)
    b = router_bias(cfg)
    out["b_router"] = None if b is None else b.astype(np.float64)
    return out
