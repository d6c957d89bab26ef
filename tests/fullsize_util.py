"""Helpers of the full-size parity tests: the oracle on sampled expert rows and
tokens of a full workload.

The routed experts' weights of a full workload (97 GB at Base-1) do not fit
in host memory and take seconds per expert to generate on the host, so these
tests read the experts they check from the device copy that the input
generator's fill kernel wrote (the generator's own bytes: a GPU test checks
the device fill against the host generator bit for bit, and every expert read
here is checked again on slices of each matrix), widened exactly to float64.
No value computed by the layer's kernels is an oracle input.
"""
from __future__ import annotations

import concurrent.futures
import os

import numpy as np
import torch

import oracle
from moe_synth import gen
from tests import gpu_util as U

BLOCK = 32   # M tiles start on multiples of 32 rows of an expert's segment


def device_f64(t: torch.Tensor) -> np.ndarray:
    """A bf16 (or fp32) device tensor as a float64 host array (exact)."""
    return t.to(torch.float64).cpu().numpy()


def _check_slices(cfg, name, e, arr):
    """The device copy of expert e's matrix `name` equals the host generator
    on three slices (start, middle, end) of its flattened values."""
    shape, sigma = gen.tensor_specs(cfg)[name]
    key = gen.tensor_key(cfg.seed, gen.TID[name])
    per = int(np.prod(shape[1:]))
    flat = arr.reshape(-1)
    for off in (0, per // 2, per - 4096):
        want = gen.bf16_bits_to_f64(gen.normal_bf16_bits(key, sigma, e * per + off, 4096))
        np.testing.assert_array_equal(flat[off:off + 4096], want, err_msg=f"{name}[{e}]")


class DeviceExperts:
    """``experts[e] -> (W_gate[e], W_up[e], W_down[e])`` as float64, read from
    the generator-filled device tensors (each read checked against the host
    generator on slices), with a small cache."""

    def __init__(self, cfg, w_gate, w_up, w_down, cache=4):
        self.cfg, self.t = cfg, (w_gate, w_up, w_down)
        self._cache, self._order, self._max = {}, [], cache

    def __len__(self):
        return self.cfg.E

    def __getitem__(self, e):
        e = int(e)
        if e in self._cache:
            return self._cache[e]
        w = tuple(device_f64(t[e]) for t in self.t)
        for n, a in zip(("w_gate", "w_up", "w_down"), w):
            _check_slices(self.cfg, n, e, a)
        self._cache[e] = w
        self._order.append(e)
        if len(self._order) > self._max:
            del self._cache[self._order.pop(0)]
        return w


def choose_experts(counts, n_hot, n_ragged, rng):
    """The n_hot experts with the most rows, plus n_ragged others drawn at
    random among the experts whose last M tile is ragged (rows not a
    multiple of 32), or among the remaining used experts if there are too
    few of those."""
    counts = np.asarray(counts)
    used = np.nonzero(counts)[0]
    hot = used[np.argsort(-counts[used], kind="stable")][:n_hot]
    rest = np.setdiff1d(used, hot)
    ragged = rest[counts[rest] % BLOCK != 0]
    pool = ragged if ragged.size >= n_ragged else rest
    other = rng.choice(pool, size=min(n_ragged, pool.size), replace=False)
    return np.sort(hot), np.sort(other)


def sample_rows(a, b, rng, extra=8):
    """Rows of the segment [a, b) to check: the first and the last row of
    every 32-row block (so every M tile's first and last row, whatever the
    tile height) and `extra` random rows."""
    starts = np.arange(a, b, BLOCK)
    rows = np.concatenate([starts, np.minimum(starts + BLOCK - 1, b - 1),
                           rng.integers(a, b, size=min(extra, b - a))])
    return np.unique(rows)


def z_rows(cfg, x, w_dn, tokens, mode="bf16_operands"):
    """The oracle's latent rows of the given tokens."""
    return oracle.latent_down(x[tokens], w_dn, mode)


def check_expert_rows(tag, cfg, y_dev, offsets, row_token, experts, chosen, z_of, rng,
                      tol=U.OUT_TOL):
    """y_rows of the sampled rows of every chosen expert against the oracle's
    SwiGLU expert in bf16_operands mode on the same tokens (row_token of the
    GPU's permutation, which the caller has checked).  max|err| / RMS of the
    expert's sampled oracle rows <= tol, per expert.  Returns (rows checked,
    32-row blocks covered, worst error)."""
    n_rows = n_blocks = 0
    worst = 0.0
    for e in chosen:
        a, b = int(offsets[e]), int(offsets[e + 1])
        rows = sample_rows(a, b, rng)
        toks = row_token[rows]
        want = oracle.swiglu_expert(z_of(toks), *experts[e], mode="bf16_operands")
        got = y_dev[torch.from_numpy(rows.astype(np.int64)).to(y_dev.device)].cpu().numpy()
        err = U.rel_err(got, want)[0]
        worst = max(worst, err)
        assert err <= tol, f"{tag}: expert {e} ({b - a} rows) y max|err|/RMS {err:.3e}"
        n_rows += rows.size
        n_blocks += (b - a + BLOCK - 1) // BLOCK
    return n_rows, n_blocks, worst


def check_combine_up(tag, y_dev, topk_w, assign_row, out_dev, toks, w_lat_up, shared_out=None,
                     tol=U.OUT_TOL):
    """out of the sampled tokens against the oracle's combine (fixed slot
    order, float64) and bf16-operand up-projection of the GPU's expert rows
    and gate weights (plus the oracle's shared expert), i.e. the combine and
    up-projection stages on their own.  Returns the max|err| / RMS."""
    k = assign_row.shape[1]
    rows = assign_row[toks].reshape(-1).astype(np.int64)
    y = y_dev[torch.from_numpy(rows).to(y_dev.device)].cpu().numpy().astype(np.float64)
    c = oracle.combine(y, np.asarray(topk_w[toks], np.float64),
                       np.arange(len(toks) * k).reshape(len(toks), k))
    want = oracle.latent_up(c, w_lat_up, "bf16_operands")
    if shared_out is not None:
        want = want + shared_out
    got = out_dev[torch.from_numpy(np.asarray(toks, np.int64)).to(out_dev.device)].cpu().numpy()
    err = U.rel_err(got, want)[0]
    assert err <= tol, f"{tag}: combine + up-projection max|err|/RMS {err:.3e}"
    return err


def choose_tokens(idx, n, have, exclude, rng, pool=4096):
    """n tokens (none in `exclude`) chosen greedily to need as few experts
    outside `have` as possible (bounds the experts read for end-to-end
    checks); returns (tokens, experts needed)."""
    T = idx.shape[0]
    ok = np.setdiff1d(np.arange(T), exclude)
    cand = rng.choice(ok, size=min(pool, ok.size), replace=False)
    need = set(int(e) for e in have)
    chosen = []
    for _ in range(n):
        best = min((t for t in cand if t not in chosen),
                   key=lambda t: len(set(idx[t].tolist()) - need))
        chosen.append(int(best))
        need |= set(idx[best].tolist())
    return np.array(sorted(chosen)), need


def _threads():
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:
        return max(1, min(16, os.cpu_count() or 1))


def quantize_e4m3_rows(w, scale, chunk=256):
    """oracle.quantize_e4m3 of a weight matrix, evaluated on row chunks on a
    thread pool (the function is elementwise, so the values are identical;
    numpy releases the interpreter lock inside it)."""
    w = np.asarray(w)
    out = np.empty(w.shape, np.float64)

    def work(r0):
        out[r0:r0 + chunk] = oracle.quantize_e4m3(w[r0:r0 + chunk], scale)

    with concurrent.futures.ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(work, range(0, w.shape[0], chunk)))
    return out


def fp8_matmul_q(a, scale_a, qb, scale_b):
    """oracle.fp8_matmul(a, b, scale_a, scale_b) given qb =
    oracle.quantize_e4m3(b, scale_b) (e.g. from quantize_e4m3_rows), so a
    weight matrix used by several rows is quantized once."""
    qa = oracle.quantize_e4m3(a, scale_a)
    return (qa @ qb.T) / (float(np.float32(scale_a)) * float(np.float32(scale_b)))
