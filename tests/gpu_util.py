"""Helpers shared by the GPU parity tests: comparison rules and oracle runs.

Comparison rules (written into the tests that use them):
* routing: the GPU's topk_idx must equal the oracle's, except that position j
  of a token may hold a different expert when the oracle's float64 logits of
  the two experts differ by less than ROUTE_GAP (1e-4): a near-tie, where both
  selections are correct to FP32 precision.  Every such swap is counted.
* logits: every FP32 logit must be within LOGIT_ATOL = ROUTE_GAP / 2 = 5e-5
  of the float64 logit.  That is what makes the near-tie rule consistent: if
  each logit is off by less than gap/2, two experts can only come out in the
  other order when their exact logits are closer than the gap.  (Measured on
  MI355X at full size: 1.4e-5 at d = 6656, 2.0e-5 at d = 8704.)
* gate weights: topk_w[t, j] is compared with the oracle's probability of the
  expert the GPU selected (unique per expert) to relative ROUTE_W_RTOL.
  w = exp(l - logsumexp(l)), so its relative error is at most the error of l
  plus that of logsumexp (<= the max logit error) plus a few fp32 rounding
  steps of exp and the division: 2 * LOGIT_ATOL = 1e-4.
* permutation arrays: bit-exact.
* outputs: max |gpu - oracle| / RMS(oracle) <= OUT_TOL against the oracle in
  bf16_operands mode (GEMM operands rounded to bf16 where the GPU feeds
  MFMA; fp32 accumulation on the GPU vs float64 in the oracle).
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from moe_synth import gen

ROUTE_GAP = 1e-4
LOGIT_ATOL = ROUTE_GAP / 2
ROUTE_W_RTOL = 2 * LOGIT_ATOL
OUT_TOL = 2e-2


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_np(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return gen.bf16_bits_to_f64(t.view(torch.int16).cpu().numpy().view(np.uint16))
    return t.cpu().numpy()


def experts_of(inp):
    return [(inp["w_gate"][e], inp["w_up"][e], inp["w_down"][e]) for e in range(inp["w_gate"].shape[0])]


def oracle_forward(cfg, inp, mode, routing=None, fp8=None):
    shared = None
    if cfg.Fs:
        shared = (inp["ws_gate"], inp["ws_up"], inp["ws_down"])
    return oracle.forward(inp["x"], inp["w_router"], inp["b_router"], cfg.k, inp["w_dn"],
                          experts_of(inp), inp["w_lat_up"], shared=shared, mode=mode,
                          routing=routing, fp8=fp8)


def routing_swaps(gpu_idx, ora_idx, logits, gap=ROUTE_GAP):
    """Tokens whose GPU selection differs from the oracle's.  Raises if any
    difference is not an allowed near-tie swap."""
    gpu_idx = np.asarray(gpu_idx)
    ora_idx = np.asarray(ora_idx)
    T, k = gpu_idx.shape
    bad = np.nonzero(np.any(gpu_idx != ora_idx, axis=1))[0]
    for t in bad:
        g, o = gpu_idx[t], ora_idx[t]
        assert len(set(g.tolist())) == k, f"token {t}: repeated expert {g}"
        lg = logits[t, g]
        lo = logits[t, o]
        assert np.all(np.abs(lg - lo) < gap), (
            f"token {t}: gpu {g} vs oracle {o}; logit gaps {np.abs(lg - lo)} exceed {gap}")
    return bad


def check_topk_w(gpu_idx, gpu_w, probs, rtol=ROUTE_W_RTOL):
    want = np.take_along_axis(probs, np.asarray(gpu_idx, np.int64), axis=1)
    rel = np.abs(np.asarray(gpu_w, np.float64) - want) / want
    assert rel.max() <= rtol, f"topk_w max rel err {rel.max():.3e}"
    return rel.max()


def rel_err(got, want):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    rms = np.sqrt(np.mean(want ** 2))
    return float(np.max(np.abs(got - want)) / rms), float(np.sqrt(np.mean((got - want) ** 2)) / rms)


def check_perm_valid(idx, E, counts, offsets, row_token, assign_row):
    """Invariants of a permutation of the given routing (used where the GPU's
    own routing has allowed swaps, so no unique oracle result exists)."""
    idx = np.asarray(idx, np.int64)
    T, k = idx.shape
    np.testing.assert_array_equal(counts, np.bincount(idx.ravel(), minlength=E))
    np.testing.assert_array_equal(offsets[1:] - offsets[:-1], counts)
    assert offsets[0] == 0 and offsets[-1] == T * k
    ar = np.asarray(assign_row, np.int64)
    np.testing.assert_array_equal(np.sort(ar.ravel()), np.arange(T * k))
    np.testing.assert_array_equal(np.asarray(row_token)[ar], np.repeat(np.arange(T)[:, None], k, 1))
    exp_of_row = np.searchsorted(offsets, ar, side="right") - 1
    np.testing.assert_array_equal(exp_of_row, idx)
    for e in range(E):
        seg = np.asarray(row_token)[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(seg) > 0)
