"""GPU parity at the full workload sizes, in the launch configuration bench.py
times (LatentMoEBuffers + forward, all experts resident in HBM).

* routing: every token, against the oracle's float64/fp32 router, with the
  near-tie rule (swaps only where the oracle's logit gap is < 1e-4);
* permutation arrays: bit-exact over all T*k assignments when the routing has
  no swap (else checked for validity);
* outputs: sampled tokens, computed one by one by the oracle's per-token
  definition (only the experts those tokens use are generated on the host),
  max|err|/RMS <= 2e-2 against the bf16-operand oracle.
"""
import numpy as np
import pytest
import torch

import mixture_experts_layer_moe_amd as moe
import oracle
from moe_synth import CONFIGS, device, gen
from tests import gpu_util as U

pytestmark = [pytest.mark.gpu, pytest.mark.fullsize]

FULL = {  # workload -> number of sampled tokens for the output check
    "base1_small_batch": 3,
    "base1_compute": 3,
    "base1_imbalanced": 6,
    "base2": 2,
}


@pytest.fixture(scope="module")
def cuda():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.load()
    return torch.device("cuda:0")


def _choose_tokens(idx, n, exclude, rng):
    """n tokens (none in `exclude`), greedily preferring tokens whose experts
    are already needed, to bound the host-side weight generation."""
    T = idx.shape[0]
    ok = np.setdiff1d(np.arange(T), exclude)
    chosen = [int(rng.choice(ok))]
    need = set(idx[chosen[0]].tolist())
    cand = rng.choice(ok, size=min(4096, ok.size), replace=False)
    while len(chosen) < n:
        best = max((t for t in cand if t not in chosen),
                   key=lambda t: len(need & set(idx[t].tolist())))
        chosen.append(int(best))
        need |= set(idx[best].tolist())
    return np.array(sorted(chosen)), need


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", list(FULL))
def test_full_size_parity(cuda, name):
    cfg = CONFIGS[name]
    U.log(f"[full {name}] T={cfg.T} d={cfg.d} L={cfg.L} E={cfg.E} k={cfg.k} F={cfg.F} Fs={cfg.Fs}: "
          f"generating inputs on the GPU")
    dv = device.device_inputs(cfg, cuda)
    w = moe.LatentMoEWeights(dv["w_router"], dv["b_router"], dv["w_dn"], dv["w_gate"], dv["w_up"],
                             dv["w_down"], dv["w_lat_up"], dv.get("ws_gate"), dv.get("ws_up"),
                             dv.get("ws_down"))
    buf = moe.LatentMoEBuffers(cfg.T, cfg.d, cfg.L, cfg.E, cfg.k, cfg.F, cfg.Fs, device=cuda)
    U.log(f"[full {name}] forward pass")
    moe.forward(dv["x"], w, cfg.k, buf)
    torch.cuda.synchronize()
    g = {n: getattr(buf, n).cpu().numpy() for n in
         ("topk_idx", "topk_w", "expert_counts", "expert_offsets", "row_token", "assign_row")}
    out_dev = buf.out
    # the FP32 logits themselves, from a second routing call (same kernels)
    logits = torch.empty((cfg.T, cfg.E), dtype=torch.float32, device=cuda)
    idx2 = torch.empty_like(buf.topk_idx)
    w2 = torch.empty_like(buf.topk_w)
    moe.moe_route(dv["x"], dv["w_router"], dv["b_router"], cfg.k, idx2, w2, logits_out=logits,
                  ws=buf.ws)
    torch.cuda.synchronize()
    assert torch.equal(idx2, buf.topk_idx) and torch.equal(w2, buf.topk_w)
    g["logits"] = logits.cpu().numpy()
    del dv, w, logits, idx2, w2

    U.log(f"[full {name}] oracle routing over all {cfg.T} tokens")
    x = gen.host_tensor_f64(cfg, "x")
    b = gen.router_bias(cfg)
    ro = oracle.route(x, gen.router_weights(cfg).astype(np.float64),
                      None if b is None else b.astype(np.float64), cfg.k)
    lerr = float(np.abs(g["logits"] - ro["logits"]).max())
    U.log(f"[full {name}] max |logit err| = {lerr:.3e} (bound {U.LOGIT_ATOL:.1e})")
    assert lerr <= U.LOGIT_ATOL
    swaps = U.routing_swaps(g["topk_idx"], ro["topk_idx"], ro["logits"])
    wr = U.check_topk_w(g["topk_idx"], g["topk_w"], ro["probs"])
    U.log(f"[full {name}] near-tie swaps: {len(swaps)}; topk_w max rel err {wr:.2e}")
    assert len(swaps) <= max(2, cfg.T // 1000)

    if len(swaps) == 0:
        p = oracle.permute(ro["topk_idx"], cfg.E)
        for n in ("expert_counts", "expert_offsets", "row_token", "assign_row"):
            np.testing.assert_array_equal(g[n].reshape(p[n].shape), p[n], err_msg=n)
        U.log(f"[full {name}] permutation bit-exact over {cfg.T * cfg.k} assignments; "
              f"experts used {int(np.count_nonzero(p['expert_counts']))}, "
              f"max rows {int(p['expert_counts'].max())}")
    else:
        U.check_perm_valid(g["topk_idx"], cfg.E, g["expert_counts"], g["expert_offsets"],
                           g["row_token"], g["assign_row"])

    rng = np.random.default_rng(1234)
    toks, need = _choose_tokens(ro["topk_idx"], FULL[name], swaps, rng)
    U.log(f"[full {name}] oracle on sampled tokens {toks.tolist()} ({len(need)} experts)")
    out_rows = out_dev[torch.from_numpy(toks).to(cuda)].cpu().numpy()
    del buf, out_dev
    torch.cuda.empty_cache()
    experts = gen.LazyExperts(cfg, cache=len(need) + 1)
    shared = None
    if cfg.Fs:
        shared = tuple(gen.host_tensor_f64(cfg, n) for n in ("ws_gate", "ws_up", "ws_down"))
    ref = oracle.forward_tokens(x[toks], ro["topk_idx"][toks], ro["topk_w"][toks],
                                gen.host_tensor_f64(cfg, "w_dn"), experts,
                                gen.host_tensor_f64(cfg, "w_lat_up"), shared=shared,
                                mode="bf16_operands")
    eo = U.rel_err(out_rows, ref["out"])
    U.log(f"[full {name}] sampled out err max/rms {eo[0]:.2e}/{eo[1]:.2e}")
    assert eo[0] <= U.OUT_TOL
