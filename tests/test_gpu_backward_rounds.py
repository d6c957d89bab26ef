"""GPU parity of the backward pass on the multi-round dropless schedule
(moe_backward_rounds: the routed experts' data and weight gradients
computed round by round in buffers of min(T k, E capacity) rows).

* Against moe_backward on the same forward (the GPU's own routing), both
  gradient roundings: every row's data gradients are computed exactly as in
  the single pass (same tiles along K, same stochastic-rounding element
  indices), so dx, dW_router, db, dW_dn, dW_up and dtopk_w are bitwise
  equal; the expert weight gradients dW_gate, dW_up, dW_down sum each
  expert's rows in per-round pieces, so they equal the single pass's to
  fp32 summation order: RMS(diff)/RMS <= 1e-5 and max|diff|/RMS <= 1e-4
  (a reassociated fp32 sum of bf16 products).
* Against the oracle's backward (bf16_operands, the same rounding and seed,
  on the GPU's routing) with the rules of tests/test_gpu_backward.py.
* Schedules from one round down to many rounds, with and without capacity
  borrowing inside expert groups; a layer with a shared expert (its
  gradients from moe_shared_backward after the rounds).
* At full size, one EP-8 rank's share of Base-1 (T = 32,768, 64 experts,
  ~4,096 rows per expert) with a capacity of half the mean rows per expert in
  groups of 8 (the schedule bench.py --backward --capacity 0.5 times): the
  same comparison with the single pass at that shape, whose gradients
  tests/test_gpu_backward_fullsize.py checks against the oracle.
"""
import numpy as np
import pytest
import torch

import mixture_experts_layer_moe_amd as moe
import oracle
from moe_synth import CONFIGS, MoEConfig, device, gen
from tests import gpu_util as U
from tests.test_gpu_backward import GRAD_TOL_MAX, GRAD_TOL_RMS

pytestmark = pytest.mark.gpu

CASES = {
    "zipf": MoEConfig("zipf", T=1024, d=256, L=128, E=64, k=4, F=256, zipf_bias=True, seed=11),
    "deep": MoEConfig("deep", T=2048, d=256, L=256, E=8, k=2, F=512, seed=9),
    "shared": MoEConfig("shared", T=200, d=512, L=256, E=32, k=7, F=384, Fs=640, seed=5),
}
# (capacity as a fraction of the mean rows per expert, group size)
SCHEDULES = [(2.0, 8), (0.25, 1), (0.5, 64), (0.1, 3)]
SAME = ["dx", "dw_router", "db_router", "dw_lat_down", "dw_lat_up", "dtopk_w"]
SPLIT = ["dw_gate", "dw_up", "dw_down"]
ORACLE = [("dx", "dx"), ("dw_router", "dW_router"), ("dw_lat_down", "dW_dn"),
          ("dw_gate", "dW_gate"), ("dw_up", "dW_up"), ("dw_down", "dW_down"),
          ("dw_lat_up", "dW_lat_up"), ("dtopk_w", "dtopk_w")]


@pytest.fixture(scope="module")
def cuda():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.load()
    return torch.device("cuda:0")


_cache = {}


def _setup(name, cuda, rmode, seed):
    key = (name, rmode)
    if key in _cache:
        return _cache[key]
    cfg = CASES[name]
    host = gen.host_inputs_f64(cfg)
    dv = device.device_inputs(cfg, cuda)
    w = moe.LatentMoEWeights(dv["w_router"], dv["b_router"], dv["w_dn"], dv["w_gate"], dv["w_up"],
                             dv["w_down"], dv["w_lat_up"], dv.get("ws_gate"), dv.get("ws_up"),
                             dv.get("ws_down"))
    buf = moe.LatentMoEBuffers(cfg.T, cfg.d, cfg.L, cfg.E, cfg.k, cfg.F, cfg.Fs, device=cuda,
                               keep_logits=True)
    moe.forward(dv["x"], w, cfg.k, buf)
    wt = moe.backward_prepare(w)
    g_out = torch.from_numpy(np.random.default_rng(3000 + cfg.seed).standard_normal(
        (cfg.T, cfg.d)).astype(np.float32)).to(cuda)
    single = moe.LatentMoEGrads(cfg.T, cfg.d, cfg.L, cfg.E, cfg.k, cfg.F, device=cuda,
                                bias=dv["b_router"] is not None, Fs=cfg.Fs)
    moe.backward(dv["x"], w, wt, buf, g_out, single, rounding=rmode, seed=seed)
    torch.cuda.synchronize()
    _cache[key] = (cfg, host, dv, w, buf, wt, g_out, single)
    return _cache[key]


@pytest.mark.parametrize("sched", SCHEDULES, ids=[f"c{c}-g{g}" for c, g in SCHEDULES])
@pytest.mark.parametrize("rounding", ["rne", "sr"])
@pytest.mark.parametrize("name", list(CASES))
def test_backward_rounds(cuda, name, rounding, sched):
    seed = 2024
    rmode = moe.MOE_ROUND_STOCHASTIC if rounding == "sr" else moe.MOE_ROUND_NEAREST
    cfg, host, dv, w, buf, wt, g_out, single = _setup(name, cuda, rmode, seed)
    counts = buf.expert_counts.cpu().numpy()
    capacity = max(1, int(round(sched[0] * cfg.T * cfg.k / cfg.E)))
    group = min(sched[1], cfg.E)
    n_rounds, _ = oracle.round_schedule(buf.expert_offsets.cpu().numpy(), capacity, group)
    tag = f"bwd rounds {name}/{rounding} capacity {capacity} groups of {group}"
    U.log(f"[{tag}] {n_rounds} rounds (max rows per expert {int(counts.max())})")
    gr = moe.LatentMoEGrads(cfg.T, cfg.d, cfg.L, cfg.E, cfg.k, cfg.F, device=cuda,
                            bias=dv["b_router"] is not None, Fs=cfg.Fs, workspace=False)
    moe.backward_rounds(dv["x"], w, wt, buf, g_out, gr, capacity, group, rounding=rmode,
                        seed=seed)
    torch.cuda.synchronize()
    same = SAME + (["dws_gate", "dws_up", "dws_down"] if cfg.Fs else [])
    for n in same:
        a, b = getattr(gr, n), getattr(single, n)
        if a is None:
            continue
        assert torch.equal(a, b), f"{tag}: {n} differs from the single pass"
    for n in SPLIT:
        emax, erms = U.rel_err(U.to_np(getattr(gr, n)), U.to_np(getattr(single, n)))
        U.log(f"[{tag}] {n} vs single pass: max|diff|/RMS {emax:.1e}, RMS {erms:.1e}")
        assert emax <= 1e-4 and erms <= 1e-5, (n, emax, erms)
    # against the oracle (the GPU's routing replayed)
    routing = (U.to_np(buf.topk_idx), U.to_np(buf.topk_w).astype(np.float64))
    shared = (host["ws_gate"], host["ws_up"], host["ws_down"]) if cfg.Fs else None
    ref = oracle.backward(host["x"], host["w_router"], host["b_router"], cfg.k, host["w_dn"],
                          U.experts_of(host), host["w_lat_up"], U.to_np(g_out).astype(np.float64),
                          mode="bf16_operands", rounding=rounding, seed=seed, routing=routing,
                          shared=shared)
    for gname, oname in ORACLE:
        emax, erms = U.rel_err(U.to_np(getattr(gr, gname)), ref[oname])
        assert emax <= GRAD_TOL_MAX and erms <= GRAD_TOL_RMS, (gname, emax, erms)
    U.log(f"[{tag}] bitwise equal to the single pass on {same}; oracle rules met")


@pytest.mark.fullsize
@pytest.mark.timeout(900)
def test_backward_rounds_full_size(cuda):
    cfg = CONFIGS["base1_ep8"]
    T, d, L, E, k, F = cfg.T, cfg.d, cfg.L, cfg.E, cfg.k, cfg.F
    seed = 4321
    rmode = moe.MOE_ROUND_STOCHASTIC
    U.log(f"[bwd rounds full] {cfg.description}: inputs on the GPU, forward")
    dv = device.device_inputs(cfg, cuda)
    w = moe.LatentMoEWeights(dv["w_router"], dv["b_router"], dv["w_dn"], dv["w_gate"], dv["w_up"],
                             dv["w_down"], dv["w_lat_up"])
    buf = moe.LatentMoEBuffers(T, d, L, E, k, F, device=cuda, keep_logits=True)
    moe.forward(dv["x"], w, k, buf)
    wt = moe.backward_prepare(w)
    g = torch.Generator(device=cuda)
    g.manual_seed(seed)
    g_out = torch.randn((T, d), generator=g, dtype=torch.float32, device=cuda)
    U.log("[bwd rounds full] single pass")
    single = moe.LatentMoEGrads(T, d, L, E, k, F, device=cuda, bias=dv["b_router"] is not None)
    moe.backward(dv["x"], w, wt, buf, g_out, single, rounding=rmode, seed=seed)
    torch.cuda.synchronize()
    single.ws = None               # the single pass's workspace is not needed any more
    torch.cuda.empty_cache()
    capacity = int(round(0.5 * T * k / E))
    group = 8
    n_rounds, _ = oracle.round_schedule(buf.expert_offsets.cpu().numpy(), capacity, group)
    tag = f"bwd rounds full, capacity {capacity} in groups of {group}"
    U.log(f"[{tag}] {n_rounds} rounds")
    assert n_rounds >= 2
    gr = moe.LatentMoEGrads(T, d, L, E, k, F, device=cuda, bias=dv["b_router"] is not None,
                            workspace=False)
    moe.backward_rounds(dv["x"], w, wt, buf, g_out, gr, capacity, group, rounding=rmode,
                        seed=seed)
    torch.cuda.synchronize()
    for n in SAME:
        a, b = getattr(gr, n), getattr(single, n)
        if a is None:
            continue
        assert torch.equal(a, b), f"{tag}: {n} differs from the single pass"
    for n in SPLIT:
        a, b = getattr(gr, n), getattr(single, n)
        assert bool(torch.isfinite(a).all()), n
        dmax = dsq = bsq = 0.0
        for e in range(E):        # one expert at a time: float64 temporaries stay small
            de = (a[e] - b[e]).double()
            dmax = max(dmax, float(de.abs().max()))
            dsq += float(de.pow(2).sum())
            bsq += float(b[e].double().pow(2).sum())
        rms = (bsq / b.numel()) ** 0.5
        emax = dmax / rms
        erms = (dsq / b.numel()) ** 0.5 / rms
        U.log(f"[{tag}] {n} vs single pass: max|diff|/RMS {emax:.1e}, RMS {erms:.1e}")
        assert emax <= 1e-4 and erms <= 1e-5, (n, emax, erms)
    U.log(f"[{tag}] bitwise equal to the single pass on {SAME}")
