"""GPU parity of the Base-2 shared expert's backward (moe_shared_backward,
called by the layer's backward after moe_backward) against the CPU oracle.

* Small layers with a shared expert: the whole backward (routed experts,
  latent projections, router and shared expert) against the oracle's
  backward with the shared expert, on the GPU's routing, in bf16_operands
  mode with the same gradient rounding (nearest or stochastic, same seed);
  the rules of tests/test_gpu_backward.py (RMS(err)/RMS <= 1e-3,
  max|err|/RMS <= 5e-2) for every gradient, the shared expert's three
  weight gradients included; two runs bitwise equal.
* The shared expert alone at the full Base-2 shape (T = 16,384, d = 8,704,
  Fs = 12,288), stochastic rounding, dx accumulated onto zeros: dx of
  sampled tokens, and blocks of dWs_gate, dWs_up (sampled rows of Fs,
  sampled columns of d) and dWs_down (sampled rows of d, sampled columns of
  Fs), each summed over all 16,384 tokens, against the oracle computed one
  token or one column at a time from the same definitions.
"""
import numpy as np
import pytest
import torch

import mixture_experts_layer_moe_amd as moe
import oracle
from moe_synth import CONFIGS, MoEConfig, device, gen
from oracle import latent_moe_backward as OB
from tests import gpu_util as U
from tests.test_gpu_backward import GRAD_TOL_MAX, GRAD_TOL_RMS

pytestmark = pytest.mark.gpu

CASES = {
    "shared": MoEConfig("shared_bwd", T=200, d=512, L=256, E=32, k=7, F=384, Fs=640, seed=41),
    # T not a multiple of 64 (padded K of the weight gradients), Fs not a
    # multiple of the 256-wide tiles
    "ragged": MoEConfig("ragged_shared_bwd", T=300, d=320, L=192, E=24, k=3, F=320, Fs=448,
                        seed=43),
}


@pytest.fixture(scope="module")
def cuda():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.load()
    return torch.device("cuda:0")


def check(tag, got, want):
    emax, erms = U.rel_err(got, want)
    U.log(f"[{tag}] max|err|/RMS {emax:.2e}, RMS err {erms:.2e}")
    assert emax <= GRAD_TOL_MAX, (tag, emax)
    assert erms <= GRAD_TOL_RMS, (tag, erms)


def _gpu_backward(cfg, dv, g_out, cuda, rmode, seed):
    w = moe.LatentMoEWeights(dv["w_router"], dv["b_router"], dv["w_dn"], dv["w_gate"], dv["w_up"],
                             dv["w_down"], dv["w_lat_up"], dv["ws_gate"], dv["ws_up"],
                             dv["ws_down"])
    buf = moe.LatentMoEBuffers(cfg.T, cfg.d, cfg.L, cfg.E, cfg.k, cfg.F, cfg.Fs, device=cuda,
                               keep_logits=True)
    moe.forward(dv["x"], w, cfg.k, buf)
    wt = moe.backward_prepare(w)
    grads = moe.LatentMoEGrads(cfg.T, cfg.d, cfg.L, cfg.E, cfg.k, cfg.F, device=cuda,
                               bias=dv["b_router"] is not None, Fs=cfg.Fs)
    moe.backward(dv["x"], w, wt, buf, torch.from_numpy(g_out).to(cuda), grads, rounding=rmode,
                 seed=seed)
    torch.cuda.synchronize()
    return buf, grads


GRADS = [("dx", "dx"), ("dw_router", "dW_router"), ("dw_lat_down", "dW_dn"),
         ("dw_gate", "dW_gate"), ("dw_up", "dW_up"), ("dw_down", "dW_down"),
         ("dw_lat_up", "dW_lat_up"), ("dtopk_w", "dtopk_w"), ("dws_gate", "dWs_gate"),
         ("dws_up", "dWs_up"), ("dws_down", "dWs_down")]


@pytest.mark.parametrize("rounding", ["rne", "sr"])
@pytest.mark.parametrize("name", list(CASES))
def test_backward_with_shared_expert_matches_oracle(cuda, name, rounding):
    cfg = CASES[name]
    host = gen.host_inputs_f64(cfg)
    dv = device.device_inputs(cfg, cuda)
    g_out = np.random.default_rng(2000 + cfg.seed).standard_normal((cfg.T, cfg.d)).astype(np.float32)
    seed = 777
    rmode = moe.MOE_ROUND_STOCHASTIC if rounding == "sr" else moe.MOE_ROUND_NEAREST
    U.log(f"[shared bwd {name}/{rounding}] gpu forward + backward")
    buf, grads = _gpu_backward(cfg, dv, g_out, cuda, rmode, seed)
    routing = (U.to_np(buf.topk_idx), U.to_np(buf.topk_w).astype(np.float64))
    ref = oracle.backward(host["x"], host["w_router"], host["b_router"], cfg.k, host["w_dn"],
                          U.experts_of(host), host["w_lat_up"], g_out.astype(np.float64),
                          mode="bf16_operands", rounding=rounding, seed=seed, routing=routing,
                          shared=(host["ws_gate"], host["ws_up"], host["ws_down"]))
    for gname, oname in GRADS:
        check(f"shared bwd {name}/{rounding} {gname}", U.to_np(getattr(grads, gname)), ref[oname])
    # deterministic: a second run gives the same bits
    _, grads2 = _gpu_backward(cfg, dv, g_out, cuda, rmode, seed)
    for gname, _ in GRADS:
        assert torch.equal(getattr(grads, gname), getattr(grads2, gname)), gname


N_SAMPLE = 4
N_COLS = 16


@pytest.mark.fullsize
@pytest.mark.timeout(900)
def test_shared_backward_full_size_sampled(cuda):
    cfg = CONFIGS["base2"]
    T, d, Fs = cfg.T, cfg.d, cfg.Fs
    seed = 4242
    U.log(f"[shared bwd full] T={T} d={d} Fs={Fs}: inputs on the GPU")
    xd = device.device_tensor(cfg, "x", cuda)
    wsd = {n: device.device_tensor(cfg, n, cuda) for n in ("ws_gate", "ws_up", "ws_down")}
    g_out = np.random.default_rng(seed).standard_normal((T, d)).astype(np.float32)
    wt = {n: torch.empty(shp, dtype=torch.bfloat16, device=cuda)
          for n, shp in (("ws_gate_t", (d, Fs)), ("ws_up_t", (d, Fs)), ("ws_down_t", (Fs, d)))}
    moe.moe_backward_prepare_shared(wsd["ws_gate"], wsd["ws_up"], wsd["ws_down"], wt["ws_gate_t"],
                                    wt["ws_up_t"], wt["ws_down_t"])
    dx = torch.zeros((T, d), dtype=torch.float32, device=cuda)
    dws = {n: torch.empty(shp, dtype=torch.float32, device=cuda)
           for n, shp in (("dws_gate", (Fs, d)), ("dws_up", (Fs, d)), ("dws_down", (d, Fs)))}
    ws = torch.empty(moe.moe_workspace_bytes(7, T, d, 0, 1, 1, 0, Fs), dtype=torch.uint8,
                     device=cuda)
    U.log("[shared bwd full] backward on the GPU")
    moe.moe_shared_backward(xd, torch.from_numpy(g_out).to(cuda), wsd["ws_gate"], wsd["ws_up"],
                            wt["ws_gate_t"], wt["ws_up_t"], wt["ws_down_t"],
                            moe.MOE_ROUND_STOCHASTIC, seed, dx, dws["dws_gate"], dws["dws_up"],
                            dws["dws_down"], ws)
    torch.cuda.synchronize()
    for n, t in list(dws.items()) + [("dx", dx)]:
        assert bool(torch.isfinite(t).all()), n
    rng = np.random.default_rng(11)
    toks = np.sort(rng.choice(T, N_SAMPLE, replace=False))
    frows = np.sort(rng.choice(Fs, N_SAMPLE, replace=False))
    drows = np.sort(rng.choice(d, N_SAMPLE, replace=False))
    dcols = np.sort(rng.choice(d, N_COLS, replace=False))
    fcols = np.sort(rng.choice(Fs, N_COLS, replace=False))
    got = {"dx": dx[torch.from_numpy(toks).to(cuda)].cpu().numpy(),
           "dws_gate": dws["dws_gate"].cpu().numpy()[np.ix_(frows, dcols)],
           "dws_up": dws["dws_up"].cpu().numpy()[np.ix_(frows, dcols)],
           "dws_down": dws["dws_down"].cpu().numpy()[np.ix_(drows, fcols)]}
    del dx, dws, wt, wsd, xd, ws
    torch.cuda.empty_cache()

    U.log("[shared bwd full] oracle: host inputs and the stochastic cast of g_out")
    x = gen.host_tensor_f64(cfg, "x")
    wsg, wsu, wsdn = (gen.host_tensor_f64(cfg, n) for n in ("ws_gate", "ws_up", "ws_down"))
    go = OB.round_bf16_sr(g_out.astype(np.float64), seed, 1)          # [T, d], stream 1
    # sampled tokens: the oracle's shared-expert backward on those rows (its
    # casts of dgs, dus use each element's index t * Fs + f in the [T, Fs]
    # tensor, so the rows are cast as in the full tensor)
    gs = x[toks] @ wsg.T
    us = x[toks] @ wsu.T
    dhs = go[toks] @ wsdn
    fidx = toks[:, None].astype(np.int64) * Fs + np.arange(Fs)[None, :]
    dgs_b = OB.round_bf16_sr(dhs * us * OB.silu_grad(gs), seed, 9, index=fidx)
    dus_b = OB.round_bf16_sr(dhs * oracle.silu(gs), seed, 10, index=fidx)
    check("shared bwd full dx (sampled tokens)", got["dx"], dgs_b @ wsg + dus_b @ wsu)
    # dWs_gate, dWs_up rows frows over all tokens: the gradients' columns f
    gs_c = x @ wsg[frows].T                                          # [T, n]
    us_c = x @ wsu[frows].T
    dhs_c = go @ wsdn[:, frows]
    cidx = np.arange(T, dtype=np.int64)[:, None] * Fs + frows[None, :]
    dgs_c = OB.round_bf16_sr(dhs_c * us_c * OB.silu_grad(gs_c), seed, 9, index=cidx)
    dus_c = OB.round_bf16_sr(dhs_c * oracle.silu(gs_c), seed, 10, index=cidx)
    check("shared bwd full dWs_gate block", got["dws_gate"], dgs_c.T @ x[:, dcols])
    check("shared bwd full dWs_up block", got["dws_up"], dus_c.T @ x[:, dcols])
    # dWs_down rows drows, columns fcols: g^T hs over all tokens
    hs_c = oracle.round_bf16(oracle.silu(x @ wsg[fcols].T) * (x @ wsu[fcols].T))
    check("shared bwd full dWs_down block", got["dws_down"], go[:, drows].T @ hs_c)
