"""GPU parity of the backward pass (moe_backward, moe_grad_cast_bf16) against
the CPU oracle's backward (oracle/latent_moe_backward.py).

The GPU runs the forward (keeping the router logits), then the backward for a
seeded output gradient.  The oracle replays the GPU's routing (so near-tie
swaps cannot make the two sides differentiate different selections) in its
bf16_operands mode with the same gradient rounding (nearest or stochastic,
same seed): the rounding points and the random streams are the same on both
sides.  Rules: the stochastic-rounding cast is bit-exact against the
oracle's on identical fp32 inputs.  Gradients: both sides feed the same bf16
operands, the GPU accumulates in fp32 and the oracle in float64, so the two
differ where an operand lies within that accumulation error of a bf16
rounding boundary (nearest or stochastic) and the two sides round it to
neighbouring bf16 values: a rare 2^-8-relative change of one term of a sum.
The rule: RMS(gpu - oracle) / RMS(oracle) <= 1e-3 for every gradient (a
systematic error -- a dropped term, a wrong sign, a transposed operand or a
wrong row -- moves it to O(1)) and max |gpu - oracle| / RMS(oracle) <= 5e-2
(a single flipped operand of a short sum; measured <= 2.3e-2, while bf16
rounding itself moves the gradients by 1.5e-2 - 2.8e-1 of their RMS against
the exact oracle).  Repeated runs are bitwise identical.
"""
import numpy as np
import pytest
import torch

import mixture_experts_layer_moe_amd as moe
import oracle
from moe_synth import CONFIGS, MoEConfig, device, gen
from oracle import latent_moe_backward as OB
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

GRAD_TOL_MAX = 5e-2
GRAD_TOL_RMS = 1e-3

CASES = {
    "tiny": CONFIGS["tiny"],
    # T, L and F tails inside a tile; T not a multiple of 64 (padded K of the
    # dense weight gradients)
    "ragged": MoEConfig("ragged", T=300, d=320, L=192, E=24, k=3, F=320, seed=3),
    # several M tiles per expert (256-row tiles) and long per-expert K ranges
    "deep": MoEConfig("deep", T=2048, d=256, L=256, E=8, k=2, F=512, seed=9),
    # router bias in the logits (its gradient), hot experts and empty experts
    # (zero weight gradients from an empty K range)
    "zipf": MoEConfig("zipf", T=1024, d=256, L=128, E=64, k=4, F=256, zipf_bias=True, seed=11),
    # degenerate cases of the method: one expert (a dense latent SwiGLU FFN,
    # gate weight 1), every expert selected (k = E: a dense soft mixture), a
    # single token
    "single": MoEConfig("single", T=100, d=128, L=64, E=1, k=1, F=128, seed=15),
    "dense": MoEConfig("dense", T=64, d=128, L=64, E=8, k=8, F=128, seed=17),
    "one_token": MoEConfig("one_token", T=1, d=256, L=128, E=16, k=2, F=256, seed=19),
    # Base-1 hidden and latent widths: the dense weight gradients dW_up [d, L]
    # and dW_dn [L, d] then take the 256 x 192 tiles
    "wide": MoEConfig("wide", T=64, d=6656, L=3072, E=8, k=2, F=256, seed=21),
}


@pytest.fixture(scope="module")
def cuda():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.load()
    return torch.device("cuda:0")


_cache = {}


def setup_case(name, dev):
    if name in _cache:
        return _cache[name]
    cfg = CASES[name]
    U.log(f"[backward case {name}] {cfg}")
    host = gen.host_inputs_f64(cfg)
    dv = device.device_inputs(cfg, dev)
    g_out = np.random.default_rng(1000 + cfg.seed).standard_normal((cfg.T, cfg.d)).astype(np.float32)
    torch.cuda.synchronize()
    _cache[name] = (cfg, host, dv, g_out)
    return _cache[name]


def weights_of(dv):
    return moe.LatentMoEWeights(dv["w_router"], dv["b_router"], dv["w_dn"], dv["w_gate"],
                                dv["w_up"], dv["w_down"], dv["w_lat_up"])


def run_gpu(cfg, dv, g_out, dev, rounding, seed):
    w = weights_of(dv)
    buf = moe.LatentMoEBuffers(cfg.T, cfg.d, cfg.L, cfg.E, cfg.k, cfg.F, device=dev,
                               keep_logits=True)
    moe.forward(dv["x"], w, cfg.k, buf)
    wt = moe.backward_prepare(w)
    grads = moe.LatentMoEGrads(cfg.T, cfg.d, cfg.L, cfg.E, cfg.k, cfg.F, device=dev,
                               bias=dv["b_router"] is not None)
    go = torch.from_numpy(g_out).to(dev)
    moe.backward(dv["x"], w, wt, buf, go, grads, rounding=rounding, seed=seed)
    torch.cuda.synchronize()
    return buf, wt, grads


GRADS = [("dx", "dx"), ("dw_router", "dW_router"), ("dw_lat_down", "dW_dn"),
         ("dw_gate", "dW_gate"), ("dw_up", "dW_up"), ("dw_down", "dW_down"),
         ("dw_lat_up", "dW_lat_up"), ("dtopk_w", "dtopk_w")]


@pytest.mark.parametrize("rounding", ["rne", "sr"])
@pytest.mark.parametrize("name", list(CASES))
def test_backward_matches_oracle(cuda, name, rounding):
    cfg, host, dv, g_out = setup_case(name, cuda)
    seed = 12345
    rmode = moe.MOE_ROUND_STOCHASTIC if rounding == "sr" else moe.MOE_ROUND_NEAREST
    U.log(f"[{name}/{rounding}] gpu forward + backward")
    buf, wt, grads = run_gpu(cfg, dv, g_out, cuda, rmode, seed)
    gidx = U.to_np(buf.topk_idx)
    gw = U.to_np(buf.topk_w).astype(np.float64)
    U.log(f"[{name}/{rounding}] oracle backward")
    ref = oracle.backward(host["x"], host["w_router"], host["b_router"], cfg.k, host["w_dn"],
                          U.experts_of(host), host["w_lat_up"], g_out.astype(np.float64),
                          mode="bf16_operands", rounding=rounding, seed=seed,
                          routing=(gidx, gw))
    # the transposed weights are exact copies
    np.testing.assert_array_equal(U.to_np(wt.w_gate_t), np.transpose(host["w_gate"], (0, 2, 1)))
    np.testing.assert_array_equal(U.to_np(wt.w_down_t), np.transpose(host["w_down"], (0, 2, 1)))
    np.testing.assert_array_equal(U.to_np(wt.w_lat_up_t), host["w_lat_up"].T)
    errs = {}
    for gname, oname in GRADS:
        got = U.to_np(getattr(grads, gname))
        want = np.asarray(ref[oname])
        if not np.any(want):
            # an exactly zero gradient (one expert: the softmax has no
            # freedom, so the router gets none) must come out exactly zero
            assert not np.any(got), gname
            continue
        errs[gname] = U.rel_err(got, want)
    if grads.db_router is not None and np.any(ref["db_router"]):
        errs["db_router"] = U.rel_err(U.to_np(grads.db_router), ref["db_router"])
    U.log(f"[{name}/{rounding}] max|err|/RMS: " +
          ", ".join(f"{k} {v[0]:.2e}" for k, v in errs.items()))
    for gname, (emax, erms) in errs.items():
        assert emax <= GRAD_TOL_MAX, (gname, emax)
        assert erms <= GRAD_TOL_RMS, (gname, erms)
    # experts that received no rows have exactly zero weight gradients
    counts = np.bincount(gidx.ravel(), minlength=cfg.E)
    for e in np.nonzero(counts == 0)[0]:
        assert not np.any(U.to_np(grads.dw_down[e]))
        assert not np.any(U.to_np(grads.dw_gate[e]))


def test_backward_bitwise_determinism(cuda):
    cfg, host, dv, g_out = setup_case("zipf", cuda)
    runs = []
    for _ in range(2):
        _, _, g = run_gpu(cfg, dv, g_out, cuda, moe.MOE_ROUND_STOCHASTIC, 7)
        runs.append([g.dx.cpu(), g.dw_gate.cpu(), g.dw_down.cpu(), g.dw_router.cpu(),
                     g.db_router.cpu()])
    for a, b in zip(*runs):
        assert torch.equal(a, b)


@pytest.mark.parametrize("stream_id,seed", [(1, 0), (2, 12345), (5, 0xFFFFFFFF)])
def test_grad_cast_bit_exact(cuda, stream_id, seed):
    rng = np.random.default_rng(stream_id)
    n = (1 << 20) + 64
    v = (rng.standard_normal(n) * np.exp2(rng.integers(-30, 30, n))).astype(np.float32)
    src = torch.from_numpy(v).to(cuda)
    dst = torch.empty(n, dtype=torch.bfloat16, device=cuda)
    moe.moe_grad_cast_bf16(src, moe.MOE_ROUND_STOCHASTIC, seed, stream_id, dst)
    torch.cuda.synchronize()
    got = dst.view(torch.int16).cpu().numpy().view(np.uint16)
    want = OB.bf16_bits(OB.round_bf16_sr(v, seed, stream_id))
    np.testing.assert_array_equal(got, want)
    moe.moe_grad_cast_bf16(src, moe.MOE_ROUND_NEAREST, seed, stream_id, dst)
    torch.cuda.synchronize()
    got = dst.view(torch.int16).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(got, OB.bf16_bits(oracle.round_bf16(v.astype(np.float64))))


def test_backward_selection_bias_mode(cuda):
    """Loss-free-balancer bias (selection only): the weights are the softmax of
    the unbiased logits, the bias gets no gradient."""
    cfg, host, dv, g_out = setup_case("zipf", cuda)
    w = weights_of(dv)
    buf = moe.LatentMoEBuffers(cfg.T, cfg.d, cfg.L, cfg.E, cfg.k, cfg.F, device=cuda,
                               keep_logits=True)
    moe.moe_route_ex(dv["x"], dv["w_router"], dv["b_router"], moe.MOE_BIAS_SELECTION, cfg.k,
                     buf.topk_idx, buf.topk_w, logits_out=buf.logits, ws=buf.ws)
    moe.forward(dv["x"], w, cfg.k, buf, route=False)
    wt = moe.backward_prepare(w)
    grads = moe.LatentMoEGrads(cfg.T, cfg.d, cfg.L, cfg.E, cfg.k, cfg.F, device=cuda)
    moe.backward(dv["x"], w, wt, buf, torch.from_numpy(g_out).to(cuda), grads,
                 rounding=moe.MOE_ROUND_STOCHASTIC, seed=3, bias_mode=moe.MOE_BIAS_SELECTION)
    torch.cuda.synchronize()
    gidx = U.to_np(buf.topk_idx)
    ref = oracle.backward(host["x"], host["w_router"], host["b_router"], cfg.k, host["w_dn"],
                          U.experts_of(host), host["w_lat_up"], g_out.astype(np.float64),
                          mode="bf16_operands", rounding="sr", seed=3,
                          routing=(gidx, U.to_np(buf.topk_w).astype(np.float64)),
                          bias_mode="selection")
    assert not np.any(U.to_np(grads.db_router))
    for gname, oname in GRADS:
        emax, erms = U.rel_err(U.to_np(getattr(grads, gname)), np.asarray(ref[oname]))
        U.log(f"[zipf/selection] {gname}: max {emax:.2e} rms {erms:.2e}")
        assert emax <= GRAD_TOL_MAX and erms <= GRAD_TOL_RMS, (gname, emax, erms)
