"""GPU parity of the backward pass with FP8 data gradients (moe_backward_fp8,
moe_grad_cast_e5m2) against the oracle's backward with grad_fp8
(oracle/latent_moe_backward.py).

* The E5M2 gradient cast: bit-exact (decoded values, +0 == -0) against the
  oracle's nearest and stochastic E5M2 rounding on fp32 inputs that include
  exact ties between E5M2 values, subnormals, the saturation point and zeros.
* The backward on the oracle's routing (fed to the GPU, as in the forward FP8
  test), with every scale computed on the oracle side: the weight scales 448 /
  amax of each expert matrix (the GPU's must equal them bit for bit), the
  gradient scales 448 / amax of the oracle's own bf16-mode dy, dg, du.
  Gradients that no FP8 GEMM feeds (dW_up, dW_down, the gate weights, the
  router) keep the bf16 backward's rule: RMS(err)/RMS <= 1e-3, max <= 5e-2.
  Gradients downstream of the FP8 GEMMs (dW_gate and dW_up through dh; dx and
  dW_dn through dz): the two sides round the same E5M2 operands at the same
  points and differ where an fp32 (GPU) and a float64 (oracle) value fall on
  different sides of an E5M2 rounding boundary.  Such a flip has probability
  ~|delta| / q and size q (q the rounding step, delta the difference of the
  two unrounded values), so the error it adds scales as sqrt(q): E5M2's step
  is 2^-2 relative against bf16's 2^-8, 8x the bf16 rule's RMS bound:
  RMS(err)/RMS <= 8e-3.  One flipped operand moves a sum of K terms by one
  step of one term; the max rule is 1.5e-1 of RMS.  A wrong scale, format,
  stream or operand moves the RMS ratio to >= 5e-2 (E5M2's own quantization
  noise) or O(1).
* The step's maxima: max |dy| within 2^-8 relative of the oracle's (fp32 vs
  float64 products), max |dg| and max |du| within 2^-4 (they come from dh,
  which the E5M2 flips move).
* Two steps with the same scales are bitwise identical; the delayed-scaling
  history records each step's maxima and the next scale is 448 / its max.
"""
import numpy as np
import pytest
import torch

import mixture_experts_layer_moe_amd as moe
import oracle
from moe_synth import MoEConfig, device, gen
from oracle import latent_moe_backward as OB
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

TOL_BF16_RMS, TOL_BF16_MAX = 1e-3, 5e-2
TOL_FP8_RMS, TOL_FP8_MAX = 8e-3, 1.5e-1

CASES = {
    "tiny": MoEConfig("tiny8b", T=256, d=512, L=256, E=16, k=2, F=512, seed=41),
    # ragged T and E; F a multiple of 128 but not of the 256-wide tiles
    "ragged": MoEConfig("ragged8b", T=300, d=320, L=256, E=24, k=3, F=384, seed=43),
    # several M tiles per expert (256-row tiles)
    "deep": MoEConfig("deep8b", T=2048, d=256, L=256, E=8, k=2, F=512, seed=45),
    # hot and empty experts
    "zipf": MoEConfig("zipf8b", T=1024, d=256, L=128, E=64, k=4, F=256, zipf_bias=True, seed=47),
    # one expert (dense latent SwiGLU FFN), every expert selected, one token
    "single": MoEConfig("single8b", T=100, d=128, L=128, E=1, k=1, F=128, seed=49),
    "dense": MoEConfig("dense8b", T=64, d=128, L=128, E=8, k=8, F=128, seed=51),
    "one_token": MoEConfig("one8b", T=1, d=256, L=128, E=16, k=2, F=256, seed=53),
}

# gradients no FP8 GEMM feeds, and those downstream of one
GRADS_BF16 = [("dw_router", "dW_router"), ("dw_down", "dW_down"), ("dw_lat_up", "dW_lat_up"),
              ("dtopk_w", "dtopk_w")]
GRADS_FP8 = [("dx", "dx"), ("dw_lat_down", "dW_dn"), ("dw_gate", "dW_gate"), ("dw_up", "dW_up")]


@pytest.fixture(scope="module")
def cuda():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.load()
    return torch.device("cuda:0")


def _e5m2_decode(b):
    b = np.asarray(b, np.int64)
    s = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 2) & 31
    m = b & 3
    assert not np.any(e == 31), "inf or NaN code"
    v = np.where(e == 0, m * 2.0 ** -16, (1.0 + m / 4.0) * np.exp2(e - 15.0))
    return s * v


def _e5m2_values():
    """All finite non-negative E5M2 values, ascending."""
    return _e5m2_decode(np.arange(0x7C))


@pytest.mark.parametrize("stream_id,seed", [(6, 0), (7, 12345), (8, 0xFFFFFFFF)])
def test_e5m2_cast_bit_exact(cuda, stream_id, seed):
    rng = np.random.default_rng(100 + stream_id)
    n = (1 << 20) + 64
    v = (rng.standard_normal(n) * np.exp2(rng.integers(-40, 18, n))).astype(np.float32)
    tab = _e5m2_values()
    mids = (tab[:-1] + tab[1:]) / 2            # exact ties at scale 1/128 (all fp32-exact)
    v[:mids.size] = (mids / 128.0).astype(np.float32)
    v[mids.size:2 * mids.size] = -(mids / 128.0).astype(np.float32)
    v[2 * mids.size:2 * mids.size + 6] = [0.0, -0.0, 448.0, 449.0, -1e9, 3e-9]
    src = torch.from_numpy(v).to(cuda)
    dst = torch.empty(n, dtype=torch.uint8, device=cuda)
    for scale_v in (1.0, 0.37):
        scale = torch.tensor([scale_v], dtype=torch.float32, device=cuda)
        x32 = v * np.float32(128.0 * np.float32(scale_v))
        for rounding, want in ((moe.MOE_ROUND_NEAREST, OB.round_e5m2(x32.astype(np.float64))),
                               (moe.MOE_ROUND_STOCHASTIC, OB.round_e5m2_sr(x32, seed, stream_id))):
            moe.moe_grad_cast_e5m2(src, scale, rounding, seed, stream_id, dst)
            torch.cuda.synchronize()
            got = _e5m2_decode(dst.cpu().numpy())
            bad = np.nonzero(got != want)[0]
            U.log(f"[e5m2 cast stream {stream_id} scale {scale_v} rounding {rounding}] "
                  f"{bad.size} of {n} differ")
            assert bad.size == 0, [(float(x32[i]), got[i], want[i]) for i in bad[:6]]


_cache = {}


def _setup(name, dev):
    if name in _cache:
        return _cache[name]
    cfg = CASES[name]
    U.log(f"[fp8 backward case {name}] {cfg}")
    host = gen.host_inputs_f64(cfg)
    dv = device.device_inputs(cfg, dev)
    g_out = np.random.default_rng(2000 + cfg.seed).standard_normal((cfg.T, cfg.d)).astype(np.float32)
    ro = oracle.route(host["x"], host["w_router"], host["b_router"], cfg.k)
    routing = (ro["topk_idx"], np.asarray(ro["topk_w"], np.float32).astype(np.float64))
    # weight scales: 448 / amax of each expert matrix (float32)
    w_scale = []
    for n in ("w_gate", "w_up", "w_down"):
        am = np.abs(host[n]).reshape(cfg.E, -1).max(axis=1).astype(np.float32)
        w_scale.append(np.float32(448.0) / am)
    # gradient scales from the oracle's own bf16-mode gradients
    rb = OB.backward(host["x"], host["w_router"], host["b_router"], cfg.k, host["w_dn"],
                     U.experts_of(host), host["w_lat_up"], g_out.astype(np.float64),
                     mode="bf16_operands", rounding="rne", routing=routing)
    gmax = [float(np.abs(rb[n]).max()) for n in ("dy_b", "dg_b", "du_b")]
    g_scale = tuple(np.float32(448.0) / np.float32(m) for m in gmax)
    torch.cuda.synchronize()
    _cache[name] = (cfg, host, dv, g_out, routing, w_scale, g_scale)
    return _cache[name]


def _run_gpu(cfg, dv, g_out, routing, g_scale, dev, rounding, seed):
    w = moe.LatentMoEWeights(dv["w_router"], dv["b_router"], dv["w_dn"], dv["w_gate"],
                             dv["w_up"], dv["w_down"], dv["w_lat_up"])
    buf = moe.LatentMoEBuffers(cfg.T, cfg.d, cfg.L, cfg.E, cfg.k, cfg.F, device=dev,
                               keep_logits=True)
    # the router's logits for the backward, then the oracle's routing
    moe.moe_route(dv["x"], w.w_router, w.b_router, cfg.k, buf.topk_idx, buf.topk_w,
                  logits_out=buf.logits, ws=buf.ws)
    buf.topk_idx.copy_(torch.from_numpy(np.asarray(routing[0], np.int32)))
    buf.topk_w.copy_(torch.from_numpy(np.asarray(routing[1], np.float32)))
    moe.forward(dv["x"], w, cfg.k, buf, route=False)
    wt = moe.backward_prepare(w)
    w8 = moe.quantize_experts(w)
    wt8 = moe.quantize_transposed(wt, w8)
    grads = moe.LatentMoEGrads(cfg.T, cfg.d, cfg.L, cfg.E, cfg.k, cfg.F, device=dev,
                               bias=dv["b_router"] is not None, fp8=True)
    sc = moe.Fp8GradScaling(hist_len=16, device=dev)
    sc.scale.copy_(torch.tensor(g_scale, dtype=torch.float32))
    moe.backward_fp8(dv["x"], w, wt, wt8, buf, torch.from_numpy(g_out).to(dev), grads, sc,
                     rounding=rounding, seed=seed, update_scaling=False)
    torch.cuda.synchronize()
    return buf, wt8, grads, sc


@pytest.mark.parametrize("rounding", ["rne", "sr"])
@pytest.mark.parametrize("name", list(CASES))
def test_backward_fp8_matches_oracle(cuda, name, rounding):
    cfg, host, dv, g_out, routing, w_scale, g_scale = _setup(name, cuda)
    seed = 777
    rmode = moe.MOE_ROUND_STOCHASTIC if rounding == "sr" else moe.MOE_ROUND_NEAREST
    U.log(f"[fp8 backward {name}/{rounding}] gpu forward + backward")
    buf, wt8, grads, sc = _run_gpu(cfg, dv, g_out, routing, g_scale, cuda, rmode, seed)
    np.testing.assert_array_equal(wt8.w_scale.cpu().numpy(), np.concatenate(w_scale))
    # the E4M3 transposes are the forward's quantized weights, transposed
    np.testing.assert_array_equal(
        _e4m3_bytes_to_f64(wt8.w_down_t8.cpu().numpy()),
        np.transpose(oracle.quantize_e4m3(host["w_down"], w_scale[2][:, None, None]), (0, 2, 1)))
    U.log(f"[fp8 backward {name}/{rounding}] oracle backward")
    ref = OB.backward(host["x"], host["w_router"], host["b_router"], cfg.k, host["w_dn"],
                      U.experts_of(host), host["w_lat_up"], g_out.astype(np.float64),
                      mode="bf16_operands", rounding=rounding, seed=seed, routing=routing,
                      grad_fp8={"grad_scale": g_scale, "w_scale": tuple(w_scale)})
    errs = {}
    for group, rules in ((GRADS_BF16, (TOL_BF16_MAX, TOL_BF16_RMS)),
                         (GRADS_FP8, (TOL_FP8_MAX, TOL_FP8_RMS))):
        for gname, oname in group:
            got = U.to_np(getattr(grads, gname))
            want = np.asarray(ref[oname])
            if not np.any(want):
                assert not np.any(got), gname
                continue
            errs[gname] = (*U.rel_err(got, want), rules)
    if grads.db_router is not None and np.any(ref["db_router"]):
        errs["db_router"] = (*U.rel_err(U.to_np(grads.db_router), ref["db_router"]),
                             (TOL_BF16_MAX, TOL_BF16_RMS))
    am = sc.amax.cpu().numpy().astype(np.float64)
    ram = np.asarray(ref["grad_amax"])
    U.log(f"[fp8 backward {name}/{rounding}] max/rms err: " +
          ", ".join(f"{k} {v[0]:.2e}/{v[1]:.2e}" for k, v in errs.items()) +
          f"; amax dy/dg/du {am} (oracle {ram})")
    for gname, (emax, erms, (tmax, trms)) in errs.items():
        assert emax <= tmax, (gname, emax)
        assert erms <= trms, (gname, erms)
    assert abs(am[0] - ram[0]) <= ram[0] * 2.0 ** -8
    assert np.all(np.abs(am[1:] - ram[1:]) <= ram[1:] * 2.0 ** -4)
    counts = np.bincount(np.asarray(routing[0]).ravel(), minlength=cfg.E)
    for e in np.nonzero(counts == 0)[0]:
        assert not np.any(U.to_np(grads.dw_gate[e]))
        assert not np.any(U.to_np(grads.dw_up[e]))


def _e4m3_bytes_to_f64(b):
    b = np.asarray(b, np.int64)
    s = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 15
    m = b & 7
    v = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    return s * v


def test_backward_fp8_deterministic_and_history(cuda):
    cfg, host, dv, g_out, routing, w_scale, g_scale = _setup("zipf", cuda)
    w = moe.LatentMoEWeights(dv["w_router"], dv["b_router"], dv["w_dn"], dv["w_gate"],
                             dv["w_up"], dv["w_down"], dv["w_lat_up"])
    buf = moe.LatentMoEBuffers(cfg.T, cfg.d, cfg.L, cfg.E, cfg.k, cfg.F, device=cuda,
                               keep_logits=True)
    moe.forward(dv["x"], w, cfg.k, buf)
    wt = moe.backward_prepare(w)
    wt8 = moe.quantize_transposed(wt, moe.quantize_experts(w))
    grads = moe.LatentMoEGrads(cfg.T, cfg.d, cfg.L, cfg.E, cfg.k, cfg.F, device=cuda, fp8=True)
    sc = moe.Fp8GradScaling(hist_len=8, device=cuda)
    go = torch.from_numpy(g_out).to(cuda)
    # the same scales twice: bitwise identical gradients and maxima
    sc.scale.copy_(torch.tensor(g_scale, dtype=torch.float32))
    runs = []
    for _ in range(2):
        moe.backward_fp8(dv["x"], w, wt, wt8, buf, go, grads, sc, seed=5, update_scaling=False)
        torch.cuda.synchronize()
        runs.append([grads.dx.clone(), grads.dw_gate.clone(), grads.dw_lat_down.clone(),
                     sc.amax.clone()])
    for a, b in zip(*runs):
        assert torch.equal(a, b)
    # delayed scaling: three steps record their maxima in the history, and the
    # scale for the next step is 448 / the history's maximum
    sc = moe.Fp8GradScaling(hist_len=8, device=cuda)
    recorded = []
    for _ in range(3):
        moe.backward_fp8(dv["x"], w, wt, wt8, buf, go, grads, sc, seed=5)
        torch.cuda.synchronize()
        recorded.append(sc.amax.cpu().numpy())
    hist = sc.history.cpu().numpy()
    np.testing.assert_array_equal(hist[:, :3], np.stack(recorded, axis=1))
    np.testing.assert_array_equal(hist[:, 3:], 0.0)
    assert np.all(hist[:, :3] > 0)
    np.testing.assert_array_equal(sc.scale.cpu().numpy(), oracle.fp8_scale_from_history(hist))
    U.log(f"[fp8 backward steps] maxima {np.stack(recorded)}; scales {sc.scale.cpu().numpy()}")
