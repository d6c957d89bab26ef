"""Pins of the backward oracle (CPU only).

The backward oracle is checked against things other than itself:
* central finite differences of the forward oracle (itself pinned by
  tests/test_oracle.py) for every parameter and the input, in exact mode, on
  a small layer whose top-k selection has clear gaps (so the perturbation
  never changes which experts are selected);
* invariants: each token's router-logit gradient sums to zero (softmax),
  linearity in the output gradient, the combine gradient's two halves;
* the stochastic rounding's definition: the result is one of the two bf16
  neighbours, bf16 values pass unchanged, the choice is unbiased, and the
  generator is a bijection of the index for a fixed key.
"""
import numpy as np
import pytest

import oracle
from oracle import latent_moe_backward as B

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def small_layer(seed=0, T=5, d=6, L=4, E=4, k=2, Fw=3, bias=True, Fs=0):
    rng = np.random.default_rng(seed)
    p = {
        "x": rng.standard_normal((T, d)),
        "w_router": rng.standard_normal((E, d)) / np.sqrt(d),
        "b_router": 0.3 * rng.standard_normal(E) if bias else None,
        "w_dn": rng.standard_normal((L, d)) / np.sqrt(d),
        "w_gate": rng.standard_normal((E, Fw, L)) / np.sqrt(L),
        "w_up": rng.standard_normal((E, Fw, L)) / np.sqrt(L),
        "w_down": rng.standard_normal((E, L, Fw)) / np.sqrt(Fw),
        "w_lat_up": rng.standard_normal((d, L)) / np.sqrt(L),
        "g_out": rng.standard_normal((T, d)),
    }
    if Fs:
        p["ws_gate"] = rng.standard_normal((Fs, d)) / np.sqrt(d)
        p["ws_up"] = rng.standard_normal((Fs, d)) / np.sqrt(d)
        p["ws_down"] = rng.standard_normal((d, Fs)) / np.sqrt(Fs)
    return p, k


def _shared(p):
    return (p["ws_gate"], p["ws_up"], p["ws_down"]) if "ws_gate" in p else None


def fwd_out(p, k):
    experts = [(p["w_gate"][e], p["w_up"][e], p["w_down"][e]) for e in range(p["w_gate"].shape[0])]
    return oracle.forward(p["x"], p["w_router"], p["b_router"], k, p["w_dn"], experts,
                          p["w_lat_up"], shared=_shared(p), mode="exact")


def bwd(p, k, **kw):
    experts = [(p["w_gate"][e], p["w_up"][e], p["w_down"][e]) for e in range(p["w_gate"].shape[0])]
    return oracle.backward(p["x"], p["w_router"], p["b_router"], k, p["w_dn"], experts,
                           p["w_lat_up"], p["g_out"], shared=_shared(p), **kw)


def loss(p, k):
    return float(np.sum(p["g_out"] * fwd_out(p, k)["out"]))


def selection_gap(p, k):
    lg = np.sort(oracle.router_logits(p["x"], p["w_router"], p["b_router"]), axis=1)[:, ::-1]
    return float(np.min(lg[:, k - 1] - lg[:, k]))


GRAD_OF = {"x": "dx", "w_router": "dW_router", "b_router": "db_router", "w_dn": "dW_dn",
           "w_gate": "dW_gate", "w_up": "dW_up", "w_down": "dW_down", "w_lat_up": "dW_lat_up"}


SHARED_GRAD_OF = {"x": "dx", "ws_gate": "dWs_gate", "ws_up": "dWs_up", "ws_down": "dWs_down",
                  "w_lat_up": "dW_lat_up", "w_dn": "dW_dn"}


@pytest.mark.parametrize("seed,Fs", [(0, 0), (1, 0), (2, 0), (5, 4), (6, 7)])
def test_finite_differences_every_parameter(seed, Fs):
    """Every parameter and x; with Fs > 0 the layer has a shared expert (its
    three weights too, and its part of dx)."""
    p, k = small_layer(seed, Fs=Fs)
    assert selection_gap(p, k) > 1e-3      # the perturbation below never changes selection
    g = bwd(p, k, mode="exact")
    eps = 1e-6
    names = dict(GRAD_OF, **SHARED_GRAD_OF) if Fs else GRAD_OF
    for name, gname in names.items():
        base = p[name]
        num = np.zeros_like(base)
        for i in np.ndindex(base.shape):
            old = base[i]
            base[i] = old + eps
            lp = loss(p, k)
            base[i] = old - eps
            lm = loss(p, k)
            base[i] = old
            num[i] = (lp - lm) / (2 * eps)
        ana = np.asarray(g[gname])
        scale = max(np.max(np.abs(num)), 1e-3)
        assert np.max(np.abs(ana - num)) / scale < 1e-6, (name, np.max(np.abs(ana - num)), scale)


def test_finite_differences_gate_weights():
    """dtopk_w is the gradient w.r.t. the combine weights with the selection
    fixed: perturb w through forward with replayed routing."""
    p, k = small_layer(3)
    g = bwd(p, k, mode="exact")
    fwd = fwd_out(p, k)
    experts = [(p["w_gate"][e], p["w_up"][e], p["w_down"][e]) for e in range(4)]
    idx, w = fwd["topk_idx"], fwd["topk_w"].copy()
    eps = 1e-6

    def lossw(wv):
        o = oracle.forward(p["x"], p["w_router"], p["b_router"], k, p["w_dn"], experts,
                           p["w_lat_up"], mode="exact", routing=(idx, wv))["out"]
        return float(np.sum(p["g_out"] * o))
    num = np.zeros_like(w)
    for i in np.ndindex(w.shape):
        wp = w.copy(); wp[i] += eps
        wm = w.copy(); wm[i] -= eps
        num[i] = (lossw(wp) - lossw(wm)) / (2 * eps)
    assert np.max(np.abs(g["dtopk_w"] - num)) < 1e-7 * max(1.0, np.max(np.abs(num)))


def test_selection_only_bias_gets_no_gradient():
    p, k = small_layer(4)
    g = bwd(p, k, mode="exact", bias_mode="selection")
    assert np.all(g["db_router"] == 0)
    # the weights are the softmax of the unbiased logits: finite differences
    # of W_r through that mode's forward
    experts = [(p["w_gate"][e], p["w_up"][e], p["w_down"][e]) for e in range(4)]

    def lossr(wr):
        r = oracle.route(p["x"], wr, p["b_router"], k, bias_mode="selection")
        o = oracle.forward(p["x"], wr, p["b_router"], k, p["w_dn"], experts, p["w_lat_up"],
                           mode="exact", routing=(r["topk_idx"], r["topk_w"]))["out"]
        return float(np.sum(p["g_out"] * o))
    wr = p["w_router"]
    i = (1, 2)
    eps = 1e-6
    wp = wr.copy(); wp[i] += eps
    wm = wr.copy(); wm[i] -= eps
    num = (lossr(wp) - lossr(wm)) / (2 * eps)
    assert abs(g["dW_router"][i] - num) < 1e-7 * max(1.0, abs(num))


def test_logit_gradient_rows_sum_to_zero():
    p, k = small_layer(5, T=9)
    g = bwd(p, k, mode="exact")
    assert np.max(np.abs(g["dlogits"].sum(axis=1))) < 1e-12


def test_linear_in_output_gradient():
    p, k = small_layer(6)
    g1 = bwd(p, k, mode="exact")
    p2 = dict(p)
    p2["g_out"] = -2.5 * p["g_out"]
    g2 = bwd(p2, k, mode="exact")
    for name in GRAD_OF.values():
        np.testing.assert_allclose(g2[name], -2.5 * np.asarray(g1[name]), rtol=1e-12, atol=1e-14)


def test_combine_backward_by_hand():
    # two tokens, k = 2: c_0 = 0.25 y_1 + 0.5 y_0, c_1 = 1.0 y_2 + 0.75 y_3
    y = np.array([[1.0, 2.0], [3.0, -1.0], [0.5, 0.5], [-2.0, 4.0]])
    w = np.array([[0.25, 0.5], [1.0, 0.75]])
    ar = np.array([[1, 0], [2, 3]])
    dc = np.array([[2.0, -1.0], [1.0, 3.0]])
    dy, dw = B.combine_backward(dc, y, w, ar)
    np.testing.assert_array_equal(dy, [[1.0, -0.5], [0.5, -0.25], [1.0, 3.0], [0.75, 2.25]])
    np.testing.assert_array_equal(dw, [[2 * 3 - 1 * -1, 2 * 1 - 1 * 2], [0.5 + 1.5, -2 + 12]])


def test_silu_grad_matches_difference_quotient():
    v = np.linspace(-8, 8, 101)
    h = 1e-6
    num = (oracle.silu(v + h) - oracle.silu(v - h)) / (2 * h)
    assert np.max(np.abs(B.silu_grad(v) - num)) < 1e-8
    assert B.silu_grad(np.array([0.0]))[0] == 0.5


def test_bf16_mode_close_to_exact():
    p, k = small_layer(7, T=12, d=16, L=8, E=4, k=2, Fw=8)
    ge = bwd(p, k, mode="exact")
    for rounding in ("rne", "sr"):
        gb = bwd(p, k, mode="bf16_operands", rounding=rounding, seed=11)
        for name in ("dx", "dW_dn", "dW_gate", "dW_down", "dW_lat_up"):
            a, b = np.asarray(ge[name]), np.asarray(gb[name])
            assert np.max(np.abs(a - b)) / np.sqrt(np.mean(a ** 2)) < 0.1, (rounding, name)


# ---------------------------------------------------------------------------
# stochastic rounding and its generator
# ---------------------------------------------------------------------------

def _bf16_neighbours(v):
    v32 = np.asarray(v, np.float32)
    u = v32.view(np.uint32)
    lo = (u & np.uint32(0xFFFF0000)).view(np.float32).astype(np.float64)
    hi = ((u & np.uint32(0xFFFF0000)) + np.uint32(0x10000)).view(np.float32).astype(np.float64)
    return lo, hi


def test_sr_picks_a_neighbour_and_keeps_bf16_values():
    rng = np.random.default_rng(0)
    v = (rng.standard_normal(4096) * np.exp2(rng.integers(-20, 20, 4096))).astype(np.float32)
    r = B.round_bf16_sr(v, seed=3, stream=2)
    lo, hi = _bf16_neighbours(v)       # truncation and one bf16 step up in magnitude
    assert np.all((r == lo) | (r == hi))
    exact = oracle.round_bf16(v.astype(np.float64))
    np.testing.assert_array_equal(B.round_bf16_sr(exact, seed=9, stream=1), exact)


def test_sr_is_unbiased():
    # 1 + 0.3 ulp(bf16): rounds up with probability 0.3
    v = np.full(200000, 1.0 + 0.3 * 2.0 ** -7, np.float32)
    r = B.round_bf16_sr(v, seed=1, stream=5)
    frac_up = np.mean(r > 1.0)
    assert abs(frac_up - 0.3) < 4 * np.sqrt(0.3 * 0.7 / v.size)
    assert abs(np.mean(r) - float(v[0])) < 1e-4 * 2 ** -7 * 50


def test_sr_depends_on_seed_stream_and_index_only():
    v = np.full(1000, 1.0 + 0.5 * 2.0 ** -7, np.float32)
    a = B.round_bf16_sr(v, 5, 2)
    np.testing.assert_array_equal(a, B.round_bf16_sr(v, 5, 2))
    assert np.any(a != B.round_bf16_sr(v, 6, 2))
    assert np.any(a != B.round_bf16_sr(v, 5, 3))


def test_lowbias32_is_a_bijection_by_its_inverse():
    """Each step of the mixer is invertible (xorshift, odd multiplier); undo
    them in reverse order and recover the input."""
    x = np.arange(0, 1 << 20, 7, dtype=np.uint64) * np.uint64(2654435761) & np.uint64(0xFFFFFFFF)
    y = B.lowbias32(x).astype(np.uint64)
    m32 = np.uint64(0xFFFFFFFF)

    def unxs(v, s):
        r = v.copy()
        for _ in range(32 // s + 1):
            r = v ^ (r >> np.uint64(s))
        return r & m32
    inv1 = np.uint64(pow(0x7FEB352D, -1, 1 << 32))
    inv2 = np.uint64(pow(0x846CA68B, -1, 1 << 32))
    v = unxs(y, 16)
    v = (v * inv2) & m32
    v = unxs(v, 15)
    v = (v * inv1) & m32
    v = unxs(v, 16)
    np.testing.assert_array_equal(v, x)
    # and the published mixer's first values are well spread
    assert len(np.unique(B.lowbias32(np.arange(1 << 16)))) == 1 << 16


# ---------------------------------------------------------------------------
# FP8 E5M2 data gradients
# ---------------------------------------------------------------------------

def _e5m2_values():
    """Every finite non-negative E5M2 value, from the code layout (sign,
    5 exponent bits with bias 15, 2 fraction bits; exponent field 31 is
    inf/NaN): subnormals m 2^-16, normals (1 + m/4) 2^(e - 15)."""
    vals = [m * 2.0 ** -16 for m in range(4)]
    for e in range(1, 31):
        vals += [(1 + m / 4) * 2.0 ** (e - 15) for m in range(4)]
    return np.array(vals)


def test_e5m2_grid_closed_form():
    v = _e5m2_values()
    assert v.max() == 57344.0 and v[1] == 2.0 ** -16 and v[4] == 2.0 ** -14
    assert np.array_equal(B.round_e5m2(v), v)
    assert np.array_equal(B.round_e5m2(-v), -v)


def test_e5m2_rne_midpoints_and_saturation():
    v = _e5m2_values()
    mid = (v[:-1] + v[1:]) / 2
    got = B.round_e5m2(mid)
    # ties go to the neighbour with an even fraction field
    lo_even = (np.arange(v.size - 1) % 2) == 0
    assert np.array_equal(got, np.where(lo_even, v[:-1], v[1:]))
    assert np.array_equal(B.round_e5m2(mid * (1 + 1e-9)), v[1:])
    assert np.array_equal(B.round_e5m2(mid * (1 - 1e-9)), v[:-1])
    assert np.array_equal(B.round_e5m2([1e9, -7e4, 61440.0]), [57344.0, -57344.0, 57344.0])


def _e5m2_neighbours(x):
    v = _e5m2_values()
    a = np.minimum(np.abs(x), 57344.0)
    i = np.searchsorted(v, a, side="right") - 1
    lo = v[i]
    hi = v[np.minimum(i + 1, v.size - 1)]
    return np.copysign(lo, x), np.copysign(hi, x)


def test_e5m2_sr_picks_a_neighbour_and_keeps_exact_values():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal(20000) * np.exp2(rng.integers(-13, 15, 20000))).astype(np.float32)
    got = B.round_e5m2_sr(x, seed=3, stream=6)
    lo, hi = _e5m2_neighbours(x.astype(np.float64))
    assert np.all((got == lo) | (got == hi))
    v = np.concatenate([_e5m2_values(), -_e5m2_values()]).astype(np.float32)
    assert np.array_equal(B.round_e5m2_sr(v, seed=9, stream=7), v.astype(np.float64))
    # below 2^-14: nearest even; above 57344: saturated
    tiny = np.array([3e-5, 1.3e-5, -4.2e-5], np.float32)
    assert np.array_equal(B.round_e5m2_sr(tiny, 1, 8), B.round_e5m2(tiny.astype(np.float64)))
    assert np.array_equal(B.round_e5m2_sr(np.array([9e4, -1e30], np.float32), 1, 6),
                          [57344.0, -57344.0])


def test_e5m2_sr_is_unbiased():
    # 1.1 lies between 1 and 1.25: rounds up with probability 0.4
    n = 200000
    x = np.full(n, 1.1, np.float32)
    up = (B.round_e5m2_sr(x, seed=5, stream=7) == 1.25).mean()
    p = (float(np.float32(1.1)) - 1.0) / 0.25
    assert abs(up - p) < 5 * np.sqrt(p * (1 - p) / n)


def test_grad_quantizer_scales_in_float32():
    v = np.array([0.001, -0.02, 3.5e-3])
    s = np.float32(448.0 / 0.03)
    q = B.quantize_grad_e5m2(v, s, "rne", 0, "dy")
    x32 = v.astype(np.float32) * (np.float32(128.0) * s)
    assert np.array_equal(q, B.round_e5m2(x32.astype(np.float64)))


def _fp8_args(p, gscale=(1.0, 1.0, 1.0)):
    E = p["w_gate"].shape[0]
    ws = [np.float32(448.0) / np.abs(p[n].reshape(E, -1)).max(axis=1).astype(np.float32)
          for n in ("w_gate", "w_up", "w_down")]
    return {"grad_scale": gscale, "w_scale": ws}


def _amax_scales(p, k):
    """Scales 224 / max of the step's own dy, dg, du (one binade of headroom:
    the FP8 run's dg, du differ from those of the run that measured them)."""
    r = bwd(p, k, mode="bf16_operands", rounding="rne", grad_fp8=_fp8_args(p))
    return tuple(np.float32(224.0) / np.float32(m) for m in r["grad_amax"])


def test_fp8_grad_mode_with_identity_quantizers_equals_bf16_mode(monkeypatch):
    """The FP8 data-gradient path divides its scales back out and pairs the
    operands like the bf16 path: with both quantizers replaced by exact
    scaling, it reproduces bf16_operands mode."""
    p, k = small_layer(seed=3)
    ref = bwd(p, k, mode="bf16_operands", rounding="sr", seed=2)
    # the bf16 path's operand (same stochastic rounding), scaled exactly
    monkeypatch.setattr(B, "quantize_grad_e5m2",
                        lambda v, s, r, seed, name, index=None:
                        B.round_bf16_sr(v, seed, B.SR_STREAM[name])
                        * float(np.float32(128.0) * np.float32(s)))
    monkeypatch.setattr(B.F, "quantize_e4m3",
                        lambda v, s: np.asarray(v, np.float64) * float(np.float32(s)))
    got = bwd(p, k, mode="bf16_operands", rounding="sr", seed=2,
              grad_fp8=_fp8_args(p, (0.75, 3.0, 40.0)))
    for n in ("dx", "dW_dn", "dW_gate", "dW_up", "dW_down", "dzp", "dh"):
        np.testing.assert_allclose(got[n], ref[n], rtol=1e-12, atol=1e-14, err_msg=n)


def test_fp8_grad_mode_invariant_to_power_of_two_scales():
    """Scaling a gradient tensor's scale by 2^j shifts its E5M2 exponents and
    nothing else (no value reaches saturation or the subnormal range here):
    the dequantized GEMMs, hence every gradient, are unchanged."""
    p, k = small_layer(seed=5)
    s = _amax_scales(p, k)
    a = bwd(p, k, mode="bf16_operands", rounding="sr", seed=4, grad_fp8=_fp8_args(p, s))
    s2 = (s[0] * np.float32(0.25), s[1] * np.float32(0.5), s[2] * np.float32(0.125))
    b = bwd(p, k, mode="bf16_operands", rounding="sr", seed=4, grad_fp8=_fp8_args(p, s2))
    for n in ("dx", "dW_dn", "dW_gate", "dW_up", "dW_down", "dzp", "dh"):
        np.testing.assert_allclose(a[n], b[n], rtol=1e-13, atol=1e-15, err_msg=n)


def test_fp8_grad_mode_close_to_bf16_mode_and_reports_maxima():
    p, k = small_layer(seed=6, T=40, d=16, L=24, E=4, k=2, Fw=32)
    s = _amax_scales(p, k)
    ref = bwd(p, k, mode="bf16_operands", rounding="rne")
    got = bwd(p, k, mode="bf16_operands", rounding="rne", grad_fp8=_fp8_args(p, s))
    dy = np.zeros_like(got["dy_b"])
    for j in range(k):
        dy[got["assign_row"][:, j]] = got["topk_w"][:, j:j + 1] * got["dc"]
    assert got["grad_amax"][0] == np.abs(dy).max()
    for n in ("dh", "dzp", "dx"):
        rel = np.sqrt(np.mean((got[n] - ref[n]) ** 2) / np.mean(ref[n] ** 2))
        assert 1e-4 < rel < 0.1, (n, rel)     # FP8 noise: present, and small
    for n in ("dW_down", "dW_lat_up"):        # upstream of / outside the FP8 GEMMs
        np.testing.assert_array_equal(got[n], ref[n])


def test_shared_expert_gradients_alone():
    """With W_up = 0 and W_r = 0 (uniform routing, no routed contribution to
    out) the layer is the shared expert alone: its gradients are those of a
    dense SwiGLU FFN, checked here by finite differences of the forward
    oracle's shared_expert directly; dx is the shared expert's alone (the
    latent path's dz is 0 because dc = g_out W_up = 0)."""
    p, k = small_layer(7, Fs=5)
    p["w_lat_up"][:] = 0.0
    g = bwd(p, k, mode="exact")
    eps = 1e-6

    def lossf(q):
        return float(np.sum(p["g_out"] * oracle.shared_expert(q["x"], q["ws_gate"], q["ws_up"],
                                                                q["ws_down"], mode="exact")))
    for name, gname in (("ws_gate", "dWs_gate"), ("ws_up", "dWs_up"), ("ws_down", "dWs_down")):
        base = p[name]
        num = np.zeros_like(base)
        for i in np.ndindex(base.shape):
            old = base[i]
            base[i] = old + eps
            lp = lossf(p)
            base[i] = old - eps
            lm = lossf(p)
            base[i] = old
            num[i] = (lp - lm) / (2 * eps)
        assert np.max(np.abs(g[gname] - num)) < 1e-6 * max(1.0, np.max(np.abs(num))), name
    assert np.all(g["dx_latent"] == 0)
    np.testing.assert_allclose(g["dx_shared"] + g["dx_router"], g["dx"], rtol=0, atol=1e-12)


def test_shared_expert_stochastic_rounding_streams():
    """In bf16_operands mode with stochastic rounding the shared expert's
    gate and up gradients are cast stochastically: every cast value is one
    of the two bf16 neighbours of the float32 value (truncated, or one bf16
    step further from zero), both occur, and another seed changes the bits;
    nearest rounding gives the nearest neighbour."""
    p, k = small_layer(8, T=40, Fs=16)
    g1 = bwd(p, k, mode="bf16_operands", rounding="sr", seed=1)
    g2 = bwd(p, k, mode="bf16_operands", rounding="sr", seed=2)
    gn = bwd(p, k, mode="bf16_operands", rounding="rne", seed=1)
    gs = p["x"] @ p["ws_gate"].T
    us = p["x"] @ p["ws_up"].T
    hs = oracle.round_bf16(oracle.silu(gs) * us)
    np.testing.assert_array_equal(g1["hs_b"], hs)
    exact = {"dgs_b": g1["dhs"] * us * B.silu_grad(gs), "dus_b": g1["dhs"] * oracle.silu(gs)}
    for name, v in exact.items():
        u = np.ascontiguousarray(v.astype(np.float32)).view(np.uint32).astype(np.uint64)
        lo = (u & 0xFFFF0000).astype(np.uint32).view(np.float32).astype(np.float64)
        hi = ((u & 0xFFFF0000) + 0x10000).astype(np.uint32).view(np.float32).astype(np.float64)
        got = g1[name]
        assert np.all((got == lo) | (got == hi)), name
        assert np.any(got == lo) and np.any(got == hi), name
        assert not np.array_equal(got, g2[name]), name
    # nearest rounding (g_out itself is then rounded to nearest, so dhs differs)
    ex_n = {"dgs_b": gn["dhs"] * us * B.silu_grad(gs), "dus_b": gn["dhs"] * oracle.silu(gs)}
    for name, v in ex_n.items():
        np.testing.assert_array_equal(gn[name], oracle.round_bf16(v.astype(np.float32)))
