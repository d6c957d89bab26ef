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


def small_layer(seed=0, T=5, d=6, L=4, E=4, k=2, Fw=3, bias=True):
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
    return p, k


def fwd_out(p, k):
    experts = [(p["w_gate"][e], p["w_up"][e], p["w_down"][e]) for e in range(p["w_gate"].shape[0])]
    return oracle.forward(p["x"], p["w_router"], p["b_router"], k, p["w_dn"], experts,
                          p["w_lat_up"], mode="exact")


def bwd(p, k, **kw):
    experts = [(p["w_gate"][e], p["w_up"][e], p["w_down"][e]) for e in range(p["w_gate"].shape[0])]
    return oracle.backward(p["x"], p["w_router"], p["b_router"], k, p["w_dn"], experts,
                           p["w_lat_up"], p["g_out"], **kw)


def loss(p, k):
    return float(np.sum(p["g_out"] * fwd_out(p, k)["out"]))


def selection_gap(p, k):
    lg = np.sort(oracle.router_logits(p["x"], p["w_router"], p["b_router"]), axis=1)[:, ::-1]
    return float(np.min(lg[:, k - 1] - lg[:, k]))


GRAD_OF = {"x": "dx", "w_router": "dW_router", "b_router": "db_router", "w_dn": "dW_dn",
           "w_gate": "dW_gate", "w_up": "dW_up", "w_down": "dW_down", "w_lat_up": "dW_lat_up"}


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_finite_differences_every_parameter(seed):
    p, k = small_layer(seed)
    assert selection_gap(p, k) > 1e-3      # the perturbation below never changes selection
    g = bwd(p, k, mode="exact")
    eps = 1e-6
    for name, gname in GRAD_OF.items():
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
