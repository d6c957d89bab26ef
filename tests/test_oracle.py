"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Each test ties one part of ``oracle/latent_moe.py`` to something other than
the oracle itself: a closed form worked out by hand, a brute-force evaluation
over all experts, an invariant, or a special case that reduces to a known
routine.  Together they are chosen so that a dropped term, a wrong sign, a
wrong index or a transposed operand anywhere in the oracle fails at least one.
"""
import math

import numpy as np
import pytest
import scipy.special

import oracle
from oracle import latent_moe as om

LN3 = math.log(3.0)


def _rng(seed):
    return np.random.default_rng(seed)


def _random_layer(seed, T=37, d=24, L=16, E=8, k=3, F=20, Fs=0, bias=False):
    r = _rng(seed)
    x = r.standard_normal((T, d))
    w_r = r.standard_normal((E, d)) / math.sqrt(d)
    b = r.standard_normal(E) if bias else None
    w_dn = r.standard_normal((L, d)) / math.sqrt(d)
    experts = [(r.standard_normal((F, L)) / math.sqrt(L), r.standard_normal((F, L)) / math.sqrt(L),
                r.standard_normal((L, F)) / math.sqrt(F)) for _ in range(E)]
    w_up = r.standard_normal((d, L)) / math.sqrt(L)
    shared = None
    if Fs:
        shared = (r.standard_normal((Fs, d)) / math.sqrt(d), r.standard_normal((Fs, d)) / math.sqrt(d),
                  r.standard_normal((d, Fs)) / math.sqrt(Fs))
    return dict(x=x, w_router=w_r, b_router=b, k=k, w_dn=w_dn, experts=experts, w_lat_up=w_up,
                shared=shared)


def _fp8_scales(lay):
    """Per-tensor FP8 scales for a random layer: 448 / amax of z, of h (over
    every expert applied to every token, a bound of the routed rows' amax)
    and of each expert weight."""
    z = om.latent_down(lay["x"], lay["w_dn"], "bf16_operands")
    amax = lambda a: float(np.max(np.abs(a)))  # noqa: E731
    h_amax = max(amax(om.silu(z @ g.T) * (z @ u.T)) for g, u, _ in lay["experts"])
    return {"z": np.float32(448.0 / amax(z)), "h": np.float32(448.0 / h_amax),
            "w_gate": [np.float32(448.0 / amax(g)) for g, _, _ in lay["experts"]],
            "w_up": [np.float32(448.0 / amax(u)) for _, u, _ in lay["experts"]],
            "w_down": [np.float32(448.0 / amax(d)) for _, _, d in lay["experts"]]}


def _fp8_for(lay, mode):
    return _fp8_scales(lay) if mode == "fp8_operands" else None


# ---------------------------------------------------------------------------
# bf16 rounding
# ---------------------------------------------------------------------------

def test_round_bf16_exact_values():
    u = 2.0 ** -7   # bf16 spacing just above 1.0
    cases = {
        1.0: 1.0,
        1.0 + u: 1.0 + u,                      # representable
        1.0 + u / 2: 1.0,                      # midpoint, ties to even (down)
        1.0 + 3 * u / 2: 1.0 + 2 * u,          # midpoint, ties to even (up)
        1.0 + u / 2 + 2.0 ** -30: 1.0 + u,     # just above the midpoint
        -(1.0 + u / 2 + 2.0 ** -30): -(1.0 + u),
        3.0: 3.0,
        0.0: 0.0,
        1.0 / 3.0: 0.333984375,                # 0x3EAB
        1e-3: 0.00099945068359375,             # 0x3A83
    }
    for v, want in cases.items():
        assert om.round_bf16(np.array([v]))[0] == want, v


def test_round_bf16_matches_bit_level_rounding_of_float32():
    # For values that are exactly float32, rounding to bf16 is the classic
    # 16-bit truncation with round-half-even on the float32 bit pattern.
    r = _rng(1)
    v = (r.standard_normal(20000) * np.exp(r.uniform(-20, 20, 20000))).astype(np.float32)
    bits = v.view(np.uint32).astype(np.uint64)
    rounded = ((bits + 0x7FFF + ((bits >> 16) & 1)) >> 16) << 16
    want = rounded.astype(np.uint32).view(np.float32).astype(np.float64)
    np.testing.assert_array_equal(om.round_bf16(v.astype(np.float64)), want)


# ---------------------------------------------------------------------------
# router: softmax gating and stable top-k
# ---------------------------------------------------------------------------

def test_softmax_closed_form():
    p = om.softmax(np.log(np.array([[1.0, 2.0, 3.0, 4.0]])))
    np.testing.assert_allclose(p, [[0.1, 0.2, 0.3, 0.4]], rtol=0, atol=1e-15)


def test_softmax_sums_to_one_and_matches_scipy():
    l = _rng(2).standard_normal((50, 512)) * 3
    p = om.softmax(l)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-12)
    np.testing.assert_allclose(p, scipy.special.softmax(l, axis=1), rtol=1e-12, atol=0)
    # invariant to a per-token shift of all logits
    np.testing.assert_allclose(om.softmax(l + 7.5), p, rtol=1e-12)


def _router_for_logits(target):
    """x = I (T = E = d) and W_r = target^T give logits == target exactly."""
    T, E = target.shape
    return np.eye(T), target.T.copy()


def test_route_closed_form_not_renormalised():
    target = np.log(np.array([[1.0, 2.0, 3.0, 4.0],
                              [4.0, 3.0, 2.0, 1.0],
                              [1.0, 4.0, 2.0, 3.0],
                              [2.0, 2.0, 2.0, 2.0]]))
    x, w_r = _router_for_logits(target)
    r = om.route(x, w_r, None, 2)
    np.testing.assert_array_equal(r["topk_idx"], [[3, 2], [0, 1], [1, 3], [0, 1]])
    np.testing.assert_allclose(r["topk_w"], [[0.4, 0.3], [0.4, 0.3], [0.4, 0.3], [0.25, 0.25]],
                               atol=1e-15)


def test_route_bias_enters_before_softmax():
    target = np.log(np.array([[1.0, 2.0, 3.0, 4.0]]))
    x, w_r = _router_for_logits(target)
    r = om.route(x, w_r, np.log(np.array([10.0, 1.0, 1.0, 1.0])), 2)
    np.testing.assert_array_equal(r["topk_idx"], [[0, 3]])
    np.testing.assert_allclose(r["topk_w"], [[10 / 19, 4 / 19]], atol=1e-15)


def test_route_bias_for_selection_only():
    # loss-free balancer: the bias picks expert 0, the weights stay those of
    # the unbiased softmax (0.1, 0.2, 0.3, 0.4), not renormalised
    target = np.log(np.array([[1.0, 2.0, 3.0, 4.0]]))
    x, w_r = _router_for_logits(target)
    r = om.route(x, w_r, np.log(np.array([10.0, 1.0, 1.0, 1.0])), 2, bias_mode="selection")
    np.testing.assert_array_equal(r["topk_idx"], [[0, 3]])
    np.testing.assert_allclose(r["topk_w"], [[0.1, 0.4]], atol=1e-15)
    np.testing.assert_allclose(r["probs"], [[0.1, 0.2, 0.3, 0.4]], atol=1e-15)
    # without a bias both modes are the same
    a = om.route(x, w_r, None, 2, bias_mode="selection")
    b = om.route(x, w_r, None, 2)
    np.testing.assert_array_equal(a["topk_idx"], b["topk_idx"])
    np.testing.assert_array_equal(a["topk_w"], b["topk_w"])
    with pytest.raises(ValueError):
        om.route(x, w_r, None, 2, bias_mode="other")


def test_lbl_stats_closed_form_and_invariants():
    target = np.log(np.array([[1.0, 2.0, 3.0, 4.0], [4.0, 3.0, 2.0, 1.0], [2.0, 2.0, 2.0, 2.0]]))
    x, w_r = _router_for_logits(target)
    r = om.route(x, w_r, None, 2)
    st = om.lbl_stats(r["probs"], r["topk_idx"], 4)
    # selections: (3,2), (0,1), (0,1)
    np.testing.assert_array_equal(st["counts"], [2, 2, 1, 1])
    np.testing.assert_allclose(st["prob_sum"], [0.1 + 0.4 + 0.25, 0.2 + 0.3 + 0.25,
                                                0.3 + 0.2 + 0.25, 0.4 + 0.1 + 0.25], atol=1e-15)
    lay = _random_layer(21, T=50, E=12, k=3, bias=True)
    for mode in om.BIAS_MODES:
        rr = om.route(lay["x"], lay["w_router"], lay["b_router"], 3, bias_mode=mode)
        s2 = om.lbl_stats(rr["probs"], rr["topk_idx"], 12)
        assert s2["counts"].sum() == 50 * 3
        np.testing.assert_allclose(s2["prob_sum"].sum(), 50.0, rtol=1e-13)
        # additive over micro-batches
        h1 = om.lbl_stats(rr["probs"][:20], rr["topk_idx"][:20], 12)
        h2 = om.lbl_stats(rr["probs"][20:], rr["topk_idx"][20:], 12)
        np.testing.assert_array_equal(h1["counts"] + h2["counts"], s2["counts"])
        np.testing.assert_allclose(h1["prob_sum"] + h2["prob_sum"], s2["prob_sum"], rtol=1e-13)


def test_route_ties_go_to_lower_index():
    x, w_r = _router_for_logits(np.zeros((3, 6)))
    r = om.route(x, w_r, None, 4)
    np.testing.assert_array_equal(r["topk_idx"], [[0, 1, 2, 3]] * 3)
    np.testing.assert_allclose(r["topk_w"], 1 / 6, atol=1e-15)
    # partial tie: experts 4 and 1 share the top logit -> 1 first, then 4
    t = np.array([[0.0, 5.0, 1.0, -2.0, 5.0, 1.0]])
    x, w_r = _router_for_logits(t)
    np.testing.assert_array_equal(om.route(x, w_r, None, 4)["topk_idx"], [[1, 4, 2, 5]])


def _topk_by_repeated_argmax(scores, k):
    s = np.array(scores, dtype=np.float64, copy=True)
    out = np.empty((s.shape[0], k), np.int64)
    for j in range(k):
        a = np.argmax(s, axis=1)          # first occurrence of the max = lowest index
        out[:, j] = a
        s[np.arange(s.shape[0]), a] = -np.inf
    return out


@pytest.mark.parametrize("E,k", [(16, 2), (512, 8), (512, 7), (64, 16), (5, 5), (1, 1)])
def test_topk_matches_brute_force(E, k):
    r = _rng(E * 31 + k)
    l = r.standard_normal((200, E)).astype(np.float32)
    l[::7, : E // 2] = 0.25            # planted ties
    np.testing.assert_array_equal(om.topk_stable(l, k), _topk_by_repeated_argmax(l, k))


def test_route_selects_on_fp32_logits():
    # two logits that differ in float64 but round to the same float32 value:
    # the selection sees a tie and keeps the lower index
    a = 1.0
    b = 1.0 + 2.0 ** -30
    x, w_r = _router_for_logits(np.array([[a, b, -1.0]]))
    r = om.route(x, w_r, None, 1)
    assert r["topk_idx"][0, 0] == 0
    assert r["logits"][0, 1] > r["logits"][0, 0]


# ---------------------------------------------------------------------------
# permutation
# ---------------------------------------------------------------------------

def _check_perm_invariants(idx, E, p):
    T, k = idx.shape
    counts, off, rt, ar = (p["expert_counts"], p["expert_offsets"], p["row_token"], p["assign_row"])
    np.testing.assert_array_equal(counts, np.bincount(idx.ravel(), minlength=E))
    assert off[0] == 0 and off[-1] == T * k
    np.testing.assert_array_equal(np.diff(off), counts)
    # assign_row is a bijection onto [0, T*k)
    np.testing.assert_array_equal(np.sort(ar.ravel()), np.arange(T * k))
    for t in range(T):
        for j in range(k):
            r = ar[t, j]
            assert rt[r] == t
            e = np.searchsorted(off, r, side="right") - 1
            assert e == idx[t, j]
    for e in range(E):
        seg = rt[off[e]:off[e + 1]]
        assert np.all(np.diff(seg) > 0)           # ascending tokens inside an expert
    np.testing.assert_array_equal(np.bincount(rt, minlength=T), np.full(T, k))


def _distinct_topk(r, T, E, k, hot=False):
    if hot:   # every token picks the same k experts
        return np.tile(np.arange(E - k, E), (T, 1))
    return np.stack([r.permutation(E)[:k] for _ in range(T)])


@pytest.mark.parametrize("T,E,k,hot", [(1, 4, 1, False), (17, 16, 2, False), (64, 8, 8, False),
                                       (50, 32, 4, True), (33, 1024, 16, False), (200, 512, 8, False)])
def test_permute_invariants(T, E, k, hot):
    r = _rng(T + E + k)
    idx = _distinct_topk(r, T, E, k, hot)
    _check_perm_invariants(idx, E, om.permute(idx, E))


def test_permute_brute_force_small():
    idx = np.array([[2, 0], [0, 1], [2, 1], [1, 0], [3, 2]])
    p = om.permute(idx, 5)
    rows = []
    for e in range(5):
        for t in range(idx.shape[0]):
            for j in range(idx.shape[1]):
                if idx[t, j] == e:
                    rows.append((t, j))
    np.testing.assert_array_equal(p["row_token"], [t for t, _ in rows])
    for r_, (t, j) in enumerate(rows):
        assert p["assign_row"][t, j] == r_
    np.testing.assert_array_equal(p["expert_counts"], [3, 3, 3, 1, 0])
    np.testing.assert_array_equal(p["expert_offsets"], [0, 3, 6, 9, 10, 10])


def test_permute_empty_input():
    p = om.permute(np.zeros((0, 3), np.int32), 4)
    np.testing.assert_array_equal(p["expert_offsets"], [0, 0, 0, 0, 0])
    assert p["row_token"].size == 0


# ---------------------------------------------------------------------------
# SwiGLU, projections, combine: closed forms
# ---------------------------------------------------------------------------

def test_silu_closed_forms():
    v = np.array([0.0, LN3, -LN3, 40.0, -40.0])
    np.testing.assert_allclose(om.silu(v), [0.0, 0.75 * LN3, -0.25 * LN3, 40.0, -40.0 / (1 + math.exp(40))],
                               rtol=1e-15, atol=1e-300)
    w = _rng(3).standard_normal(1000) * 5
    np.testing.assert_allclose(om.silu(w) - om.silu(-w), w, rtol=1e-13, atol=1e-13)


def _hand_layer():
    """A 2-wide layer with asymmetric matrices whose output is worked out by hand.

    x = [1, 0];  z = W_dn x = [1, 0]   (W_dn^T x would be [1, 2])
    g = W_g z = [ln 3, 0]              (W_g^T z would be [ln 3, 5])
    u = W_u z = [2, 3]
    h = silu(g) * u = [0.75 ln3 * 2, 0] = [1.5 ln 3, 0]
    y = W_d h = [1.5 ln 3, 3 ln 3]
    out = W_up y = [4.5 ln 3, 6 ln 3]
    """
    x = np.array([[1.0, 0.0]])
    w_dn = np.array([[1.0, 2.0], [0.0, 1.0]])
    w_g = np.array([[LN3, 5.0], [0.0, 7.0]])
    w_u = np.array([[2.0, 1.0], [3.0, 4.0]])
    w_d = np.array([[1.0, 4.0], [2.0, 3.0]])
    w_up = np.array([[1.0, 1.0], [0.0, 2.0]])
    return x, w_dn, (w_g, w_u, w_d), w_up


def test_single_expert_closed_form():
    x, w_dn, ex, w_up = _hand_layer()
    res = om.forward(x, np.zeros((1, 2)), None, 1, w_dn, [ex], w_up)
    np.testing.assert_allclose(res["z"], [[1.0, 0.0]], atol=1e-15)
    np.testing.assert_allclose(res["y_rows"], [[1.5 * LN3, 3 * LN3]], rtol=1e-14)
    np.testing.assert_allclose(res["out"], [[4.5 * LN3, 6 * LN3]], rtol=1e-14)


def test_two_experts_weight_not_renormalised():
    # expert 0 has logit ln 3, expert 1 logit 0 -> p = (0.75, 0.25); top-1 keeps 0.75
    x, w_dn, ex, w_up = _hand_layer()
    zero = tuple(np.zeros_like(a) for a in ex)
    w_r = np.array([[LN3, 0.0], [0.0, 0.0]])
    res = om.forward(x, w_r, None, 1, w_dn, [ex, zero], w_up)
    np.testing.assert_array_equal(res["topk_idx"], [[0]])
    np.testing.assert_allclose(res["topk_w"], [[0.75]], atol=1e-15)
    np.testing.assert_allclose(res["out"], [[0.75 * 4.5 * LN3, 0.75 * 6 * LN3]], rtol=1e-14)
    # top-2 over both experts: the zero expert adds nothing, weights stay (0.75, 0.25)
    res2 = om.forward(x, w_r, None, 2, w_dn, [ex, zero], w_up)
    np.testing.assert_allclose(res2["topk_w"], [[0.75, 0.25]], atol=1e-15)
    np.testing.assert_allclose(res2["out"], res["out"], rtol=1e-14)


def test_shared_expert_closed_form_and_isolation():
    # W_lat_up = 0 isolates the shared expert; with the hand matrices applied
    # directly to x (no latent projection): g = W_g x = [ln3, 0], u = [2, 3],
    # h = [1.5 ln3, 0], s = W_d h = [1.5 ln3, 3 ln3]
    x, w_dn, (w_g, w_u, w_d), w_up = _hand_layer()
    lay = _random_layer(5, T=1, d=2, L=2, E=3, k=2, F=4)
    res = om.forward(x, lay["w_router"], None, 2, w_dn, lay["experts"], np.zeros((2, 2)),
                     shared=(w_g, w_u, w_d))
    np.testing.assert_allclose(res["out"], [[1.5 * LN3, 3 * LN3]], rtol=1e-14)


def test_combine_fixed_order_weighted_sum():
    y = np.array([[1.0, 2.0], [10.0, 20.0], [100.0, 200.0]])
    w = np.array([[0.5, 0.25], [1.0, 2.0]])
    ar = np.array([[2, 0], [1, 2]])
    np.testing.assert_allclose(om.combine(y, w, ar), [[50.25, 100.5], [210.0, 420.0]], rtol=1e-15)


# ---------------------------------------------------------------------------
# whole layer: brute force, special cases, invariants
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seed,k,bias,Fs", [(0, 3, False, 0), (1, 1, True, 0), (2, 8, False, 0),
                                            (3, 2, True, 12)])
def test_permuted_path_equals_dense_bruteforce(seed, k, bias, Fs):
    lay = _random_layer(seed, k=k, bias=bias, Fs=Fs)
    for mode in oracle.MODES:
        a = om.forward(**lay, mode=mode, fp8=_fp8_for(lay, mode))
        b = om.forward_dense_bruteforce(**lay, mode=mode, fp8=_fp8_for(lay, mode))
        np.testing.assert_array_equal(a["topk_idx"], b["topk_idx"])
        scale = np.sqrt(np.mean(b["out"] ** 2))
        assert np.max(np.abs(a["out"] - b["out"])) <= 1e-12 * scale


def test_per_token_definition_equals_permuted_path():
    lay = _random_layer(7, k=3, Fs=8)
    for mode in oracle.MODES:
        a = om.forward(**lay, mode=mode, fp8=_fp8_for(lay, mode))
        b = om.forward_tokens(lay["x"], a["topk_idx"], a["topk_w"], lay["w_dn"], lay["experts"],
                              lay["w_lat_up"], shared=lay["shared"], mode=mode,
                              fp8=_fp8_for(lay, mode))
        np.testing.assert_allclose(b["out"], a["out"], rtol=1e-12, atol=1e-12)


def test_identity_experts_give_input_times_selected_weight_sum():
    lay = _random_layer(11, T=29, d=16, L=16, E=6, k=3, F=16)
    eye = np.eye(16)
    res = om.forward(lay["x"], lay["w_router"], None, 3, eye, None, eye,
                     expert_fn=lambda e, zr: zr)
    want = lay["x"] * res["topk_w"].sum(axis=1, keepdims=True)
    np.testing.assert_allclose(res["out"], want, rtol=1e-13, atol=1e-13)


def test_k_equals_E_is_the_dense_soft_mixture():
    lay = _random_layer(12, T=9, E=5, k=5)
    res = om.forward(**lay)
    z = lay["x"] @ lay["w_dn"].T
    probs = om.softmax(lay["x"] @ lay["w_router"].T)
    c = sum(probs[:, e:e + 1] * om.swiglu_expert(z, *lay["experts"][e]) for e in range(5))
    np.testing.assert_allclose(res["out"], c @ lay["w_lat_up"].T, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(res["topk_w"].sum(axis=1), 1.0, atol=1e-12)


def test_single_expert_is_a_dense_latent_swiglu_ffn():
    lay = _random_layer(13, E=1, k=1)
    res = om.forward(**lay)
    np.testing.assert_allclose(res["topk_w"], 1.0, atol=1e-15)
    z = lay["x"] @ lay["w_dn"].T
    wg, wu, wd = lay["experts"][0]
    g, u = z @ wg.T, z @ wu.T
    want = ((g * scipy.special.expit(g) * u) @ wd.T) @ lay["w_lat_up"].T
    np.testing.assert_allclose(res["out"], want, rtol=1e-12, atol=1e-12)


def test_linearity_in_output_weights():
    lay = _random_layer(14, k=2)
    base = om.forward(**lay)["out"]
    lay2 = dict(lay, w_lat_up=lay["w_lat_up"] * 3.0)
    np.testing.assert_allclose(om.forward(**lay2)["out"], 3.0 * base, rtol=1e-12)
    lay3 = dict(lay, experts=[(g, u, -2.0 * d) for g, u, d in lay["experts"]])
    np.testing.assert_allclose(om.forward(**lay3)["out"], -2.0 * base, rtol=1e-12)


def test_token_permutation_equivariance():
    lay = _random_layer(15, T=41, k=3)
    perm = _rng(15).permutation(41)
    a = om.forward(**lay)
    b = om.forward(**dict(lay, x=lay["x"][perm]))
    np.testing.assert_allclose(b["out"], a["out"][perm], rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(b["topk_idx"], a["topk_idx"][perm])


def test_bf16_mode_rounds_only_gemm_operands():
    lay = _random_layer(16, k=2, Fs=8)
    ex = om.forward(**lay, mode="exact")
    bf = om.forward(**lay, mode="bf16_operands")
    np.testing.assert_array_equal(bf["z"], om.round_bf16(ex["z"]))
    rel = np.max(np.abs(bf["out"] - ex["out"])) / np.sqrt(np.mean(ex["out"] ** 2))
    assert 1e-5 < rel < 5e-2


# ---------------------------------------------------------------------------
# FP8 E4M3 operands (forward GEMMs in FP8 with per-tensor scales)
# ---------------------------------------------------------------------------

def _e4m3_values():
    """Every finite non-negative E4M3FN value in code order, decoded from the
    bit fields (exponent bias 7, 3 fraction bits; code 0x7F is NaN)."""
    vals = []
    for code in range(0x7F):
        e, m = code >> 3, code & 7
        vals.append((m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7))
    return np.array(vals)


def test_e4m3_table_landmarks():
    tab = _e4m3_values()
    assert tab[-1] == 448.0 and tab[1] == 2.0 ** -9 and tab[8] == 2.0 ** -6 and tab[0x38] == 1.0
    assert np.all(np.diff(tab) > 0)


def test_round_e4m3_exact_values():
    cases = [(1.0, 1.0), (1.0625, 1.0), (1.1875, 1.25), (1.125, 1.125), (3 * 2.0 ** -10, 2.0 ** -8),
             (2.0 ** -10, 0.0), (2.0 ** -9, 2.0 ** -9), (464.0, 448.0), (479.0, 448.0),
             (500.0, 448.0), (1e9, 448.0), (-1.0625, -1.0), (0.0146484375, 0.015625), (3.3, 3.25),
             (-3.3, -3.25), (240.0, 240.0), (256.0, 256.0), (0.0, 0.0), (1e-8, 0.0)]
    for v, want in cases:
        assert om.round_e4m3(np.array([v]))[0] == want, v


def test_round_e4m3_is_the_nearest_value_ties_to_even_code():
    tab = _e4m3_values()
    r = _rng(21)
    mags = np.exp(r.uniform(np.log(2.0 ** -12), np.log(600.0), 20000))
    mids = (tab[:-1] + tab[1:]) / 2                      # every tie
    v = np.concatenate([mags, -mags, mids, -mids, tab, [600.0, 1e6]])
    got = om.round_e4m3(v)
    a = np.minimum(np.abs(v), 448.0)                     # saturating conversion
    dist = np.abs(tab[None, :] - a[:, None])
    cand = dist == dist.min(axis=1, keepdims=True)
    even = (np.arange(tab.size) % 2 == 0)[None, :]
    pick = np.where(cand.sum(axis=1) > 1, np.argmax(cand & even, axis=1), np.argmax(cand, axis=1))
    np.testing.assert_array_equal(got, np.copysign(tab[pick], v))


def test_quantize_e4m3_saturates_and_scales():
    np.testing.assert_array_equal(om.quantize_e4m3(np.array([1000.0, -1000.0, 3.0]), 1.0),
                                  [448.0, -448.0, 3.0])
    # 0.75 * 2**-3 = 0.09375 = 1.5 * 2**-4 (exact); with scale 8 it is 0.75
    np.testing.assert_array_equal(om.quantize_e4m3(np.array([0.09375]), 8.0), [0.75])


def test_fp8_matmul_exact_for_representable_operands_and_power_of_two_scales():
    tab = _e4m3_values()
    r = _rng(22)
    # normal values 2**-5 .. 7.5: times 4 or halved they stay normal and below 448
    a = np.copysign(r.choice(tab[16:80], (5, 16)), r.standard_normal((5, 16)))
    b = np.copysign(r.choice(tab[16:80], (7, 16)), r.standard_normal((7, 16)))
    np.testing.assert_array_equal(om.fp8_matmul(a, b, 1.0, 1.0), a @ b.T)
    # power-of-two scales shift whole binades (no saturation, no underflow here)
    np.testing.assert_array_equal(om.fp8_matmul(a, b, 4.0, 0.5), a @ b.T)
    # and the division by the scales is not dropped: one operand is scaled 2x
    np.testing.assert_array_equal(om.fp8_matmul(a, 2 * b, 1.0, 0.5), 2 * (a @ b.T))


def test_fp8_scale_from_history():
    h = np.array([[0.5, 2.0, 1.0], [0.0, 0.0, 0.0], [448.0, 1.0, 3.0], [0.0, 7.0, 0.0]], np.float32)
    np.testing.assert_array_equal(om.fp8_scale_from_history(h),
                                  np.array([224.0, 1.0, 1.0, 64.0], np.float32))


def test_fp8_mode_quantizes_expert_operands_only():
    lay = _random_layer(23, k=2, Fs=8)
    sc = _fp8_scales(lay)
    bf = om.forward(**lay, mode="bf16_operands")
    f8 = om.forward(**lay, mode="fp8_operands", fp8=sc)
    np.testing.assert_array_equal(f8["z"], bf["z"])           # z itself stays bf16
    # one expert by hand: every operand through e4m3 with its scale
    e, zr = 0, bf["z"][:3]
    wg, wu, wd = lay["experts"][e]
    qz = om.round_e4m3(np.float32(zr) * sc["z"])
    g = (qz @ om.round_e4m3(np.float32(wg) * sc["w_gate"][e]).T) / (float(sc["z"]) * float(sc["w_gate"][e]))
    u = (qz @ om.round_e4m3(np.float32(wu) * sc["w_up"][e]).T) / (float(sc["z"]) * float(sc["w_up"][e]))
    h = om.round_bf16(g / (1 + np.exp(-g)) * u)
    y = (om.round_e4m3(np.float32(h) * sc["h"]) @ om.round_e4m3(np.float32(wd) * sc["w_down"][e]).T) \
        / (float(sc["h"]) * float(sc["w_down"][e]))
    got = om.swiglu_expert(zr, wg, wu, wd, mode="fp8_operands", fp8=om.expert_fp8_scales(sc, e))
    np.testing.assert_allclose(got, y, rtol=1e-12, atol=1e-15)
    rel = np.max(np.abs(f8["out"] - bf["out"])) / np.sqrt(np.mean(bf["out"] ** 2))
    assert 1e-3 < rel < 0.3


# ---------------------------------------------------------------------------
# multi-round dropless schedule (fixed per-expert capacity, borrowing inside
# expert groups)
# ---------------------------------------------------------------------------

def test_round_schedule_hand_worked():
    # 4 experts in groups of 2, capacity 2: group 0 holds 5 + 0 rows (4 slots
    # per round: expert 0 borrows expert 1's two slots, then overflows into a
    # second round), group 1 holds 1 + 1 rows (one round)
    offsets = np.array([0, 5, 5, 6, 7])
    rounds, plan = om.round_schedule(offsets, capacity=2, group_size=2)
    assert rounds == 2
    assert plan[0] == [(0, 4, 0), (5, 5, 4), (5, 6, 4), (6, 7, 5)]
    assert plan[1] == [(4, 5, 0), (5, 5, 1), (6, 6, 4), (7, 7, 4)]


def test_round_schedule_without_borrowing_or_with_one_group():
    offsets = np.array([0, 5, 5, 6, 7])
    # groups of one expert: no borrowing, expert 0 needs ceil(5 / 2) = 3 rounds
    assert om.round_schedule(offsets, 2, 1)[0] == 3
    # one group of all four: 8 slots per round hold all 7 rows
    assert om.round_schedule(offsets, 2, 4)[0] == 1
    # nothing routed: no round
    assert om.round_schedule(np.zeros(5, np.int64), 2, 2)[0] == 0


@pytest.mark.parametrize("capacity,group", [(3, 2), (8, 4), (1, 3), (50, 8)])
def test_round_schedule_invariants(capacity, group):
    r = _rng(capacity * 10 + group)
    counts = r.poisson(r.uniform(0, 20, 13))
    offsets = np.concatenate([[0], np.cumsum(counts)])
    rounds, plan = om.round_schedule(offsets, capacity, group)
    E = counts.size
    seen = np.zeros(offsets[-1], np.int64)
    for rr in plan:
        used = np.zeros(E * capacity, np.int64)
        for e, (b, en, h) in enumerate(rr):
            assert offsets[e] <= b <= en <= offsets[e + 1]
            seen[b:en] += 1
            used[h:h + (en - b)] += 1
            g0 = e // group * group
            assert g0 * capacity <= h and h + (en - b) <= min(g0 + group, E) * capacity
        assert used.max(initial=0) <= 1          # slots of one round never overlap
    np.testing.assert_array_equal(seen, 1)       # every row in exactly one round
    loads = [offsets[min(g + group, E)] - offsets[g] for g in range(0, E, group)]
    caps = [(min(g + group, E) - g) * capacity for g in range(0, E, group)]
    assert rounds == max(-(-ld // c) for ld, c in zip(loads, caps))
