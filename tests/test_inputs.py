"""Seeded synthetic inputs (CPU side) and the oracle's golden values."""
import json
import os
import zlib

import numpy as np
import pytest
from scipy.special import ndtr

import oracle
from moe_synth import CONFIGS, gen

HERE = os.path.dirname(os.path.abspath(__file__))


def test_same_seed_same_bytes_and_keys_differ():
    cfg = CONFIGS["tiny"]
    a = gen.host_tensor_bits(cfg, "x")
    b = gen.host_tensor_bits(cfg, "x")
    np.testing.assert_array_equal(a, b)
    c = gen.host_tensor_bits(cfg.replace(seed=1), "x")
    assert np.mean(a == c) < 0.01
    keys = {gen.tensor_key(s, t) for s in range(4) for t in gen.TID.values()}
    assert len(keys) == 4 * len(gen.TID)


def test_sub_tensor_indexing_matches_whole_tensor():
    cfg = CONFIGS["tiny"]
    whole = gen.host_tensor_bits(cfg, "w_gate")
    np.testing.assert_array_equal(gen.host_tensor_bits(cfg, "w_gate", (5,)), whole[5])
    np.testing.assert_array_equal(gen.host_tensor_bits(cfg, "w_gate", (5, 17)), whole[5, 17])
    x = gen.host_tensor_bits(cfg, "x")
    np.testing.assert_array_equal(gen.host_rows_f64(cfg, "x", [3, 200]),
                                  gen.bf16_bits_to_f64(x[[3, 200]]))


def test_high_counter_word_is_used():
    key = gen.tensor_key(0, 5)
    a = gen.hash_counter(2 ** 32 + 7, 64, key)
    b = gen.hash_counter(7, 64, key)
    assert np.mean(a == b) < 0.05


def test_table_is_a_bf16_quantile_table():
    t = gen.bf16_bits_to_f64(gen.normal_table_bits(1.0))
    assert np.all(np.diff(t) >= 0)
    np.testing.assert_array_equal(t, -t[::-1])          # symmetric
    # each entry is within one bf16 rounding of its quantile
    q = (np.arange(65536) + 0.5) / 65536
    np.testing.assert_allclose(ndtr(t), q, atol=2e-3)


@pytest.mark.parametrize("name", ["x", "w_dn", "w_gate", "w_down", "w_lat_up"])
def test_moments(name):
    cfg = CONFIGS["tiny"]
    shape, sigma = gen.tensor_specs(cfg)[name]
    v = gen.host_tensor_f64(cfg, name)
    assert abs(v.mean()) < 4 * sigma / np.sqrt(v.size) + 1e-3 * sigma
    assert abs(v.std() / sigma - 1) < 0.02


def test_router_inputs():
    cfg = CONFIGS["tiny"]
    w = gen.router_weights(cfg)
    assert w.dtype == np.float32 and w.shape == (cfg.E, cfg.d)
    assert abs(w.std() * np.sqrt(cfg.d) - 1) < 0.05
    assert gen.router_bias(cfg) is None
    b = gen.router_bias(CONFIGS["base1_imbalanced"])
    ranks = np.rint(np.exp(-b.astype(np.float64) / 2.4)).astype(int)
    np.testing.assert_array_equal(np.sort(ranks), np.arange(1, 513))


def test_ladder_shapes_of_the_configs():
    rows = [l.split() for l in open(os.path.join(HERE, "golden", "ladder_shapes.txt"))
            if l.strip() and not l.startswith("#")]
    ladder = {r[3]: (int(r[0]), int(r[1]), int(r[2])) for r in rows}
    for name, (layers, hidden, heads) in ladder.items():
        assert hidden * 3 == 256 * layers
        assert heads == 16 * round(layers / 16)
    assert CONFIGS["base1_compute"].d == ladder["MAI-Base-1"][1]
    assert CONFIGS["base2"].d == ladder["MAI-Base-2"][1]


def test_oracle_golden_values_tiny():
    want = json.load(open(os.path.join(HERE, "golden", "tiny_oracle.json")))
    cfg = CONFIGS["tiny"]
    inp = gen.host_inputs_f64(cfg)
    experts = [(inp["w_gate"][e], inp["w_up"][e], inp["w_down"][e]) for e in range(cfg.E)]
    crc = lambda a: zlib.crc32(np.ascontiguousarray(a, dtype=np.int32).tobytes())  # noqa: E731
    for mode in ("exact", "bf16_operands"):
        r = oracle.forward(inp["x"], inp["w_router"], inp["b_router"], cfg.k, inp["w_dn"], experts,
                           inp["w_lat_up"], mode=mode)
        w = want[mode]
        assert crc(r["topk_idx"]) == w["crc_topk_idx"]
        assert crc(r["expert_offsets"]) == w["crc_expert_offsets"]
        assert crc(r["row_token"]) == w["crc_row_token"]
        assert crc(r["assign_row"]) == w["crc_assign_row"]
        assert list(r["expert_counts"]) == w["expert_counts"]
        np.testing.assert_allclose(r["topk_w"].sum(), w["topk_w_sum"], rtol=1e-12)
        np.testing.assert_allclose(np.abs(r["out"]).sum(), w["out_abs_sum"], rtol=1e-10)
        np.testing.assert_allclose(r["out"][0, :8], w["out_first"], rtol=1e-9, atol=1e-12)
        np.testing.assert_allclose(r["out"][-1, -8:], w["out_last"], rtol=1e-9, atol=1e-12)
