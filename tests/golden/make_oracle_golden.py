"""Writes tests/golden/tiny_oracle.json: golden values of the oracle on the tiny
LatentMoE workload (seed 0), in the style of golden-configuration regression
tests (page "The Training and RL Infrastructure Behind MAI-Thinking-1",
section 2 "Numerics", "Bitwise determinism": golden configurations whose
values are updated deliberately when numerics change).

Calls only the oracle and the seeded input generator.  Re-run it only when the
oracle's arithmetic changes on purpose, and say why in the commit message.
"""
import json
import os
import sys
import zlib

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
from moe_synth import CONFIGS, gen  # noqa: E402


def crc(a):
    return zlib.crc32(np.ascontiguousarray(a, dtype=np.int32).tobytes())


def main():
    cfg = CONFIGS["tiny"]
    inp = gen.host_inputs_f64(cfg)
    experts = [(inp["w_gate"][e], inp["w_up"][e], inp["w_down"][e]) for e in range(cfg.E)]
    out = {"config": cfg.name, "seed": cfg.seed}
    for mode in ("exact", "bf16_operands"):
        r = oracle.forward(inp["x"], inp["w_router"], inp["b_router"], cfg.k, inp["w_dn"], experts,
                           inp["w_lat_up"], mode=mode)
        out[mode] = {
            "crc_topk_idx": crc(r["topk_idx"]),
            "crc_expert_offsets": crc(r["expert_offsets"]),
            "crc_row_token": crc(r["row_token"]),
            "crc_assign_row": crc(r["assign_row"]),
            "expert_counts": [int(v) for v in r["expert_counts"]],
            "topk_w_sum": float(r["topk_w"].sum()),
            "out_sum": float(r["out"].sum()),
            "out_abs_sum": float(np.abs(r["out"]).sum()),
            "out_first": [float(v) for v in r["out"][0, :8]],
            "out_last": [float(v) for v in r["out"][-1, -8:]],
        }
    with open(os.path.join(HERE, "tiny_oracle.json"), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
