"""GPU tests of the multi-round dropless schedule (fixed per-expert capacity,
borrowing inside expert groups).

Each row is computed exactly as by the single-pass path, so y_rows and the
layer output must be bitwise equal to moe_latent_ffn_forward's on the same
routing (the oracle's, replayed), for capacities from one round down to many
rounds, with and without borrowing; the number of rounds the device reports
must equal the oracle's schedule; and the output must match the
bf16-operand oracle as the single-pass path does.
"""
import numpy as np
import pytest
import torch

import mixture_experts_layer_moe_amd as moe
import oracle
from moe_synth import MoEConfig, device, gen
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

CASES = {
    "zipf": MoEConfig("zipf", T=1024, d=256, L=128, E=64, k=4, F=256, zipf_bias=True, seed=11),
    "hot": MoEConfig("hot", T=4096, d=256, L=256, E=64, k=4, F=256, zipf_bias=True, seed=41),
    "deep": MoEConfig("deep", T=2048, d=256, L=256, E=8, k=2, F=512, seed=9),
    "shared": MoEConfig("shared", T=200, d=512, L=256, E=32, k=7, F=384, Fs=640, seed=5),
}
# (capacity as a fraction of the mean rows per expert, group size)
SCHEDULES = [(2.0, 8), (1.0, 4), (0.25, 1), (0.5, 64), (0.1, 3)]


@pytest.fixture(scope="module")
def cuda():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.load()
    return torch.device("cuda:0")


_cache = {}


def _setup(name, cuda):
    if name in _cache:
        return _cache[name]
    cfg = CASES[name]
    U.log(f"[rounds case {name}] {cfg}")
    host = gen.host_inputs_f64(cfg)
    dv = device.device_inputs(cfg, cuda)
    w = moe.LatentMoEWeights(dv["w_router"], dv["b_router"], dv["w_dn"], dv["w_gate"], dv["w_up"],
                             dv["w_down"], dv["w_lat_up"], dv.get("ws_gate"), dv.get("ws_up"),
                             dv.get("ws_down"))
    ro = oracle.route(host["x"], host["w_router"], host["b_router"], cfg.k)
    w32 = np.asarray(ro["topk_w"], np.float32)
    buf = moe.LatentMoEBuffers(cfg.T, cfg.d, cfg.L, cfg.E, cfg.k, cfg.F, cfg.Fs, device=cuda)
    buf.topk_idx.copy_(torch.from_numpy(np.asarray(ro["topk_idx"], np.int32)))
    buf.topk_w.copy_(torch.from_numpy(w32))
    moe.forward(dv["x"], w, cfg.k, buf, route=False)
    torch.cuda.synchronize()
    ref = {"y": buf.y_rows.clone(), "out": buf.out.clone()}
    perm = oracle.permute(ro["topk_idx"], cfg.E)
    _cache[name] = (cfg, host, dv, w, ro, w32, ref, perm)
    return _cache[name]


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("sched", SCHEDULES, ids=[f"c{c}-g{g}" for c, g in SCHEDULES])
def test_rounds_bitwise_equal_to_single_pass(cuda, name, sched):
    cfg, host, dv, w, ro, w32, ref, perm = _setup(name, cuda)
    mean = cfg.T * cfg.k / cfg.E
    capacity = max(1, int(round(sched[0] * mean)))
    group = min(sched[1], cfg.E)
    want_rounds, _ = oracle.round_schedule(perm["expert_offsets"], capacity, group)
    buf = moe.LatentMoEBuffers(cfg.T, cfg.d, cfg.L, cfg.E, cfg.k, cfg.F, cfg.Fs, device=cuda)
    buf.topk_idx.copy_(torch.from_numpy(np.asarray(ro["topk_idx"], np.int32)))
    buf.topk_w.copy_(torch.from_numpy(w32))
    buf.y_rows.fill_(float("nan"))
    rounds = torch.full((1,), -1, dtype=torch.int32, device=cuda)
    moe.forward_rounds(dv["x"], w, cfg.k, buf, capacity, group, rounds_out=rounds, route=False)
    torch.cuda.synchronize()
    nb = moe.moe_workspace_bytes_rounds(cfg.T, cfg.d, cfg.L, cfg.E, cfg.k, cfg.F, cfg.Fs,
                                        capacity, group)
    U.log(f"[rounds {name}] capacity {capacity} (mean {mean:.1f}), groups of {group}: "
          f"{int(rounds.item())} rounds (oracle {want_rounds}); workspace {nb / 2**20:.1f} MiB "
          f"vs single pass {buf.ws.numel() / 2**20:.1f} MiB")
    assert int(rounds.item()) == want_rounds
    assert torch.equal(buf.y_rows, ref["y"])
    assert torch.equal(buf.out, ref["out"])


def test_rounds_match_the_oracle(cuda):
    cfg, host, dv, w, ro, w32, ref, perm = _setup("hot", cuda)
    rb = U.oracle_forward(cfg, host, "bf16_operands",
                          routing=(ro["topk_idx"], w32.astype(np.float64)))
    buf = moe.LatentMoEBuffers(cfg.T, cfg.d, cfg.L, cfg.E, cfg.k, cfg.F, cfg.Fs, device=cuda)
    buf.topk_idx.copy_(torch.from_numpy(np.asarray(ro["topk_idx"], np.int32)))
    buf.topk_w.copy_(torch.from_numpy(w32))
    moe.forward_rounds(dv["x"], w, cfg.k, buf, 16, 4, route=False)
    torch.cuda.synchronize()
    eo = U.rel_err(U.to_np(buf.out), rb["out"])
    U.log(f"[rounds hot] out vs bf16-operand oracle max/rms {eo[0]:.2e}/{eo[1]:.2e}")
    assert eo[0] <= U.OUT_TOL
