"""GPU parity at the full workload sizes, in the launch configuration bench.py
times (LatentMoEBuffers + forward, all experts resident in HBM).

* routing: every token, against the oracle's float64/fp32 router, with the
  near-tie rule (swaps only where the oracle's logit gap is < 1e-4);
* permutation arrays: bit-exact over all T*k assignments when the routing has
  no swap (else checked for validity);
* expert rows (the grouped GEMMs at scale): y_rows of the 8 experts with the
  most rows and of 64 more experts whose last M tile is ragged, on the first
  and last row of every 32-row block of each (every M tile's first and last
  row whatever the tile height) plus random rows, against the oracle's
  SwiGLU expert on the same tokens (bf16_operands), max|err|/RMS <= 2e-2 per
  expert; the imbalanced workload uses 48 experts, so all of them;
* combine and up-projection: out of 256 random tokens against the oracle's
  fixed-order combine and up-projection of the GPU's expert rows and gate
  weights (plus the oracle's shared expert), <= 2e-2;
* end to end: out of 8 tokens through the oracle's per-token definition on
  its own routing (router replay), <= 2e-2;
* the multi-round schedule (imbalanced workload, capacity 2x the mean rows
  per expert, groups of 8): its round count equals the oracle's schedule,
  its expert rows are bitwise those of the single pass, and the sampled
  rows match the oracle;
* FP8 experts (small batch, compute, imbalanced, Base-2): the per-expert
  weight scales bit-exact; for the sampled rows of the 8 hottest and 24
  ragged experts, the E4M3 codes of z and h
  equal the oracle's except valid roundings within the accumulation-error
  interval; tokens whose z codes flipped are recomputed by the oracle from
  the GPU's (validated) z codes; y_rows within 2e-2 of RMS of the
  fp8_operands oracle beyond the bound of what the flipped h codes carry;
  combine and up-projection as for bf16.
Expert weights are read from the generator-filled device tensors (see
tests/fullsize_util.py); each read is checked against the host generator.
"""
import numpy as np
import pytest
import torch

import mixture_experts_layer_moe_amd as moe
import oracle
from moe_synth import CONFIGS, device, gen
from tests import fullsize_util as FU
from tests import gpu_util as U

pytestmark = [pytest.mark.gpu, pytest.mark.fullsize]

FULL = ["base1_small_batch", "base1_compute", "base1_imbalanced", "base2", "base1_f5120"]
FULL_FP8 = ["base1_small_batch", "base1_compute", "base1_imbalanced", "base2"]
# multi-round schedule at full size: capacity as a multiple of the mean rows per expert
ROUNDS_CAP = {"base1_imbalanced": 2, "base2": 0.5}
N_HOT, N_RAGGED, N_TOK, N_E2E = 8, 64, 256, 8
N_RAGGED_FP8 = 24   # the oracle's E4M3 rounding of each expert's weights costs ~1 s


@pytest.fixture(scope="module")
def cuda():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.load()
    return torch.device("cuda:0")


_res = {}


def _workload(name, cuda):
    """Device inputs and the host-side oracle routing of one workload (one
    workload resident at a time)."""
    if _res.get("name") == name:
        return _res
    _res.clear()
    torch.cuda.empty_cache()
    cfg = CONFIGS[name]
    U.log(f"[full {name}] T={cfg.T} d={cfg.d} L={cfg.L} E={cfg.E} k={cfg.k} F={cfg.F} "
          f"Fs={cfg.Fs}: generating inputs on the GPU")
    dv = device.device_inputs(cfg, cuda)
    w = moe.LatentMoEWeights(dv["w_router"], dv["b_router"], dv["w_dn"], dv["w_gate"], dv["w_up"],
                             dv["w_down"], dv["w_lat_up"], dv.get("ws_gate"), dv.get("ws_up"),
                             dv.get("ws_down"))
    U.log(f"[full {name}] oracle routing over all {cfg.T} tokens")
    x = gen.host_tensor_f64(cfg, "x")
    b = gen.router_bias(cfg)
    ro = oracle.route(x, gen.router_weights(cfg).astype(np.float64),
                      None if b is None else b.astype(np.float64), cfg.k)
    host = {"x": x, "w_dn": gen.host_tensor_f64(cfg, "w_dn"),
            "w_lat_up": gen.host_tensor_f64(cfg, "w_lat_up")}
    if cfg.Fs:
        host["shared"] = tuple(gen.host_tensor_f64(cfg, n) for n in ("ws_gate", "ws_up", "ws_down"))
    _res.update(name=name, cfg=cfg, dv=dv, w=w, ro=ro, host=host)
    return _res


def _z_of(cfg, host):
    return lambda toks: FU.z_rows(cfg, host["x"], host["w_dn"], toks)


def _shared_out(cfg, host, toks):
    if not cfg.Fs:
        return None
    return oracle.shared_expert(host["x"][toks], *host["shared"], mode="bf16_operands")


def _check_routing(tag, cfg, dv, buf, ro):
    """Routing over all tokens and the permutation; returns the GPU's arrays
    and the tokens with an allowed near-tie swap."""
    g = {n: getattr(buf, n).cpu().numpy() for n in
         ("topk_idx", "topk_w", "expert_counts", "expert_offsets", "row_token", "assign_row")}
    # the FP32 logits themselves, from a second routing call (same kernels)
    logits = torch.empty((cfg.T, cfg.E), dtype=torch.float32, device=buf.topk_idx.device)
    idx2 = torch.empty_like(buf.topk_idx)
    w2 = torch.empty_like(buf.topk_w)
    moe.moe_route(dv["x"], dv["w_router"], dv["b_router"], cfg.k, idx2, w2, logits_out=logits,
                  ws=buf.ws)
    torch.cuda.synchronize()
    assert torch.equal(idx2, buf.topk_idx) and torch.equal(w2, buf.topk_w)
    lerr = float(np.abs(logits.cpu().numpy() - ro["logits"]).max())
    del logits, idx2, w2
    U.log(f"[{tag}] max |logit err| = {lerr:.3e} (bound {U.LOGIT_ATOL:.1e})")
    assert lerr <= U.LOGIT_ATOL
    swaps = U.routing_swaps(g["topk_idx"], ro["topk_idx"], ro["logits"])
    wr = U.check_topk_w(g["topk_idx"], g["topk_w"], ro["probs"])
    U.log(f"[{tag}] near-tie swaps: {len(swaps)}; topk_w max rel err {wr:.2e}")
    assert len(swaps) <= max(2, cfg.T // 1000)
    if len(swaps) == 0:
        p = oracle.permute(ro["topk_idx"], cfg.E)
        for n in ("expert_counts", "expert_offsets", "row_token", "assign_row"):
            np.testing.assert_array_equal(g[n].reshape(p[n].shape), p[n], err_msg=n)
        U.log(f"[{tag}] permutation bit-exact over {cfg.T * cfg.k} assignments; experts used "
              f"{int(np.count_nonzero(p['expert_counts']))}, max rows "
              f"{int(p['expert_counts'].max())}")
    else:
        U.check_perm_valid(g["topk_idx"], cfg.E, g["expert_counts"], g["expert_offsets"],
                           g["row_token"], g["assign_row"])
    return g, swaps


def _check_rows_and_out(tag, cfg, host, buf, g, experts, rng):
    hot, other = FU.choose_experts(g["expert_counts"], N_HOT, N_RAGGED, rng)
    chosen = np.concatenate([hot, other])
    n_rows, n_blk, worst = FU.check_expert_rows(tag, cfg, buf.y_rows, g["expert_offsets"],
                                                g["row_token"], experts, chosen,
                                                _z_of(cfg, host), rng)
    U.log(f"[{tag}] expert rows: {len(hot)} hottest ({g['expert_counts'][hot].tolist()} rows) + "
          f"{len(other)} more, {n_rows} rows over all {n_blk} of their 32-row blocks "
          f"(every M tile's first and last row): y max|err|/RMS {worst:.2e}")
    toks = np.sort(rng.choice(cfg.T, size=min(N_TOK, cfg.T), replace=False))
    ec = FU.check_combine_up(tag, buf.y_rows, g["topk_w"], g["assign_row"], buf.out, toks,
                             host["w_lat_up"], _shared_out(cfg, host, toks))
    U.log(f"[{tag}] combine + up-projection on {toks.size} tokens: max|err|/RMS {ec:.2e}")
    return chosen


# modes grouped by workload, so each workload's inputs are generated once
CASES = [(n, m) for n in FULL for m in ("bf16", "rounds", "fp8")
         if m == "bf16" or (m == "fp8" and n in FULL_FP8) or (m == "rounds" and n in ROUNDS_CAP)]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,mode", CASES, ids=[f"{n}-{m}" for n, m in CASES])
def test_full_size(cuda, name, mode):
    {"bf16": _full_bf16, "rounds": _full_rounds, "fp8": _full_fp8}[mode](cuda, name)


def _full_bf16(cuda, name):
    r = _workload(name, cuda)
    cfg, dv, w, ro, host = r["cfg"], r["dv"], r["w"], r["ro"], r["host"]
    buf = moe.LatentMoEBuffers(cfg.T, cfg.d, cfg.L, cfg.E, cfg.k, cfg.F, cfg.Fs, device=cuda)
    U.log(f"[full {name}] forward pass")
    moe.forward(dv["x"], w, cfg.k, buf)
    torch.cuda.synchronize()
    tag = f"full {name}"
    g, swaps = _check_routing(tag, cfg, dv, buf, ro)
    rng = np.random.default_rng(1234)
    experts = FU.DeviceExperts(cfg, dv["w_gate"], dv["w_up"], dv["w_down"])
    chosen = _check_rows_and_out(tag, cfg, host, buf, g, experts, rng)

    # end to end: tokens on the oracle's own routing, per-token definition
    toks, need = FU.choose_tokens(ro["topk_idx"], N_E2E, chosen[:N_HOT], swaps, rng)
    experts = FU.DeviceExperts(cfg, dv["w_gate"], dv["w_up"], dv["w_down"], cache=len(need) + 1)
    ref = oracle.forward_tokens(host["x"][toks], ro["topk_idx"][toks], ro["topk_w"][toks],
                                host["w_dn"], experts, host["w_lat_up"], shared=host.get("shared"),
                                mode="bf16_operands")
    out_rows = buf.out[torch.from_numpy(toks).to(cuda)].cpu().numpy()
    eo = U.rel_err(out_rows, ref["out"])
    U.log(f"[{tag}] end to end on tokens {toks.tolist()} ({len(need)} experts): out max/rms "
          f"{eo[0]:.2e}/{eo[1]:.2e}")
    assert eo[0] <= U.OUT_TOL
    if name == "base1_imbalanced":
        _res["y_single"] = buf.y_rows
        _res["g"] = g


def _full_rounds(cuda, name):
    """The multi-round schedule at full size, groups of 8 experts: on the
    imbalanced workload with a capacity of 2x the mean rows per expert
    (1,024), on Base-2 (with its shared expert) of half the mean (112)."""
    r = _workload(name, cuda)
    cfg, dv, w, ro, host = r["cfg"], r["dv"], r["w"], r["ro"], r["host"]
    tag = f"full rounds {name}"
    buf = moe.LatentMoEBuffers(cfg.T, cfg.d, cfg.L, cfg.E, cfg.k, cfg.F, cfg.Fs, device=cuda)
    cap = int(ROUNDS_CAP[name] * cfg.T * cfg.k // cfg.E)
    group = 8
    rounds = torch.zeros(1, dtype=torch.int32, device=cuda)
    U.log(f"[{tag}] capacity {cap}, groups of {group}: forward")
    moe.forward_rounds(dv["x"], w, cfg.k, buf, cap, group, rounds_out=rounds)
    torch.cuda.synchronize()
    g, _ = _check_routing(tag, cfg, dv, buf, ro)
    want_rounds, _plan = oracle.round_schedule(g["expert_offsets"], cap, group)
    U.log(f"[{tag}] rounds {int(rounds.item())} (oracle schedule {want_rounds})")
    assert int(rounds.item()) == want_rounds and want_rounds >= 2
    if "y_single" in _res:
        same = torch.equal(_res["y_single"], buf.y_rows)
        U.log(f"[{tag}] expert rows bitwise equal to the single pass: {same}")
        assert same
    rng = np.random.default_rng(99)
    experts = FU.DeviceExperts(cfg, dv["w_gate"], dv["w_up"], dv["w_down"])
    _check_rows_and_out(tag, cfg, host, buf, g, experts, rng)


def _full_fp8(cuda, name):
    """The FP8 expert path at full size (quantized weights, delayed scales set
    on the host: s_z = 448 / amax of the oracle's z over all tokens, s_h =
    448 / 16), on sampled rows of the hottest and of ragged experts."""
    from tests.test_gpu_fp8 import _code_flips, _e4m3_table, _encode_e4m3
    r = _workload(name, cuda)
    cfg, dv, w, ro, host = r["cfg"], r["dv"], r["w"], r["ro"], r["host"]
    tag = f"full fp8 {name}"
    U.log(f"[{tag}] quantizing the experts on the GPU")
    w8 = moe.quantize_experts(w)
    torch.cuda.synchronize()
    U.log(f"[{tag}] oracle latent over all tokens")
    z_exact = oracle.latent_down(host["x"], host["w_dn"], "exact")
    z_bf = oracle.round_bf16(z_exact)
    s_z = np.float32(448.0) / np.float32(np.abs(z_bf).max())
    s_h = np.float32(448.0 / 16.0)

    buf = moe.LatentMoEBuffers(cfg.T, cfg.d, cfg.L, cfg.E, cfg.k, cfg.F, cfg.Fs, device=cuda)
    sc = moe.Fp8Scaling(hist_len=1024, device=cuda)
    sc.scale.copy_(torch.tensor([s_z, s_h], dtype=torch.float32))
    U.log(f"[{tag}] forward pass")
    # forward_fp8's launches, with the E4M3 codes of z and h copied out of
    # the workspace before the combine reuses it: the workspace holds z
    # (E4M3, [T, L]) then H (E4M3, [T*k, F], expert order)
    moe.moe_route(dv["x"], w.w_router, w.b_router, cfg.k, buf.topk_idx, buf.topk_w, ws=buf.ws)
    moe.moe_permute(buf.topk_idx, cfg.E, buf.expert_counts, buf.expert_offsets, buf.row_token,
                    buf.assign_row, buf.ws)
    moe.moe_latent_ffn_forward_fp8(dv["x"], w.w_lat_down, buf.expert_offsets, buf.row_token,
                                   w8.w_gate, w8.w_up, w8.w_down, w8.w_scale, sc.scale, w.ws_gate,
                                   w.ws_up, cfg.k, buf.y_rows, buf.hs, sc.amax, buf.ws)
    h_off = (cfg.T * cfg.L + 255) // 256 * 256
    z8_all = buf.ws[:cfg.T * cfg.L].view(cfg.T, cfg.L).clone()
    h8_all = buf.ws[h_off:h_off + cfg.T * cfg.k * cfg.F].view(cfg.T * cfg.k, cfg.F).clone()
    moe.moe_combine(buf.y_rows, buf.topk_w, buf.assign_row, w.w_lat_up, buf.hs, w.ws_down,
                    buf.out, buf.ws)
    torch.cuda.synchronize()
    g, _ = _check_routing(tag, cfg, dv, buf, ro)
    ws_all = w8.w_scale.cpu().numpy().reshape(3, cfg.E)
    rng = np.random.default_rng(4321)
    hot, other = FU.choose_experts(g["expert_counts"], N_HOT, N_RAGGED_FP8, rng)
    experts = FU.DeviceExperts(cfg, dv["w_gate"], dv["w_up"], dv["w_down"])
    tab = _e4m3_table()
    amax = lambda a: np.float32(np.abs(a).max())  # noqa: E731
    n_rows = zflip_tok = hflip = 0
    worst_y = 0.0
    for e in np.concatenate([hot, other]):
        wg, wu, wd = experts[e]
        sg, su, sd = (np.float32(448.0) / amax(wg), np.float32(448.0) / amax(wu),
                      np.float32(448.0) / amax(wd))
        np.testing.assert_array_equal(ws_all[:, e], np.array([sg, su, sd], np.float32))
        a, b = int(g["expert_offsets"][e]), int(g["expert_offsets"][e + 1])
        rows = FU.sample_rows(a, b, rng)
        toks = g["row_token"][rows]
        # z: the GPU's codes must be valid roundings; tokens with a flipped
        # code continue from the GPU's codes (each validated), so that the
        # oracle's h and y follow the same operand
        z8 = z8_all[torch.from_numpy(toks.astype(np.int64)).to(cuda)].cpu().numpy()
        zq = oracle.quantize_e4m3(z_bf[toks], s_z)
        zf = _code_flips(z8, zq, z_exact[toks] * float(s_z))
        z_op = z_bf[toks].copy()
        if zf.size:
            bad_tok = np.unique(zf // cfg.L)
            zflip_tok += bad_tok.size
            codes = z8[bad_tok].astype(np.int64)
            dec = np.where(codes & 0x80, -1.0, 1.0) * tab[np.minimum(codes & 0x7F, 126)]
            z_op[bad_tok] = dec / float(s_z)
        qwg, qwu, qwd = (FU.quantize_e4m3_rows(m, s) for m, s in ((wg, sg), (wu, su), (wd, sd)))
        gg = FU.fp8_matmul_q(z_op, s_z, qwg, sg)
        uu = FU.fp8_matmul_q(z_op, s_z, qwu, su)
        h_ex = oracle.silu(gg) * uu
        h_bf = oracle.round_bf16(h_ex)
        hq = oracle.quantize_e4m3(h_bf, s_h)
        h8 = h8_all[torch.from_numpy(rows.astype(np.int64)).to(cuda)].cpu().numpy()
        hf = _code_flips(h8, hq, h_ex * float(s_h))
        hflip += hf.size
        y_ref = FU.fp8_matmul_q(h_bf, s_h, qwd, sd)
        # bound of what the flipped h codes carry through the down projection
        dy = np.zeros_like(y_ref)
        if hf.size:
            rr, cc = hf // cfg.F, hf % cfg.F
            g8 = h8.ravel()[hf].astype(np.int64) & 0x7F
            o8 = _encode_e4m3(hq.ravel()[hf]).astype(np.int64) & 0x7F
            step = np.abs(tab[np.minimum(g8, 126)] - tab[np.minimum(o8, 126)]) / float(s_h)
            wdq = np.abs(qwd / float(sd))
            for r_, c_, st_ in zip(rr, cc, step):
                dy[r_] += st_ * wdq[:, c_]
        y_gpu = buf.y_rows[torch.from_numpy(rows.astype(np.int64)).to(cuda)].cpu().numpy()
        rms = np.sqrt(np.mean(y_ref ** 2))
        excess = (np.abs(y_gpu - y_ref) - dy).max() / rms
        worst_y = max(worst_y, float(excess))
        assert excess <= U.OUT_TOL, f"[{tag}] expert {e}: y beyond the flip bound {excess:.3e}"
        n_rows += rows.size
    U.log(f"[{tag}] expert rows: {len(hot)} hottest + {len(other)} more, {n_rows} rows; tokens "
          f"with a flipped z code {zflip_tok}, flipped h codes {hflip}; y beyond the flip "
          f"bound max/RMS {worst_y:.2e}")
    toks = np.sort(rng.choice(cfg.T, size=min(N_TOK, cfg.T), replace=False))
    ec = FU.check_combine_up(tag, buf.y_rows, g["topk_w"], g["assign_row"], buf.out, toks,
                             host["w_lat_up"], _shared_out(cfg, host, toks))
    U.log(f"[{tag}] combine + up-projection on {toks.size} tokens: max|err|/RMS {ec:.2e}")
    del buf, w8, z8_all, h8_all
    torch.cuda.empty_cache()
