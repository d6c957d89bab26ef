"""LatentMoE layer forward throughput on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config NAME] [--no-cpu-baseline]

One step = one forward pass of the whole layer (moe_route -> moe_permute ->
moe_latent_ffn_forward -> moe_combine, every stage a libmoe HIP kernel) over
one batch of seeded synthetic input already resident in HBM.  Prints one JSON
line: tokens/s of the timed steps, the roofline of the dominant kernel (the
grouped gate/up GEMM) measured with HIP events recorded by the library around
that kernel on the stream it runs on, per-kernel average times, and the CPU
oracle timed on a bounded sample of the same workload.

Default workload: the MAI-Base-1-shaped layer at T=32,768 tokens (d=6,656,
latent 3,072, 512 experts, top-8, SwiGLU width 10,240; bf16 operands, fp32
accumulation; ~512 routed rows per expert, compute-bound), all 512 experts
resident (~97 GB of expert weights).  The same layer at T=4,096 tokens
(small batch, bound by streaming the weights from HBM) is timed in the same
run on the same weights (its x is the first 4,096 tokens) and reported under
"secondary", with its own roofline.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12          # MI355X HBM3E, bytes/s
MFMA_BF16_PEAK = 2.5e15    # MI355X dense bf16 MFMA, FLOP/s
MFMA_FP8_PEAK = 5.0e15     # MI355X dense fp8 MFMA, FLOP/s
METRIC = "LatentMoE layer fwd tokens/sec on 1 MI355X; % bf16 MFMA peak / % HBM BW"
KERNEL_NAMES = ["router_gemm", "router_topk", "permute", "latent_down", "gate_up",
                "expert_down", "combine", "latent_up"]
DOMINANT = "gate_up"
# Sources that define the dominant kernel; stored counter readings are only
# valid for the code they were taken on.
DOMINANT_SOURCES = ["mixture_experts_layer_moe_amd/csrc/gemm.hpp",
                    "mixture_experts_layer_moe_amd/csrc/expert.hip"]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--config", default=None,
                   help="workload (default: base1_compute; base1_ep8 with --backward; "
                        "base2_ep8 is the backward's Base-2 share, with the shared expert)")
    p.add_argument("--secondary", default="base1_small_batch",
                   help="a second workload with the same weights and a smaller batch, timed in "
                        "the same run and reported under 'secondary' ('none' to skip)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--fp8", action="store_true",
                   help="routed experts' GEMMs in FP8 E4M3 with delayed scaling (not the headline "
                        "configuration, which is bf16)")
    p.add_argument("--capacity", type=float, default=0.0,
                   help="multi-round dropless experts: per-expert capacity per round as a "
                        "multiple of the mean rows per expert (0: single pass)")
    p.add_argument("--group-size", type=int, default=8,
                   help="experts sharing capacity in the multi-round schedule")
    p.add_argument("--balancer", action="store_true",
                   help="route with moe_route_ex: the router bias steers the selection only "
                        "(loss-free balancer) and the per-expert probability sums of the "
                        "load-balancing loss are computed (bf16 single-pass forward)")
    p.add_argument("--backward", action="store_true",
                   help="time the backward pass (moe_backward) after one forward pass instead "
                        "of the forward (default workload then: base1_ep8)")
    p.add_argument("--grad-fp8", action="store_true",
                   help="with --backward: the experts' data-gradient GEMMs in FP8 (E5M2 "
                        "gradients, E4M3 weights, delayed scaling)")
    p.add_argument("--rounding", choices=["sr", "rne"], default="sr",
                   help="backward gradient casts: stochastic (the pages' choice) or nearest")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a plain device copy of known size (for HBM counter scaling)")
    return p.parse_args()


class HipEvents:
    """hipEvent_t handles from the HIP runtime torch has loaded (same process runtime)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        e = ctypes.c_void_p()
        assert self.hip.hipEventCreate(ctypes.byref(e)) == 0
        return e.value

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if rc != 0:
            self.hip.hipGetLastError()   # clear it: a later runtime check must not report it
            return None                  # a kernel that this path does not launch
        return ms.value

    def destroy(self, e):
        self.hip.hipEventDestroy(ctypes.c_void_p(e))


def sources_digest():
    h = hashlib.sha256()
    for rel in DOMINANT_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(config_name):
    """HBM bytes per launch of the dominant kernel from committed rocprofv3
    counter readings, if they were taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"{DOMINANT}_{config_name}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("sources_sha256_16") != sources_digest():
        return None
    return rec.get("traffic_bytes_per_launch")


def dominant_work(cfg, counts, esize=2):
    """Algorithmic FLOPs and bytes of one launch of the grouped gate/up GEMM:
    2 GEMMs of 2*rows*L*F FLOPs; bytes = gate+up weights of every expert that
    received a row (each read once) + the latent rows z (each token's row
    once: the GEMM gathers it k times, the algorithm needs it once) + H out,
    all of esize bytes per value (2: bf16, 1: FP8 E4M3)."""
    import numpy as np
    touched = int(np.count_nonzero(counts))
    rows = cfg.T * cfg.k
    flops = 4.0 * rows * cfg.L * cfg.F
    nbytes = (touched * 2.0 * cfg.F * cfg.L + cfg.T * cfg.L + rows * cfg.F) * esize
    return flops, nbytes, touched


def layer_bytes(cfg, touched, esize=2):
    """Algorithmic HBM bytes of the whole layer: weights touched once (expert
    weights esize bytes per value), x in, fp32 out (intermediates excluded)."""
    T, d, L, E, F, Fs = cfg.T, cfg.d, cfg.L, cfg.E, cfg.F, cfg.Fs
    w = touched * 3.0 * F * L * esize + 2.0 * d * L * 2 + E * d * 4.0 + 3.0 * d * Fs * 2
    return w + T * d * 2.0 + T * d * 4.0


def cpu_baseline(cfg, n_tok=4096, n_exp=192, rows_budget=12288, seed=0, fp8=False, reps=3):
    """The oracle (float64 numpy, as it stands) on a bounded sample of the
    workload, extrapolated to tokens/s of the whole layer:
      router + permutation over all T tokens (timed in full),
      latent down, combine and up-projection on n_tok tokens (x T/n_tok),
      randomly drawn experts' SwiGLU FFNs on their routed rows, up to n_exp
      experts or rows_budget rows (x all T*k rows / the rows done), each
      timed reps times (the mean is used: ~10-20 s of timed work on the
      Base-1 shapes: 192 experts at T = 4,096, ~24 at T = 32,768).
    Input generation is not timed.  fp8: the experts in the oracle's
    fp8_operands mode (scales from the sample's own ranges)."""
    import numpy as np
    import oracle
    from moe_synth import gen
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    x = gen.host_tensor_f64(cfg, "x")
    w_r = gen.router_weights(cfg).astype(np.float64)
    b = gen.router_bias(cfg)
    b = None if b is None else b.astype(np.float64)
    w_dn = gen.host_tensor_f64(cfg, "w_dn")
    w_up = gen.host_tensor_f64(cfg, "w_lat_up")
    shared = None
    if cfg.Fs:
        shared = tuple(gen.host_tensor_f64(cfg, n) for n in ("ws_gate", "ws_up", "ws_down"))
    t0 = time.perf_counter()
    r = oracle.route(x, w_r, b, cfg.k)
    p = oracle.permute(r["topk_idx"], cfg.E)
    t_route = time.perf_counter() - t0
    rng = np.random.default_rng(seed)
    toks = np.sort(rng.choice(cfg.T, size=min(n_tok, cfg.T), replace=False))
    t0 = time.perf_counter()
    z = oracle.latent_down(x[toks], w_dn, "bf16_operands")
    ys = np.stack([z] * cfg.k, axis=1).reshape(-1, cfg.L)     # stand-in expert rows, same shapes
    ar = np.arange(len(toks) * cfg.k).reshape(len(toks), cfg.k)
    c = oracle.combine(ys, r["topk_w"][toks], ar)
    out = oracle.latent_up(c, w_up, "bf16_operands")
    if shared is not None:
        out = out + oracle.shared_expert(x[toks], *shared, mode="bf16_operands")
    t_tok = time.perf_counter() - t0
    counts = p["expert_counts"]
    nonempty = np.nonzero(counts)[0]
    order = rng.permutation(nonempty)
    csum = np.cumsum(counts[order])
    n_take = min(n_exp, int(np.searchsorted(csum, rows_budget)) + 1, order.size)
    sample = order[:n_take]
    t_exp = 0.0
    t_gen = 0.0
    rows_done = 0
    for e in sample:
        tg = time.perf_counter()
        wts = gen.expert_weights_f64(cfg, int(e))
        t_gen += time.perf_counter() - tg
        a, bnd = int(p["expert_offsets"][e]), int(p["expert_offsets"][e + 1])
        zr = oracle.latent_down(x[p["row_token"][a:bnd]], w_dn, "bf16_operands")
        sc = None
        if fp8:
            s_w = [np.float32(448.0) / np.float32(np.abs(wt).max()) for wt in wts]
            s_z = np.float32(448.0) / np.float32(np.abs(zr).max())
            sc = (s_z, s_w[0], s_w[1], np.float32(1.0), s_w[2])
            h = oracle.swiglu_activation(zr, wts[0], wts[1], "fp8_operands", sc)
            sc = (s_z, s_w[0], s_w[1], np.float32(448.0) / np.float32(np.abs(h).max()), s_w[2])
        t0 = time.perf_counter()
        for _ in range(reps):
            oracle.swiglu_expert(zr, *wts, mode="fp8_operands" if fp8 else "bf16_operands",
                                 fp8=sc)
        t_exp += (time.perf_counter() - t0) / reps
        rows_done += bnd - a
        del wts
    # experts scale by rows (their cost is linear in the rows they receive)
    t_exp_total = t_exp * (cfg.T * cfg.k) / max(rows_done, 1)
    total = t_route + t_tok * cfg.T / len(toks) + t_exp_total
    return {
        "value": cfg.T / total, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
        "sample": (f"float64 numpy oracle{' (experts in fp8_operands mode)' if fp8 else ''}: "
                   f"router + permutation over all {cfg.T} tokens "
                   f"({t_route:.2f} s), latent down/combine/up on {len(toks)} tokens "
                   f"({t_tok:.2f} s, scaled x{cfg.T / len(toks):.0f}), SwiGLU experts on "
                   f"{len(sample)} sampled experts = {rows_done} routed rows ({t_exp:.2f} s, "
                   f"mean of {reps} timings, scaled by rows to all {cfg.T * cfg.k}); "
                   f"{t_route + t_tok + reps * t_exp:.1f} s of timed oracle work, extrapolated "
                   f"{total:.1f} s per forward pass (weight generation, {t_gen:.0f} s, not "
                   f"timed)"),
    }


BWD_KERNELS = ["bwd_up", "bwd_combine", "bwd_dgrad", "bwd_wgrad", "bwd_latent", "bwd_router"]


def backward_flops(cfg):
    """(model, executed) FLOPs of one backward pass.  Model: twice the
    forward's (the data and the weight gradient of every GEMM), the count MFU
    uses on the pages (recomputation excluded).  Executed adds the
    recomputation of z (2TdL), of the experts' gate/up (4TkLF) and of the
    shared expert's gate/up (4TdFs)."""
    T, d, L, E, k, F, Fs = cfg.T, cfg.d, cfg.L, cfg.E, cfg.k, cfg.F, cfg.Fs
    model = 2.0 * (2.0 * T * d * E + 4.0 * T * d * L + 6.0 * T * k * L * F + 6.0 * T * d * Fs)
    return model, model + 2.0 * T * d * L + 4.0 * T * k * L * F + 4.0 * T * d * Fs


def bench_backward(args, cfg, dev):
    """Time K backward passes (after one forward pass that keeps the router
    logits) of the layer on seeded synthetic inputs and output gradient: the
    single pass (moe_backward, or moe_backward_fp8), or with --capacity the
    multi-round schedule (moe_backward_rounds); a layer with a shared expert
    adds moe_shared_backward."""
    import numpy as np
    import torch

    import mixture_experts_layer_moe_amd as moe
    from moe_synth import device
    if args.capacity > 0 and args.grad_fp8:
        print("--capacity with --backward runs the bf16 gradients only", file=sys.stderr)
        sys.exit(2)
    print(f"[bench] backward: {cfg.description}; generating inputs on the GPU", file=sys.stderr,
          flush=True)
    dv = device.device_inputs(cfg, dev)
    w = moe.LatentMoEWeights(dv["w_router"], dv["b_router"], dv["w_dn"], dv["w_gate"], dv["w_up"],
                             dv["w_down"], dv["w_lat_up"], dv.get("ws_gate"), dv.get("ws_up"),
                             dv.get("ws_down"))
    buf = moe.LatentMoEBuffers(cfg.T, cfg.d, cfg.L, cfg.E, cfg.k, cfg.F, cfg.Fs, device=dev,
                               keep_logits=True)
    moe.forward(dv["x"], w, cfg.k, buf)
    wt = moe.backward_prepare(w)
    rounds_info = None
    grads = moe.LatentMoEGrads(cfg.T, cfg.d, cfg.L, cfg.E, cfg.k, cfg.F, device=dev,
                               bias=dv["b_router"] is not None, fp8=args.grad_fp8, Fs=cfg.Fs,
                               workspace=args.capacity <= 0)
    g = torch.Generator(device=dev)
    g.manual_seed(1234)
    g_out = torch.randn((cfg.T, cfg.d), generator=g, dtype=torch.float32, device=dev)
    rounding = moe.MOE_ROUND_STOCHASTIC if args.rounding == "sr" else moe.MOE_ROUND_NEAREST
    if args.grad_fp8:
        # E4M3 transposed expert weights (the forward's scales) and the
        # gradients' delayed scaling; warmup steps fill the amax history
        wt8 = moe.quantize_transposed(wt, moe.quantize_experts(w))
        gsc = moe.Fp8GradScaling(device=dev)
        step = lambda i: moe.backward_fp8(dv["x"], w, wt, wt8, buf, g_out, grads, gsc,  # noqa: E731
                                          rounding=rounding, seed=i)
    elif args.capacity > 0:
        cap = max(1, int(round(args.capacity * cfg.T * cfg.k / cfg.E)))
        gs = min(args.group_size, cfg.E)
        nb = moe.moe_workspace_bytes_backward_rounds(cfg.T, cfg.d, cfg.L, cfg.E, cfg.k, cfg.F,
                                                     cap, gs)
        if cfg.Fs:
            nb = max(nb, moe.moe_workspace_bytes(moe.MOE_OP_SHARED_BACKWARD, cfg.T, cfg.d, cfg.L,
                                                 cfg.E, cfg.k, cfg.F, cfg.Fs))
        ws_r = torch.empty(nb, dtype=torch.uint8, device=dev)
        rounds_info = {"capacity": cap, "group_size": gs, "workspace_bytes": nb,
                       "single_pass_workspace_bytes": moe.moe_workspace_bytes(
                           moe.MOE_OP_BACKWARD, cfg.T, cfg.d, cfg.L, cfg.E, cfg.k, cfg.F)}
        step = lambda i: moe.backward_rounds(dv["x"], w, wt, buf, g_out, grads,  # noqa: E731
                                             cap, gs, ws_rounds=ws_r, rounding=rounding, seed=i)
    else:
        step = lambda i: moe.backward(dv["x"], w, wt, buf, g_out, grads,  # noqa: E731
                                      rounding=rounding, seed=i)
    bwd_kernels = BWD_KERNELS + (["bwd_shared"] if cfg.Fs else [])
    torch.cuda.synchronize()
    print(f"[bench] warmup {args.warmup} backward steps", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    hip = HipEvents()
    ev = {name: [(hip.create(), hip.create()) for _ in range(args.steps)] for name in bwd_kernels}
    print(f"[bench] timing {args.steps} backward steps", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for i in range(args.steps):
        for name in bwd_kernels:
            moe.moe_set_kernel_events(name, *ev[name][i])
        step(args.warmup + i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for name in bwd_kernels:
        moe.moe_set_kernel_events(name, None, None)
    kern_ms = {}
    for n in bwd_kernels:
        vals = [hip.elapsed_ms(a, b) for a, b in ev[n]]
        if all(v is not None for v in vals):     # groups this path records
            kern_ms[n] = float(np.mean(vals))
    for pairs in ev.values():
        for a, b in pairs:
            hip.destroy(a)
            hip.destroy(b)
    elapsed = t1 - t0
    ms = elapsed / args.steps * 1e3
    model, executed = backward_flops(cfg)
    # the experts' data-gradient group (gate/up recompute, dh + SwiGLU
    # backward, the rows' latent gradient): 10 T k L F executed FLOPs; on the
    # multi-round schedule the group brackets every round, whose expert
    # weight gradients (6 T k L F) it then includes
    tkLF = cfg.T * cfg.k * cfg.L * cfg.F
    wgrad_flops = 6.0 * tkLF
    rounds = rounds_info is not None
    dgrad_flops = (16.0 if rounds else 10.0) * tkLF
    # its time at peak: all bf16, or (FP8 data gradients) the gate/up
    # recompute (4 T k L F) at the bf16 peak and dh + dz rows (6 T k L F) at
    # the FP8 peak
    dgrad_peak_s = (4.0 * tkLF / MFMA_BF16_PEAK + 6.0 * tkLF / MFMA_FP8_PEAK) if args.grad_fp8 \
        else dgrad_flops / MFMA_BF16_PEAK
    dgrad_s = kern_ms["bwd_dgrad"] * 1e-3
    line = {
        "metric": "LatentMoE layer bwd tokens/sec on 1 MI355X; % bf16 MFMA peak",
        "value": cfg.T * args.steps / elapsed, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16, fp8 data gradients" if args.grad_fp8 else "bf16", "data": "synthetic",
        "config": {"workload": cfg.description, "T": cfg.T, "d": cfg.d, "latent": cfg.L,
                   "experts": cfg.E, "top_k": cfg.k, "ffn": cfg.F, "shared_ffn": cfg.Fs,
                   "seed": cfg.seed, "rounding": args.rounding, "grad_fp8": bool(args.grad_fp8),
                   "multi_round": rounds_info},
        "roofline": {"bound": "mfma", "kernel": "expert data-gradient group (gate/up "
                     "recompute, dh + SwiGLU backward, dz rows" +
                     ("; every round, with its expert weight gradients)" if rounds else ")"),
                     "achieved": dgrad_flops / dgrad_s / 1e12,
                     "peak": dgrad_flops / dgrad_peak_s / 1e12, "unit": "TFLOP/s",
                     "frac": dgrad_peak_s / dgrad_s,
                     "traffic": None},
        "layer": {"model_flops": model, "executed_flops": executed,
                  "mfma_frac_model": model / (ms * 1e-3) / MFMA_BF16_PEAK,
                  "mfma_frac_executed": executed / (ms * 1e-3) / MFMA_BF16_PEAK,
                  "expert_wgrad_tflops": (wgrad_flops / (kern_ms["bwd_wgrad"] * 1e-3) / 1e12
                                          if "bwd_wgrad" in kern_ms else None),
                  "kernels_ms": {k: round(v, 4) for k, v in kern_ms.items()}},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def same_weights(a, b):
    """Two workloads whose weights are the same tensors (same shapes, seed and
    router bias): the generator keys every tensor by (seed, tensor), so their
    weights are bit-identical and x of the smaller batch is the first rows of
    the larger one's."""
    return (a.d, a.L, a.E, a.k, a.F, a.Fs, a.zipf_bias, a.seed) == \
        (b.d, b.L, b.E, b.k, b.F, b.Fs, b.zipf_bias, b.seed)


def time_forward(args, cfg, w, x, dev, w8=None):
    """Warm up, then time args.steps forward passes of workload cfg on one
    stream with inputs resident in HBM; per-kernel HIP events are recorded by
    the library around each kernel on that stream.  Returns the result
    fields of one workload (without the CPU baseline)."""
    import numpy as np
    import torch

    import mixture_experts_layer_moe_amd as moe
    buf = moe.LatentMoEBuffers(cfg.T, cfg.d, cfg.L, cfg.E, cfg.k, cfg.F, cfg.Fs, device=dev)
    step = lambda: moe.forward(x, w, cfg.k, buf)  # noqa: E731
    rounds_info = None
    if args.capacity > 0:
        cap = max(1, int(round(args.capacity * cfg.T * cfg.k / cfg.E)))
        gs = min(args.group_size, cfg.E)
        nb = moe.moe_workspace_bytes_rounds(cfg.T, cfg.d, cfg.L, cfg.E, cfg.k, cfg.F, cfg.Fs, cap,
                                            gs)
        ws_r = torch.empty(nb, dtype=torch.uint8, device=dev)
        rounds_t = torch.zeros(1, dtype=torch.int32, device=dev)
        rounds_info = {"capacity": cap, "group_size": gs, "workspace_bytes": nb}
        step = lambda: moe.forward_rounds(x, w, cfg.k, buf, cap, gs, ws_rounds=ws_r,  # noqa: E731
                                          rounds_out=rounds_t)
    if args.balancer:
        prob_sum = torch.zeros(cfg.E, dtype=torch.float32, device=dev)

        def step():
            moe.moe_route_ex(x, w.w_router, w.b_router, moe.MOE_BIAS_SELECTION, cfg.k,
                             buf.topk_idx, buf.topk_w, prob_sum=prob_sum, ws=buf.ws)
            moe.forward(x, w, cfg.k, buf, route=False)
    if w8 is not None:
        scaling = moe.Fp8Scaling(hist_len=1024, device=dev)
        step = lambda: moe.forward_fp8(x, w, w8, cfg.k, buf, scaling)  # noqa: E731
    torch.cuda.synchronize()
    print(f"[bench] {cfg.name}: warmup {args.warmup} steps", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    hip = HipEvents()
    ev = {name: [(hip.create(), hip.create()) for _ in range(args.steps)] for name in KERNEL_NAMES}
    print(f"[bench] {cfg.name}: timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        for name in KERNEL_NAMES:
            moe.moe_set_kernel_events(name, *ev[name][i])
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for name in KERNEL_NAMES:
        moe.moe_set_kernel_events(name, None, None)
    kern_ms = {}
    for name in KERNEL_NAMES:
        t = [hip.elapsed_ms(a, b) for a, b in ev[name]]
        kern_ms[name] = None if any(v is None for v in t) else float(np.mean(t))
    for pairs in ev.values():
        for a, b in pairs:
            hip.destroy(a)
            hip.destroy(b)

    elapsed = t1 - t0
    ms_per_step = elapsed / args.steps * 1e3
    counts = buf.expert_counts.cpu().numpy()
    fp8 = w8 is not None
    esize = 1 if fp8 else 2
    mfma_peak = MFMA_FP8_PEAK if fp8 else MFMA_BF16_PEAK
    flops, nbytes, touched = dominant_work(cfg, counts, esize)
    dom_s = kern_ms[DOMINANT] * 1e-3
    if flops / nbytes < mfma_peak / HBM_PEAK:
        roof = {"bound": "hbm", "achieved": nbytes / dom_s / 1e9, "peak": HBM_PEAK / 1e9,
                "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": flops / dom_s / 1e12, "peak": mfma_peak / 1e12,
                "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = stored_traffic(cfg.name + ("_fp8" if fp8 else ""))
    roof["kernel"] = ("grouped gate/up GEMM + SwiGLU (gemm_kernel GROUPED GATHER EPI_SWIGLU"
                      + (" FP8 E4M3, E4M3 output)" if fp8 else ")"))
    roof["algorithmic_per_launch"] = {"flops": flops, "bytes": nbytes, "experts_touched": touched,
                                      "mean_launch_ms": kern_ms[DOMINANT]}

    step_s = ms_per_step * 1e-3
    lb = layer_bytes(cfg, touched, esize)
    lf = cfg.flops()
    # the whole layer against the roofline of its own arithmetic intensity
    layer_bound = "hbm" if lf / lb < mfma_peak / HBM_PEAK else "mfma"
    layer = {
        "bound": layer_bound,
        "frac": (lb / step_s / HBM_PEAK) if layer_bound == "hbm" else (lf / step_s / mfma_peak),
        "mfma_frac": lf / step_s / mfma_peak,
        "hbm_frac": lb / step_s / HBM_PEAK,
        "algorithmic": {"flops": lf, "bytes": lb},
        "kernels_ms": {k: (None if v is None else round(v, 4)) for k, v in kern_ms.items()},
    }
    res = {"workload": cfg.description, "value": cfg.T * args.steps / elapsed,
           "ms_per_step": ms_per_step, "roofline": roof, "layer": layer,
           "config": {"workload": cfg.description, "name": cfg.name, "T": cfg.T, "d": cfg.d,
                      "latent": cfg.L, "experts": cfg.E, "top_k": cfg.k, "ffn": cfg.F,
                      "shared_ffn": cfg.Fs, "seed": cfg.seed}}
    if args.balancer:
        res["config"]["router"] = ("moe_route_ex: selection-only bias (loss-free balancer), "
                                   "per-expert probability sums")
    if rounds_info is not None:
        rounds_info["rounds"] = int(rounds_t.item())
        res["config"]["multi_round"] = rounds_info
        res["roofline"] = None   # the gate/up events bracket every round of both GEMMs
    del buf
    return res


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)
    import torch

    import mixture_experts_layer_moe_amd as moe
    from moe_synth import CONFIGS, device

    if args.config is None:
        args.config = "base1_ep8" if args.backward else "base1_compute"
    cfg = CONFIGS[args.config]
    dev = torch.device("cuda:0")
    if args.backward:
        return bench_backward(args, cfg, dev)
    if args.capacity > 0 and args.fp8:
        print("--capacity runs the bf16 experts only", file=sys.stderr)
        sys.exit(2)
    if args.balancer and (args.fp8 or args.capacity > 0):
        print("--balancer runs the bf16 single-pass forward only", file=sys.stderr)
        sys.exit(2)
    sec = None
    if args.secondary and args.secondary != "none":
        sec = CONFIGS[args.secondary]
        if sec.name == cfg.name:
            sec = None     # the workload itself: nothing more to time
        elif not same_weights(cfg, sec) or sec.T > cfg.T:
            print(f"[bench] secondary workload {sec.name} does not share {cfg.name}'s weights "
                  f"and batch; not timed", file=sys.stderr)
            sec = None
    print(f"[bench] {cfg.description}; generating inputs on the GPU", file=sys.stderr, flush=True)
    dv = device.device_inputs(cfg, dev)
    w = moe.LatentMoEWeights(dv["w_router"], dv["b_router"], dv["w_dn"], dv["w_gate"], dv["w_up"],
                             dv["w_down"], dv["w_lat_up"], dv.get("ws_gate"), dv.get("ws_up"),
                             dv.get("ws_down"))
    x = dv["x"]
    w8 = None
    if args.fp8:
        # weights quantized once (448 / amax per expert matrix); the bf16
        # expert weights are then dropped; activation scales are delayed:
        # each step uses the history of the previous steps' maxima
        w8 = moe.quantize_experts(w)
        torch.cuda.synchronize()
        w.w_gate = w.w_up = w.w_down = None
        for n in ("w_gate", "w_up", "w_down"):
            del dv[n]
        torch.cuda.empty_cache()
    torch.cuda.synchronize()

    if args.copy_calibration:
        src = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            device.calibration_copy(src, dst)   # one dispatch: 1 GiB read + 1 GiB written
        torch.cuda.synchronize()
        del src, dst

    main_res = time_forward(args, cfg, w, x, dev, w8)
    sec_res = None
    if sec is not None:
        # the smaller batch: the first sec.T tokens (bit-identical to that
        # workload's own x), same weights, its own buffers and timing
        sec_res = time_forward(args, sec, w, x[:sec.T], dev, w8)

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(cfg, fp8=args.fp8)

    line = {
        "metric": METRIC, "value": main_res["value"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": main_res["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8_e4m3 (expert GEMMs; bf16 latent projections)" if args.fp8 else "bf16",
        "data": "synthetic",
        "config": main_res["config"],
        "roofline": main_res["roofline"], "layer": main_res["layer"], "cpu_baseline": cpu,
    }
    if sec_res is not None:
        line["secondary"] = {k: sec_res[k] for k in ("workload", "value", "ms_per_step",
                                                     "roofline", "layer", "config")}
        line["secondary"]["unit"] = "tokens/s"
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
