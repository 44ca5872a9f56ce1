#!/usr/bin/env python3
"""Throughput of the DeepSeekMoE layer (router -> dispatch -> grouped SwiGLU
experts -> combine -> bias update) on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config v3] [--gpus 1]

A step is one moe_forward with update_bias=1 over one batch of T tokens whose
inputs (u, b, weights) are already resident in HBM. K steps are timed between
two device synchronisations; the library's stage events (recorded on the same
stream) give each kernel's average duration. One JSON line goes to stdout;
progress goes to stderr.
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "f32": 157.3}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic(cfg):
    """Bytes and flops each stage must move/do at minimum, per forward."""
    T, d, N, K, Ns, I, Is = cfg.T, cfg.d, cfg.n_routed, cfg.top_k, cfg.n_shared, cfg.inter, cfg.inter_shared
    ex = {"bf16": 2, "fp8": 1, "f32": 4}[cfg.expert_dtype]
    io = {"bf16": 2, "f32": 4}[cfg.in_dtype]
    rt = {"bf16": 2, "f32": 4}[cfg.router_dtype]
    h = 2 if cfg.expert_dtype == "bf16" else 4
    y = 4 if cfg.expert_dtype == "f32" else 2
    R = T * K + Ns * T
    sc = 4.0 / (128 * 128) if cfg.expert_dtype == "fp8" else 0.0
    w13 = (N * 2 * I * d + Ns * 2 * Is * d) * (ex + sc)
    w2 = (N * d * I + Ns * d * Is) * (ex + sc)
    xin = T * d * (1 if cfg.expert_dtype == "fp8" else io)
    st = {
        "route": {"bytes": T * d * io + N * d * rt + T * K * 8, "flops": 2.0 * T * d * N},
        "permute": {"bytes": T * K * 4 + 2 * R * 4, "flops": 0.0},
        "gemm1": {"bytes": w13 + xin + T * K * I * h + Ns * T * Is * h,
                  "flops": 2.0 * d * (T * K * 2 * I + Ns * T * 2 * Is)},
        "gemm2": {"bytes": w2 + (T * K * I + Ns * T * Is) * (1 if cfg.expert_dtype == "fp8" else h) + R * d * y,
                  "flops": 2.0 * d * (T * K * I + Ns * T * Is)},
        "combine": {"bytes": R * d * y + 2 * T * d * io + T * K * 8, "flops": 0.0},
        "bias": {"bytes": N * 12, "flops": 0.0},
    }
    if cfg.expert_dtype == "fp8":
        st["quant_x"] = {"bytes": T * d * (io + 1) + T * d // 128 * 4, "flops": 0.0}
    return st


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_swiglu_v3_hbm_traffic.txt")
GEMM_SOURCES = ["expert_routing_router_amd/csrc/gemm_bf16.hip", "expert_routing_router_amd/csrc/common.h",
                "expert_routing_router_amd/csrc/lds_dma.h"]


def measured_traffic(cfg):
    """HBM bytes per launch of the gate/up GEMM from the committed counter summary
    (FETCH_SIZE and WRITE_SIZE, each scaled by a plain copy's reading), or None when
    the summary is for another workload or the kernel sources changed since."""
    import hashlib
    if cfg.name != "v3" or cfg.T != 8192 or cfg.expert_dtype != "bf16" or not os.path.exists(TRAFFIC_FILE):
        return None
    h = hashlib.sha256()
    for p in GEMM_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    fields = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if ":" in line:
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip().split()[0] if v.strip() else ""
    if fields.get("kernel_source_sha256") != h.hexdigest():
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class HostWeights:
    """The layer's weights drawn once (seeded, host memory), handed to MoELayer
    with the generator's interface and reused by the CPU oracle."""

    def __init__(self, cfg, gen):
        self.gen = gen
        self.w13, self.w2, self.w13s, self.w2s = gen.all_weights(cfg)

    def centroids(self, cfg):
        return self.gen.centroids(cfg)

    def expert_w13(self, cfg, e):
        return self.w13[e]

    def expert_w2(self, cfg, e):
        return self.w2[e]

    def shared_w13(self, cfg, s):
        return self.w13s[s]

    def shared_w2(self, cfg, s):
        return self.w2s[s]


def cpu_baseline(cfg, hw, log_fn):
    """The oracle (unchanged) on one whole step: routing of all T tokens (fp64
    logits, sigmoid, group-limited top-K, gates) and the layer output over all
    tokens (every routed expert over its rows, the shared experts over every
    token). Returns (record, the oracle's route, its fp64 affinities, its output)."""
    import numpy as np
    from oracle import ffn, numerics as nx, routing
    from workloads import gen
    cpu_model = "?"
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "?")
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        cores = max((i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"), default=1)
        blas = ",".join(sorted({i.get("internal_api", "?") for i in info if i.get("user_api") == "blas"}))
    except Exception:
        cores, blas = len(os.sched_getaffinity(0)), "?"
    u = gen.tokens(cfg, 0)
    E = gen.centroids(cfg)
    b = gen.bias_init(cfg)
    t0 = time.perf_counter()
    r, s64, _ = routing.route_tokens(nx.to_f64(u, cfg.in_dtype), nx.to_f64(E, cfg.router_dtype), b, cfg)
    t_route = time.perf_counter() - t0
    t0 = time.perf_counter()
    out = ffn.layer(cfg, u, r.idx, r.gate, hw.w13, hw.w2, hw.w13s, hw.w2s)
    t_ffn = time.perf_counter() - t0
    per_fwd = t_route + t_ffn
    log_fn("cpu oracle: route %.2fs, experts %.2fs -> %.1fs/forward" % (t_route, t_ffn, per_fwd))
    rec = {"value": cfg.T / per_fwd, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
           "sample": "one whole %d-token step (routing of every token, every routed expert over its rows, "
                     "the shared experts over every token), fp64 numpy (BLAS %s, %d threads; %s, %d cores "
                     "available); %.1f s of CPU work"
                     % (cfg.T, blas, cores, cpu_model, len(os.sched_getaffinity(0)), per_fwd)}
    return rec, r, s64, out


def parity_line(cfg, hw, u, r, s64, out_ref, out_gpu, idx_gpu):
    """Relative L2 error of the GPU's step-0 output over all [T, d] against the
    oracle's, with the oracle re-evaluated on the GPU's experts for the tokens
    that routed differently (near ties of the keys, allowed by the bar)."""
    import numpy as np
    from oracle import ffn, numerics as nx
    same = (np.sort(idx_gpu, 1) == np.sort(r.idx, 1)).all(axis=1)
    ref = out_ref.copy()
    diff = np.nonzero(~same)[0]
    if len(diff):
        idx_fix = r.idx.copy()
        gate_fix = r.gate.copy()
        for t in diff:
            idx_fix[t] = idx_gpu[t]
            sel = s64[t, idx_gpu[t]]
            gate_fix[t] = sel / sel.sum()
        ref[diff] = ffn.layer(cfg, u, idx_fix, gate_fix, hw.w13, hw.w2, hw.w13s, hw.w2s, tokens=diff)
    err = float(np.linalg.norm(out_gpu - ref) / np.linalg.norm(ref))
    u64 = nx.to_f64(u, cfg.in_dtype)
    err_ffn = float(np.linalg.norm(out_gpu - ref) / np.linalg.norm(ref - u64))
    bar = {"f32": 1e-5, "bf16": 1e-2, "fp8": 3e-2}[cfg.expert_dtype]
    rec = {"rel_l2": round(err, 6), "rel_l2_ffn_part": round(err_ffn, 6), "bar": bar, "met": err <= bar,
           "over": "all %d x %d outputs of step 0" % (cfg.T, cfg.d),
           "tokens_routed_differently": int(len(diff))}
    if cfg.expert_dtype == "fp8":
        rec["against"] = "the unquantised oracle (the E4M3 recipe alone is about 3.2e-2 off on these inputs)"
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="v3")
    ap.add_argument("--T", type=int, default=0, help="override tokens per batch")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--backward", type=int, default=5,
                    help="also time this many moe_backward calls (bf16 layers; reported beside the step; 0: skip)")
    ap.add_argument("--load-trajectory", type=int, default=0,
                    help="after the timed steps, run this many forward+update steps from the initial "
                         "bias and report the max/mean expert load of each (every 10th listed)")
    ap.add_argument("--capacity-factors", default="1.0,1.25",
                    help="also time the token-dropping baseline (per-expert capacity ceil(cf*T*K/N_r)) at "
                         "these factors, with the initial bias and with the bias after 100 balancing steps "
                         "(empty: skip)")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="only run a plain device copy of this many MiB (5 times) and exit: the "
                         "reference dispatch for scaling FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        if int(os.environ.get("RANK", "0")) == 0:
            print("bench.py measures one GPU only: this layer's hot path is built and timed on a single "
                  "MI355X (the multi-GPU sharding is described, not run). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import expert_routing_router_amd as M
    from expert_routing_router_amd.layer import MoELayer, np_to_device
    from workloads import gen, get_config

    if args.copy_calibration_mb:
        n = args.copy_calibration_mb * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n * 4, "dispatches": 5}))
        return

    cfg = get_config(args.config)
    if args.T:
        cfg = cfg.with_(T=args.T)
    torch.cuda.set_device(0)
    t0 = time.time()
    log("building %s layer (weights drawn and uploaded) ..." % cfg.name)
    hw = HostWeights(cfg, gen)
    layer = MoELayer(cfg, hw, device="cuda:0")
    log("layer ready in %.1fs" % (time.time() - t0))
    nb = max(1, min(4, args.steps + args.warmup))
    us = [np_to_device(gen.tokens(cfg, s), cfg.in_dtype, "cuda:0") for s in range(nb)]
    b = np_to_device(gen.bias_init(cfg), "f32", "cuda:0")
    torch.cuda.synchronize()

    for i in range(args.warmup):
        layer.forward(us[i % nb], b, update_bias=True)
    torch.cuda.synchronize()
    log("warmup done")

    M.moe_profile_enable(True)
    M.moe_profile_read(reset=True)
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    step_ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step_ev[i].record(stream)
        layer.forward(us[i % nb], b, update_bias=True)
    step_ev[args.steps].record(stream)
    ev1.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    per_step = sorted(step_ev[i].elapsed_time(step_ev[i + 1]) for i in range(args.steps))

    def pct(q):
        return per_step[min(len(per_step) - 1, int(round(q * (len(per_step) - 1))))]
    stage_ms, calls = M.moe_profile_read(reset=True)
    M.moe_profile_enable(False)
    ev_ms = ev0.elapsed_time(ev1)
    ms_per_step = elapsed * 1000.0 / args.steps
    tokens_per_s = cfg.T * args.steps / elapsed
    log("timed %d steps: %.3f ms/step (events %.3f ms/step), %.0f tokens/s"
        % (args.steps, ms_per_step, ev_ms / args.steps, tokens_per_s))

    # the same steps through the row-major weights the ABI takes (no K-blocked copies)
    row_major = None
    if layer.blocked:
        import ctypes
        wr = M.MoeWeights.from_buffer_copy(layer.weights)
        wr.w13_blk = wr.w2_blk = wr.w13_shared_blk = wr.w2_shared_blk = None
        desc = M.desc_from_config(cfg)
        b_rm = np_to_device(gen.bias_init(cfg), "f32", "cuda:0")

        def fwd_rm(i):
            st = M.lib().moe_forward(ctypes.byref(desc), ctypes.byref(wr), us[i % nb].data_ptr(), b_rm.data_ptr(),
                                     layer.out.data_ptr(), None, 1, layer.ws.data_ptr(), layer.ws.numel(),
                                     stream.cuda_stream)
            if st != M.MOE_OK:
                raise M.MoeError("moe_forward", st, M.lib())
        for i in range(args.warmup):
            fwd_rm(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(args.steps):
            fwd_rm(i)
        e1.record(stream)
        torch.cuda.synchronize()
        row_major = {"ms_per_step": round(e0.elapsed_time(e1) / args.steps, 4),
                     "tokens_per_s": round(cfg.T * args.steps / e0.elapsed_time(e1) * 1e3, 1),
                     "note": "moe_forward on the row-major expert weights of the ABI (no K-blocked copies), "
                             "same steps"}
        log("row-major weights: %.3f ms/step" % row_major["ms_per_step"])

    # step 0 from the initial bias, kept for the parity check against the oracle
    b0 = np_to_device(gen.bias_init(cfg), "f32", "cuda:0")
    layer.forward(us[0], b0, update_bias=False)
    torch.cuda.synchronize()
    out0 = layer.out.float().cpu().numpy().astype("float64")
    idx0 = layer.idx.cpu().numpy()

    # load balance over a few extra (untimed) steps
    loads = []
    for i in range(min(4, nb)):
        layer.forward(us[i % nb], b, update_bias=True)
        c = layer.counts.float()
        loads.append(float(c.max() / c.mean()))

    trajectory = None
    if args.load_trajectory:
        b_t = np_to_device(gen.bias_init(cfg), "f32", "cuda:0")
        ratios = []
        for i in range(args.load_trajectory):
            layer.forward(us[i % nb], b_t, update_bias=True)
            c = layer.counts.float()
            ratios.append(float(c.max() / c.mean()))
        trajectory = {"steps": args.load_trajectory, "tokens": "%d resident batches in turn" % nb,
                      "max_over_mean_every_10": [round(x, 3) for x in ratios[::10]],
                      "first": round(ratios[0], 3), "last": round(ratios[-1], 3),
                      "mean_last_20": round(sum(ratios[-20:]) / len(ratios[-20:]), 3)}
        log("load trajectory: max/mean %.3f -> %.3f over %d steps" % (ratios[0], ratios[-1], len(ratios)))

    # the token-dropping baseline: the same step with each expert capped; reported beside the step
    capacity = None
    cfs = [float(x) for x in args.capacity_factors.split(",") if x.strip()]
    if cfs and cfg.T > 0:
        b_bal = np_to_device(gen.bias_init(cfg), "f32", "cuda:0")
        for i in range(100):
            layer.forward(us[i % nb], b_bal, update_bias=True)
        biases = {"initial": np_to_device(gen.bias_init(cfg), "f32", "cuda:0"), "balanced_100": b_bal}
        capacity = []
        for cf in cfs:
            cap = int(math.ceil(cf * cfg.T * cfg.top_k / cfg.n_routed))
            row = {"cf": cf, "capacity": cap}
            for bname, bb in biases.items():
                layer.forward_capacity(us[0], bb, cap, update_bias=False)
                torch.cuda.synchronize()
                nd = []
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                n_cap = 5
                e0.record(stream)
                for i in range(n_cap):
                    layer.forward_capacity(us[i % nb], bb, cap, update_bias=False)
                    nd.append(layer.n_dropped.clone())
                e1.record(stream)
                torch.cuda.synchronize()
                frac = sum(int(x.item()) for x in nd) / (n_cap * cfg.T * cfg.top_k)
                row[bname] = {"ms": round(e0.elapsed_time(e1) / n_cap, 4), "dropped_frac": round(frac, 5)}
            capacity.append(row)
            log("capacity cf %.2f: %s" % (cf, row))
        capacity = {"no_drop_ms_per_step": round(ev_ms / args.steps, 4), "runs": capacity,
                    "note": "forward without bias update, 5 calls each over the resident batches"}

    # the sequence-wise balance loss (forward value) from this layer's router outputs:
    # timed on its own, it is not part of the forward step
    seq_balance = None
    if cfg.T > 0:
        seq_len = 4096 if cfg.T % 4096 == 0 else cfg.T
        desc = M.desc_from_config(cfg)
        sc = torch.empty((cfg.T, cfg.n_routed), dtype=torch.float32, device="cuda:0")
        ri = torch.empty((cfg.T, cfg.top_k), dtype=torch.int32, device="cuda:0")
        rg = torch.empty((cfg.T, cfg.top_k), dtype=torch.float32, device="cuda:0")
        rc = torch.empty(cfg.n_routed, dtype=torch.int32, device="cuda:0")
        M.moe_route(desc, b, ri, rg, rc, u=us[0], E=layer.E, scores_out=sc)
        bl = torch.empty(cfg.T // seq_len, dtype=torch.float32, device="cuda:0")
        bws = torch.empty(M.moe_seq_balance_workspace_bytes(desc, seq_len), dtype=torch.uint8, device="cuda:0")
        M.moe_seq_balance_loss(desc, seq_len, 1e-4, sc, ri, bl, bws)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(20):
            M.moe_seq_balance_loss(desc, seq_len, 1e-4, sc, ri, bl, bws)
        e1.record(stream)
        torch.cuda.synchronize()
        sb_ms = e0.elapsed_time(e1) / 20
        sb_bytes = cfg.T * cfg.n_routed * 4 + cfg.T * cfg.top_k * 4
        seq_balance = {"ms": round(sb_ms, 4), "GB/s": round(sb_bytes / sb_ms / 1e6, 1),
                       "hbm_frac": round(sb_bytes / sb_ms / 1e6 / PEAK_HBM_GBS, 4), "seq_len": seq_len,
                       "loss_over_alpha": [round(float(x) / 1e-4, 6) for x in bl.cpu()]}
        log("seq balance loss: %.4f ms for %d sequences" % (sb_ms, cfg.T // seq_len))

    bwd = None
    if args.backward and cfg.expert_dtype in ("bf16", "fp8") and cfg.in_dtype == "bf16":
        rng = torch.Generator(device="cuda:0").manual_seed(5)
        dout = torch.randn((cfg.T, cfg.d), generator=rng, device="cuda:0").to(torch.bfloat16)
        t0 = time.time()
        layer.backward(us[0], b, dout)           # first call: transposed weights, buffers
        torch.cuda.synchronize()
        log("backward set-up + first call %.1fs" % (time.time() - t0))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(args.backward):
            layer.backward(us[i % nb], b, dout)
        e1.record(stream)
        torch.cuda.synchronize()
        bwd_ms = e0.elapsed_time(e1) / args.backward
        R = cfg.T * cfg.top_k + cfg.n_shared * cfg.T
        w13 = (cfg.n_routed + cfg.n_shared) * 2 * cfg.inter * cfg.d
        w2 = (cfg.n_routed + cfg.n_shared) * cfg.inter * cfg.d
        # forward recompute (A|B, Y) + dH + dX + dW2 + dW13: six products of the experts' shape
        # (bf16 MFMAs, or E4M3 ones for the FP8 layer)
        flops = 3.0 * 2.0 * R * cfg.d * 3 * cfg.inter
        bwd_peak = PEAK_TFLOPS[cfg.expert_dtype]
        # weights read twice (W, W^T: 2 bytes, or 1 byte of E4M3 code), fp32 weight gradients
        # written once, u / dout / du
        wbytes = 2 if cfg.expert_dtype == "bf16" else 1
        byts = 2 * wbytes * (w13 + w2) + 4 * (w13 + w2) + cfg.T * cfg.d * (2 + 2 + 4)
        bwd = {"ms": round(bwd_ms, 3), "tokens_per_s": round(cfg.T / bwd_ms * 1e3, 1),
               "TFLOP/s": round(flops / bwd_ms / 1e9, 1), "mfma_frac": round(flops / bwd_ms / 1e9 / bwd_peak, 4),
               "GB/s": round(byts / bwd_ms / 1e6, 1), "hbm_frac": round(byts / bwd_ms / 1e6 / PEAK_HBM_GBS, 4),
               "algorithmic_flops": flops, "algorithmic_bytes": byts, "calls": args.backward}
        log("backward: %.3f ms/call (%.0f TFLOP/s, %.0f GB/s algorithmic)" % (bwd_ms, flops / bwd_ms / 1e9,
                                                                           byts / bwd_ms / 1e6))

    # the machine's ceilings, measured here: a streaming read and an MFMA-only loop
    cal_buf = torch.empty(4 << 30, dtype=torch.uint8, device="cuda:0")
    cal_sink = torch.zeros(4, dtype=torch.int32, device="cuda:0")
    M.moe_calibrate_read(cal_buf, cal_sink)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(3):
        M.moe_calibrate_read(cal_buf, cal_sink)
    e1.record(stream)
    torch.cuda.synchronize()
    read_gbs = 3 * cal_buf.numel() / e0.elapsed_time(e1) / 1e6
    del cal_buf
    iters = 4000
    fsink = torch.zeros(4, dtype=torch.float32, device="cuda:0")
    M.moe_calibrate_mfma_bf16(100, fsink)
    e0.record(stream)
    M.moe_calibrate_mfma_bf16(iters, fsink)
    e1.record(stream)
    torch.cuda.synchronize()
    mfma_tf = M.MOE_CAL_MFMA_WAVES * iters * 8 * 32768.0 / e0.elapsed_time(e1) / 1e9
    measured = {"hbm_read_GBps": round(read_gbs, 1), "mfma_bf16_TFLOPs": round(mfma_tf, 1),
                "how": "moe_calibrate_read: 3 streaming reads of 4 GiB; moe_calibrate_mfma_bf16: "
                       "8192 waves x 4000 x 8 independent 32x32x16 bf16 MFMAs"}
    log("measured ceilings: HBM read %.0f GB/s, bf16 MFMA %.0f TFLOP/s" % (read_gbs, mfma_tf))

    alg = algorithmic(cfg)
    peak_tf = PEAK_TFLOPS[cfg.expert_dtype]
    kernels = {}
    for name, a in alg.items():
        ms = stage_ms.get(name, 0.0) / max(calls, 1)
        if ms <= 0:
            continue
        k = {"ms": round(ms, 4), "GB/s": round(a["bytes"] / ms / 1e6, 1),
             "hbm_frac": round(a["bytes"] / ms / 1e6 / PEAK_HBM_GBS, 4)}
        if a["flops"]:
            tf = a["flops"] / ms / 1e9
            k["TFLOP/s"] = round(tf, 1)
            k["mfma_frac"] = round(tf / (peak_tf if name.startswith("gemm") else PEAK_TFLOPS["bf16"]), 4)
        kernels[name] = k
    if seq_balance:
        kernels["seq_balance_loss"] = seq_balance
    g_ms = (stage_ms["gemm1"] + stage_ms["gemm2"]) / max(calls, 1)
    g_tf = (alg["gemm1"]["flops"] + alg["gemm2"]["flops"]) / g_ms / 1e9
    kernels["grouped_gemm"] = {"ms": round(g_ms, 4), "TFLOP/s": round(g_tf, 1),
                               "mfma_frac": round(g_tf / peak_tf, 4)}
    if cfg.expert_dtype == "bf16":
        kernels["grouped_gemm"]["mfma_frac_of_measured"] = round(g_tf / mfma_tf, 4)
    for k in kernels.values():
        if "GB/s" in k:
            k["hbm_frac_of_measured"] = round(k["GB/s"] / read_gbs, 4)

    g1 = alg["gemm1"]
    g1_ms = stage_ms["gemm1"] / max(calls, 1)
    achieved = g1["bytes"] / g1_ms / 1e6
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": measured_traffic(cfg),
                "kernel": "grouped gate/up GEMM + SwiGLU over routed and shared rows (gemm_%s kernel)" % ("bf16_dma" if cfg.expert_dtype == "bf16" else cfg.expert_dtype),
                "bytes_per_launch": g1["bytes"], "avg_ms": round(g1_ms, 4),
                "measured_peak": round(read_gbs, 1), "frac_of_measured": round(achieved / read_gbs, 4)}

    cpu = parity = None
    if not args.no_cpu_baseline:
        del layer
        torch.cuda.empty_cache()
        cpu, r_ref, s64_ref, out_ref = cpu_baseline(cfg, hw, log)
        parity = parity_line(cfg, hw, gen.tokens(cfg, 0), r_ref, s64_ref, out_ref, out0, idx0)
        log("parity: step-0 output rel-L2 %.3e against the oracle (bar %.0e)" % (parity["rel_l2"], parity["bar"]))

    dtype = {"bf16": "bf16", "fp8": "fp8_e4m3", "f32": "f32"}[cfg.expert_dtype]
    rec = {
        "metric": "MoE-layer tokens/s (V3 shape: T=8192, d=7168, 256 routed experts top-8 in 8 groups / "
                  "M=4, 1 shared, SwiGLU I=2048) + grouped-GEMM % MFMA peak",
        "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": dtype, "data": "synthetic",
        "config": {"workload": "%s: T=%d d=%d N_r=%d K=%d G=%d M=%d q=%d N_s=%d I=%d I_s=%d experts=%s "
                               "router=%s; forward + bias update per step%s"
                               % (cfg.name, cfg.T, cfg.d, cfg.n_routed, cfg.top_k, cfg.n_groups,
                                  cfg.topk_groups, cfg.group_topk, cfg.n_shared, cfg.inter,
                                  cfg.inter_shared, cfg.expert_dtype, cfg.router_dtype,
                                  "; the timed forward reads K-blocked copies of the expert weights "
                                  "(moe_pack_expert_weights, made once before timing; the row-major ABI "
                                  "path is timed in row_major_weights)" if row_major else ""),
                   "T": cfg.T, "d": cfg.d, "n_routed": cfg.n_routed, "top_k": cfg.top_k,
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "parity": parity,
        "row_major_weights": row_major,
        "kernels": kernels,
        "grouped_gemm_mfma_frac": kernels["grouped_gemm"]["mfma_frac"],
        "max_over_mean_load": [round(x, 3) for x in loads],
        "load_trajectory": trajectory,
        "backward": bwd,
        "capacity_baseline": capacity,
        "event_ms_per_step": round(ev_ms / args.steps, 4),
        "step_ms": {"median": round(pct(0.5), 4), "p10": round(pct(0.1), 4), "p90": round(pct(0.9), 4)},
        "measured_ceilings": measured,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
