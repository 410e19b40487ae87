"""Benchmark: MoE layer forward tokens/s on one MI355X, with roofline fractions (and the
backward and a graph replay of the same step reported beside it).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config c1|c2|c3|c4|c0|c2ec|c2v3] [--no-cpu]

Prints ONE JSON line on stdout (progress goes to stderr).  A step is one
moe_layer_fwd call (route -> dispatch -> expert FFN -> combine, plus the latent
projections for the multi-head workload) over one batch of synthetic tokens
already resident in HBM.  K steps run back to back on one stream between two
device synchronisations; value = T * K / elapsed.

The layer runs without an x_perm buffer: dispatch moves indices only and the
expert FFN gathers each row from x inside its GEMM operand loads.

Per-stage times: separate calls of moe_route / moe_dispatch /
moe_expert_ffn_gather / moe_combine on the same data, timed with HIP events
recorded on the stream the kernels run on, two ways:
  cold   each call preceded (outside its events) by a read-modify-write of a
         1 GiB scratch buffer, which evicts the L2 caches and the 256 MiB
         Infinity Cache; the GPU is still busy with that write when the call
         is issued, so the events bracket device time only.  The headline
         fractions use these.
  warm   the same call captured `reps` times in one HIP graph and replayed:
         back-to-back device time with whatever the caches kept.
The roofline object is for the grouped GEMM of the expert FFN (its gate/up
launches with the SwiGLU epilogue, then its down launches), the dominant
kernel: achieved = algorithmic FLOPs of the kept rows and shared experts /
cold stage time, against the bf16 dense MFMA peak.  Beside the headline
workload (--config, default the coarse 4096-token one) the other bf16
workloads (--also, default c2,c3,c4) are measured the same way and reported
under "configs".  The CPU baseline is the float64 numpy oracle on a bounded
sample of the headline workload (routing of every token, expert FFN and
combine for a token sample).
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 matrix
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E

METRIC = "MoE layer fwd tokens/s on 1 MI355X; grouped-GEMM MFMA % + route/dispatch HBM %"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="c1")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--cpu-tokens", type=int, default=0, help="oracle sample size (0: automatic)")
    ap.add_argument("--json-out", default="", help="also append the JSON line to this file")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward timing")
    ap.add_argument("--no-graph", action="store_true", help="skip timing the step as a captured HIP graph")
    ap.add_argument("--also", default="c2,c3,c4",
                    help="further workloads measured in the same run and reported under 'configs' ('' for none)")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="after timing, run one device-to-device copy of this many MiB (a known-size "
                         "reference for the HBM byte counters of a profiler run)")
    return ap.parse_args()


def algorithmic(cfg, R):
    """Algorithmic bytes (HBM) and FLOPs of each step, for R kept rows."""
    a = 4 if cfg.act_dtype == 0 else 2
    r = 4 if cfg.router_dtype == 0 else 2
    T, d, H, dh, E, K = cfg.T, cfg.d_model, cfg.n_heads, cfg.d_head, cfg.n_experts, cfg.k_total
    m = 3 if cfg.act == 1 else 2
    out = {}
    out["route_bytes"] = T * H * dh * a + E * dh * r + T * K * 8
    # dispatch moves indices only: the expert FFN gathers its rows from x itself
    out["dispatch_bytes"] = T * K * 8 + R * 4 + (T * K * 4 if cfg.drop == 2 else 0)
    out["combine_bytes"] = R * dh * a + T * K * 8 + T * H * dh * a * (1 + (cfg.residual and not cfg.latent_proj)
                                                                        + (cfg.n_shared > 0))
    out["ffn_flops"] = 2 * R * dh * m * cfg.d_ff + 2 * T * d * m * cfg.n_shared * cfg.d_ff
    out["proj_flops"] = (2 * 2 * T * d * H * dh) if cfg.latent_proj else 0
    return out


def ffn_source_sha256():
    """sha256 over the expert FFN's kernel sources (grouped GEMM, fused MLP), in that order."""
    import hashlib
    h = hashlib.sha256()
    for f in ("gemm.hip", "mlp.hip"):
        with open(os.path.join(ROOT, "routing_dispatch_expert_router_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(cfg):
    """HBM bytes per expert-FFN call measured with rocprofv3 for this workload, if the
    FFN kernels' sources are unchanged since the measurement (else None)."""
    f = os.path.join(ROOT, "profiles", f"traffic__expert_ffn__{cfg.name}.json")
    if not os.path.exists(f):
        return None
    with open(f) as fh:
        rec = json.load(fh)
    if rec.get("ffn_source_sha256") != ffn_source_sha256():
        return None
    return rec["traffic_bytes"]


def fused_mlp(cfg):
    """Whether the library runs this workload's routed experts through the fused MLP kernel
    (bf16 experts of width 64, 128 or 256, hidden width a multiple of 32)."""
    return cfg.act_dtype == 1 and cfg.d_head in (64, 128, 256) and cfg.d_ff % 32 == 0


def time_backward(cfg, moe, W, x, inp, args, stream):
    """moe_layer_bwd on the same batch (dy synthetic, aux weight 0.01 for one head): ms per
    step, and the forward + backward step as tokens/s.  Algorithmic FLOPs of the backward:
    twice the forward's expert and projection FLOPs (input and weight gradients).  Where the
    routed experts run the grouped GEMM, the forward keeps their pre-activations (io gu) and
    the backward reads them instead of recomputing the gate/up products; that forward is
    timed too ("fwd_ms_keeping"), and the forward + backward figure uses it."""
    import torch
    T, K, E, dh, F, d = cfg.T, cfg.k_total, cfg.n_experts, cfg.d_head, cfg.d_ff, cfg.d_model
    Rm = moe.moe_rows_upper_bound(cfg)
    adt = torch.bfloat16 if cfg.act_dtype == 1 else torch.float32
    m = 2 if cfg.act == 1 else 1
    fs = cfg.n_shared * F
    e = lambda *shape, dt=adt: torch.empty(*shape, dtype=dt, device="cuda")
    io = dict(logits=e(T, E, dt=torch.float32), logits_mode=moe.MOE_LOGITS_COMPUTE_STORE,
              topk_idx=e(T, K, dt=torch.int32), topk_w=e(T, K, dt=torch.float32), demand=e(E, dt=torch.int32),
              counts=e(E, dt=torch.int32), offsets=e(E + 1, dt=torch.int32), row_of=e(T, K, dt=torch.int32),
              src_of=e(max(Rm, 1), dt=torch.int32), y_perm=e(max(Rm, 1), dh),
              shared_out=e(T, d) if fs else None,
              z=e(T, cfg.d_latent) if cfg.latent_proj else None, o=e(T, cfg.d_latent) if cfg.latent_proj else None,
              gu=e(max(Rm, 1), m * F) if not fused_mlp(cfg) else None)
    y = torch.empty_like(x)
    fws = moe.workspace(cfg)
    moe.moe_layer_fwd(cfg, W, x, y, io, fws)
    # the forward that keeps the pre-activations, timed on its own
    for _ in range(2):
        moe.moe_layer_fwd(cfg, W, x, y, io, fws)
    nf = max(3, min(args.steps, 20))
    fa, fb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fa.record(stream)
    for _ in range(nf):
        moe.moe_layer_fwd(cfg, W, x, y, io, fws)
    fb.record(stream)
    torch.cuda.synchronize()
    fwd_keep_ms = fa.elapsed_time(fb) / nf
    D = cfg.d_latent
    wt = dict(w13t=e(E, dh, m * F), w2t=e(E, F, dh), ws13t=e(d, m * fs) if fs else None,
              ws2t=e(fs, d) if fs else None, w_in_t=e(d, D) if cfg.latent_proj else None,
              w_out_t=e(D, d) if cfg.latent_proj else None)
    moe.moe_transpose_weights(cfg, W, wt)
    g = dict(dx=e(T, d), dw_router=e(E, dh, dt=torch.float32), dbias=e(E, dt=torch.float32), dw1=e(E, F, dh),
             dw3=e(E, F, dh) if cfg.act == 1 else None, dw2=e(E, dh, F), dws1=e(fs, d) if fs else None,
             dws3=e(fs, d) if (fs and cfg.act == 1) else None, dws2=e(d, fs) if fs else None,
             dw_in=e(D, d) if cfg.latent_proj else None, dw_out=e(d, D) if cfg.latent_proj else None)
    gen = torch.Generator(device="cuda").manual_seed(1234)
    dy = torch.randn(T, d, device="cuda", generator=gen).to(adt)
    ws = moe.backward_workspace(cfg)
    aux_w = 0.01 if cfg.n_heads == 1 else 0.0  # the aux loss is defined for one routing head
    step = lambda: moe.moe_layer_bwd(cfg, W, wt, x, dy, aux_w, io, g, ws)
    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()
    n = max(3, min(args.steps, 20))
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(n):
        step()
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / n
    R = int(io["offsets"][E].item())
    alg = algorithmic(cfg, R)
    flops = 2 * (alg["ffn_flops"] + alg["proj_flops"])
    tf = flops / (ms * 1e-3) / 1e12
    peak = PEAK_F32_TFLOPS if cfg.act_dtype == 0 else PEAK_BF16_TFLOPS
    log(f"[bench] backward {ms:.3f} ms/step, {tf:.4g} TFLOP/s ({tf / peak:.1%} of peak)")
    return {"ms_per_step": ms, "steps": n, "algorithmic_flops": flops, "TFLOPs": tf, "mfma_frac": tf / peak,
            "aux_weight": aux_w, "kept_preactivations": io["gu"] is not None, "fwd_ms_keeping": fwd_keep_ms}


def cpu_threads():
    try:
        from threadpoolctl import threadpool_info
        n = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        n = len(os.sched_getaffinity(0))
    return int(n)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(cfg, inp, sample, target_s=12.0):
    """The oracle on a token sample sized for about `target_s` seconds (at most all T tokens).

    Every run routes all T tokens (a fixed cost) and runs the expert FFN and
    combine on the sampled tokens (a cost per token): two short runs fit both,
    and the reported run uses the sample size the fit gives for `target_s`."""
    import oracle

    def run(n):
        toks = np.linspace(0, cfg.T - 1, n).astype(np.int64)
        t0 = time.perf_counter()
        oracle.forward(cfg, inp, tokens=toks)
        return time.perf_counter() - t0

    n1 = max(1, min(sample, cfg.T))
    dt = run(n1)
    n = n1
    if dt < target_s / 2 and n1 < cfg.T:
        n2 = min(cfg.T, 2 * n1)
        dt2 = run(n2)
        per_tok = max((dt2 - dt) / max(n2 - n1, 1), 1e-9)
        fixed = max(dt - per_tok * n1, 0.0)
        n, dt = n2, dt2
        want = int(min(cfg.T, max(n2, (target_s - fixed) / per_tok)))
        if want > n2:
            n, dt = want, run(want)
    return {"value": n / dt, "unit": "tokens/s", "cores": cpu_threads(), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"float64 numpy oracle: routing + keep rule of all {cfg.T} tokens, expert FFN and "
                      f"combine for {n} evenly spaced tokens; {dt:.1f} s wall"}


def workload(name):
    from moe_inputs import CONFIGS, VARIANTS
    short = {"c0": CONFIGS[0], "c1": CONFIGS[1], "c2": CONFIGS[2], "c3": CONFIGS[3], "c4": CONFIGS[4],
             "c2ec": VARIANTS[0], "c2v3": VARIANTS[1]}
    return short[name] if name in short else next(c for c in CONFIGS + VARIANTS if c.name == name)


class Evict:
    """A 1 GiB device buffer.  touch() writes all of it (a scratch write that evicts the L2 caches
    and the 256 MiB Infinity Cache), then reads it back: the read pass forces the write-back of the
    dirty lines the write left in the caches, so the timed call that follows finds its inputs out
    of cache without paying for another buffer's write-back.  A few hundred microseconds."""

    def __init__(self):
        import torch
        self.buf = torch.zeros(1 << 28, dtype=torch.int32, device="cuda")
        self.sink = None

    def touch(self):
        self.buf.add_(1)
        self.sink = self.buf.max()


def time_stage(fn, stream, evict, reps):
    """Device time of one call of fn, in seconds: (cold, warm).

    cold: mean over `reps` calls, each after evict.touch() and bracketed by its own events (the
    eviction is still running when the call is issued, so the events see device time only).
    warm: `reps` calls captured in one HIP graph, replayed between two events, per call."""
    import torch
    for _ in range(2):
        fn()
    torch.cuda.synchronize()
    evs = []
    for _ in range(reps):
        evict.touch()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        evs.append((a, b))
    torch.cuda.synchronize()
    cold = sum(a.elapsed_time(b) for a, b in evs) / reps * 1e-3
    # warm: a graph of reps calls on a side stream (capture needs a non-default stream)
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for _ in range(reps):
                fn()
    stream.wait_stream(side)
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    g.replay()
    b.record(stream)
    torch.cuda.synchronize()
    warm = a.elapsed_time(b) / reps * 1e-3
    del g
    return cold, warm


def measure(cfg, args, evict, headline):
    """Step time, per-stage times and roofline fractions of one workload (dict)."""
    import torch
    import routing_dispatch_expert_router_amd as moe
    from moe_inputs import generate
    log(f"[bench] {cfg.name}: generating inputs")
    t0 = time.perf_counter()
    inp = generate(cfg)
    log(f"[bench] inputs in {time.perf_counter() - t0:.1f} s; moving to HBM")

    def dev(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to("cuda").view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")

    W = dict(w_router=dev(inp.w_router), router_bias=dev(inp.bias), w1=dev(inp.w1), w3=dev(inp.w3),
             w2=dev(inp.w2), ws1=dev(inp.ws1), ws3=dev(inp.ws3), ws2=dev(inp.ws2), w_in=dev(inp.w_in),
             w_out=dev(inp.w_out), sel_bias=dev(inp.sel_bias))
    x = dev(inp.x)
    y = torch.empty_like(x)
    T, K, E, dh = cfg.T, cfg.k_total, cfg.n_experts, cfg.d_head
    Rm = moe.moe_rows_upper_bound(cfg)
    adt = torch.bfloat16 if cfg.act_dtype == 1 else torch.float32
    io = dict(topk_idx=torch.empty(T, K, dtype=torch.int32, device="cuda"),
              topk_w=torch.empty(T, K, dtype=torch.float32, device="cuda"),
              demand=torch.empty(E, dtype=torch.int32, device="cuda"),
              counts=torch.empty(E, dtype=torch.int32, device="cuda"),
              offsets=torch.empty(E + 1, dtype=torch.int32, device="cuda"),
              row_of=torch.empty(T, K, dtype=torch.int32, device="cuda"),
              src_of=torch.empty(Rm, dtype=torch.int32, device="cuda"),
              y_perm=torch.empty(Rm, dh, dtype=adt, device="cuda"),
              shared_out=torch.empty(T, cfg.d_model, dtype=adt, device="cuda") if cfg.n_shared else None,
              z=torch.empty(T, cfg.d_latent, dtype=adt, device="cuda") if cfg.latent_proj else None,
              o=torch.empty(T, cfg.d_latent, dtype=adt, device="cuda") if cfg.latent_proj else None,
              seq_loss=torch.empty(T // cfg.seq_len, dtype=torch.float32, device="cuda") if cfg.seq_len else None)
    ws = moe.workspace(cfg)
    stream = torch.cuda.current_stream()

    def step():
        moe.moe_layer_fwd(cfg, W, x, y, io, ws)

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    R = int(io["offsets"][E].item())
    steps = args.steps if headline else max(5, min(args.steps, 20))
    log(f"[bench] R = {R} kept rows; timing {steps} steps")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = ev0.elapsed_time(ev1) / steps
    log(f"[bench] {ms_step:.3f} ms/step (events), {wall / steps * 1e3:.3f} ms/step (wall)")

    # ---- the same step captured once in a HIP graph and replayed (no per-launch host work)
    graph = None
    if headline and not args.no_graph:
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        g.replay()
        torch.cuda.synchronize()
        ga, gb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ga.record(stream)
        for _ in range(steps):
            g.replay()
        gb.record(stream)
        torch.cuda.synchronize()
        gms = ga.elapsed_time(gb) / steps
        graph = {"ms_per_step": gms, "tokens_per_s": T / (gms * 1e-3), "steps": steps}
        log(f"[bench] graph replay {gms:.3f} ms/step")
        del g

    # ---- per-stage times: the four C-ABI calls on the same data
    xin = io["z"] if cfg.latent_proj else x
    reps = 20
    st = {}
    st["route"] = time_stage(lambda: moe.moe_route(cfg, xin, W["w_router"], W["router_bias"], None,
                                                   moe.MOE_LOGITS_COMPUTE, io["topk_idx"], io["topk_w"], None, ws,
                                                   sel_bias=W["sel_bias"], seq_loss=io["seq_loss"]),
                             stream, evict, reps)
    st["dispatch"] = time_stage(lambda: moe.moe_dispatch(cfg, io["topk_idx"], io["topk_w"], None, io["demand"],
                                                         io["counts"], io["offsets"], io["row_of"], io["src_of"],
                                                         None, ws), stream, evict, reps)
    st["expert_ffn"] = time_stage(lambda: moe.moe_expert_ffn_gather(cfg, xin, io["src_of"], io["offsets"],
                                                                    W["w1"], W["w3"], W["w2"], io["y_perm"],
                                                                    x if cfg.n_shared else None, W["ws1"],
                                                                    W["ws3"], W["ws2"], io["shared_out"], ws),
                                  stream, evict, min(reps, 10))
    st["combine"] = time_stage(lambda: moe.moe_combine(cfg, io["y_perm"], io["row_of"], io["topk_w"],
                                                       x if (cfg.residual and not cfg.latent_proj) else None,
                                                       io["shared_out"], io["o"] if cfg.latent_proj else y),
                               stream, evict, reps)
    if W["sel_bias"] is not None:
        # one balancing-bias update from this batch's loads, on a scratch copy of the bias
        b_tmp = W["sel_bias"].clone()
        st["sel_bias_update"] = time_stage(lambda: moe.moe_sel_bias_update(cfg, io["demand"], b_tmp, 0.001),
                                           stream, evict, reps)
    bwd = None
    if headline and not args.no_backward and moe.moe_backward_workspace_bytes(cfg) > 0:
        bwd = time_backward(cfg, moe, W, x, inp, args, stream)
    alg = algorithmic(cfg, R)
    peak = PEAK_F32_TFLOPS if cfg.act_dtype == 0 else PEAK_BF16_TFLOPS
    stages = {}
    for k, nb in (("route", "route_bytes"), ("dispatch", "dispatch_bytes"), ("combine", "combine_bytes")):
        cold, warm = st[k]
        stages[k] = {"us": cold * 1e6, "us_warm": warm * 1e6, "GBs": alg[nb] / cold / 1e9,
                     "hbm_frac": alg[nb] / cold / 1e9 / PEAK_HBM_GBS,
                     "hbm_frac_warm": alg[nb] / warm / 1e9 / PEAK_HBM_GBS, "algorithmic_bytes": alg[nb]}
    cold, warm = st["expert_ffn"]
    ffn_tf = alg["ffn_flops"] / cold / 1e12
    stages["expert_ffn"] = {"us": cold * 1e6, "us_warm": warm * 1e6, "TFLOPs": ffn_tf, "mfma_frac": ffn_tf / peak,
                            "mfma_frac_warm": alg["ffn_flops"] / warm / 1e12 / peak,
                            "algorithmic_flops": alg["ffn_flops"]}
    if "sel_bias_update" in st:
        stages["sel_bias_update"] = {"us": st["sel_bias_update"][0] * 1e6, "us_warm": st["sel_bias_update"][1] * 1e6}
    for k, v in stages.items():
        log(f"[bench]   {k:10s} " + "  ".join(f"{a}={b:.4g}" for a, b in v.items()))
    res = {"workload": cfg.name, "T": T, "kept_rows": R, "ms_per_step": ms_step, "tokens_per_s": T / (ms_step * 1e-3),
           "stages": stages, "graph": graph, "backward": bwd,
           "roofline": {"kernel": ("mlp_kernel, expert FFN (fused gate/up, activation and down product, rows "
                                   "gathered from the latent input)" if fused_mlp(cfg) else
                                   "grouped_gemm_kernel, expert FFN (gate/up and down launches, rows gathered from x)")
                        + (" + shared experts (plain grouped_gemm_kernel launches)" if cfg.n_shared else ""),
                        "bound": "mfma", "achieved": ffn_tf, "peak": peak, "unit": "TFLOP/s", "frac": ffn_tf / peak,
                        "frac_warm": alg["ffn_flops"] / warm / 1e12 / peak,
                        "traffic": measured_traffic(cfg),
                        "traffic_unit": "HBM bytes per expert-FFN call (all its launches)",
                        "algorithmic_flops": alg["ffn_flops"], "timing": "cold (L2 and Infinity Cache evicted)"}}
    if bwd is not None:
        bwd["fwd_bwd_tokens_per_s"] = T / ((bwd["fwd_ms_keeping"] + bwd["ms_per_step"]) * 1e-3)
    res["_inp"] = inp
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import routing_dispatch_expert_router_amd  # noqa: F401  (fails loudly if libmoe.so is missing)

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev_name = torch.cuda.get_device_properties(0).name
    cfg = workload(args.config)
    evict = Evict()
    log(f"[bench] {cfg.name} on {dev_name}")
    head = measure(cfg, args, evict, headline=True)
    inp = head.pop("_inp")
    others = {}
    for name in [n for n in args.also.split(",") if n.strip()]:
        oc = workload(name.strip())
        if oc.name == cfg.name:
            continue
        torch.cuda.empty_cache()
        r = measure(oc, args, evict, headline=False)
        r.pop("_inp")
        for k in ("graph", "backward"):
            r.pop(k)
        others[oc.name] = r
        torch.cuda.empty_cache()
    if args.copy_calib_mib:
        n = args.copy_calib_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    T, E = cfg.T, cfg.n_experts
    line = {
        "metric": METRIC, "value": head["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": head["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32" if cfg.act_dtype == 0 else "bf16", "data": "synthetic",
        "config": {"workload": cfg.name, "T": T, "d_model": cfg.d_model, "n_experts": E, "top_k": cfg.top_k,
                   "n_heads": cfg.n_heads, "d_ff": cfg.d_ff, "n_shared": cfg.n_shared, "kept_rows": head["kept_rows"],
                   "act": "swiglu" if cfg.act == 1 else "relu",
                   "drop": "expert_choice" if cfg.route_mode == 1 else ["none", "capacity", "affinity"][cfg.drop],
                   "capacity": cfg.capacity if cfg.drop == 1 else None,
                   "selection_bias": inp.sel_bias is not None, "seq_len": cfg.seq_len or None,
                   "parallelism": "single GPU"},
        "roofline": head["roofline"],
        "stages": head["stages"],
        "backward": head["backward"],
        "graph": head["graph"],
        "configs": others,
        "device": dev_name,
    }
    if not args.no_cpu:
        sample = args.cpu_tokens or {"c0": 256, "c1": 384, "c2": 1024, "c3": 96, "c4": 2048, "c2ec": 1024,
                                     "c2v3": 1024}.get(args.config, 384)
        log(f"[bench] oracle CPU baseline on {sample} tokens")
        line["cpu_baseline"] = cpu_baseline(cfg, inp, sample)
    s = json.dumps(line)
    print(s, flush=True)
    if args.json_out:
        with open(args.json_out, "a") as f:
            f.write(s + "\n")


if __name__ == "__main__":
    main()
