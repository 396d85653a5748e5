"""LatentMoE layer forward benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload super_decode]
    python bench.py --workload super_mamba_verify     (Mamba-2 checkpoint + replay verify)

One step is one whole layer forward (router, top-K, bucketing, W_down, grouped
expert GEMMs, combine, shared expert, W_up) over one batch of seeded synthetic
tokens already resident in HBM.  Prints one JSON line with the throughput, the
roofline of the dominant kernel (timed with HIP events on the forward's stream
during the timed steps) and the fp64 oracle timed on the host cores over a
bounded sample of the same workload.  The headline is the Super decode step;
with the default workload the line also carries a "workloads" object with the
same measurements for the Super prefill chunk (MFMA-bound), the Ultra shape
and FP4 experts.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
METRIC = "LatentMoE layer tokens/s; % HBM peak (decode) / % MFMA peak (prefill)"
PROFILES = os.path.join(ROOT, "profiles")
CSRC = "sparse_moe_layer_logits_amd/csrc/"
KERNEL_SOURCES = {  # kernel -> the files (source and included headers) whose hash pins stored counter data
    "gemm_stream_kernel": ("gemm_stream.hip", "common.hpp", "epilogue.hpp", "fp4.hpp", "fp8.hpp", "kernels.hpp"),
    "gemm_stream_pair_kernel": ("gemm_stream.hip", "common.hpp", "epilogue.hpp", "fp4.hpp", "fp8.hpp",
                                "kernels.hpp"),
    "gemm_mid_kernel": ("gemm_mid.hip", "common.hpp", "epilogue.hpp", "fp4.hpp", "fp8.hpp", "kernels.hpp"),
    "gemm_big_kernel": ("gemm_big.hip", "common.hpp", "epilogue.hpp", "kernels.hpp"),
    "ssm_verify_kernel": ("ssm_replay.hip", "common.hpp", "../../include/ssm_replay.h"),
}


def log(*a):
    print("[bench %s]" % time.strftime("%H:%M:%S"), *a, file=sys.stderr, flush=True)


def source_sha(kernel):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        h.update(open(os.path.join(ROOT, CSRC, f), "rb").read())
    return h.hexdigest()[:16]


def algorithmic(wl, touched):
    """Whole-layer algorithmic bytes and flops (what the method must move and
    compute; intermediates excluded, multiply-add = 2 flops)."""
    d, l, n, k, m, ms, T = wl.d, wl.latent, wl.n_experts, wl.top_k, wl.expert_hidden, wl.shared_hidden, wl.T
    fp4 = 0.5 + 1.0 / 16                                   # code nibble + E4M3 per 16
    beta = 2.0 if wl.experts == "bf16" else fp4
    per_expert_extra = 0 if wl.experts == "bf16" else 8    # two fp32 tensor scales
    proj = 2 * l * d * 2 if wl.proj == "bf16" else 2 * l * d + 8
    shared = 2 * d * ms * 2 if wl.shared == "bf16" else 2 * d * ms * fp4 + 8
    bytes_ = (n * d * 4 + proj + touched * (2 * l * m * beta + per_expert_extra)
              + shared + T * d * 2 + T * d * 4)
    flops = 2.0 * T * (d * n + 2 * d * l + 2 * k * l * m + 2 * d * ms)
    return bytes_, flops


def shared_rides(wl):
    """Whether the library runs the shared expert's two GEMMs inside the expert
    launches (S1 with expert up, S2 with expert down): decode-sized forwards
    (T <= 64) with bf16 experts, shared expert and projections whose experts take
    the streaming kernel."""
    return (wl.T <= 64 and wl.experts == "bf16" and wl.shared == "bf16" and wl.proj == "bf16"
            and wl.T * wl.top_k / wl.n_experts <= 48)


def expert_kernel_units(wl, touched, stage):
    """Algorithmic bytes and flops of one launch of a grouped expert GEMM:
    the touched experts' weight matrix, the T*K routed input rows, the T*K
    output rows (bf16 rows for the method's activations); plus, when the shared
    expert rides in that launch, its matrix, its T input and T output rows."""
    l, m, TK = wl.latent, wl.expert_hidden, wl.T * wl.top_k
    wbytes = l * m * (2.0 if wl.experts == "bf16" else 0.5 + 1.0 / 16)
    if stage == "expert_up":
        io = TK * l * 2 + TK * m * 2
    else:
        io = TK * m * 2 + TK * l * 2
    b, f = touched * wbytes + io, 2.0 * TK * l * m
    if shared_rides(wl):
        d, ms, T = wl.d, wl.shared_hidden, wl.T
        b += d * ms * 2 + T * ms * 2 + (T * d * 2 if stage == "expert_up" else T * d * 4)  # x or y (fp32)
        f += 2.0 * T * d * ms
    return b, f


def expert_kernel(wl):
    """The kernel the library runs the grouped expert GEMMs with: the host's choice
    by weight format and average routed rows per expert (T K / N): bf16 experts
    above 48 rows take the large-tile kernel; otherwise streaming tiles of 16 rows
    (up to 12 rows), 32 (up to 24) or 64, and FP4 experts with 64-row tiles the
    LDS-staged FP4 kernel."""
    avg_rows = wl.T * wl.top_k / wl.n_experts
    if wl.experts == "bf16" and avg_rows > 48:
        return "gemm_big_kernel"
    if wl.experts == "fp4" and avg_rows > 24 and wl.latent % 128 == 0 and wl.expert_hidden % 128 == 0:
        return "gemm_mid_kernel"
    return "gemm_stream_pair_kernel" if shared_rides(wl) else "gemm_stream_kernel"


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, x, W, budget_s=15.0, threads=None):
    """The fp64 oracle on the host cores over a bounded sample of tokens: the
    first n tokens of the batch (n sized for about budget_s of work, at most
    the whole batch), repeated until at least budget_s / 1.5 has passed.
    threads: cap numpy's BLAS threads (None: all host cores)."""
    import contextlib

    import oracle
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
    except Exception:
        threadpool_info = threadpool_limits = None
    ctx = threadpool_limits(threads) if (threads and threadpool_limits) else contextlib.nullcontext()
    with ctx:
        if threadpool_info:
            cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
        else:
            cores = threads or os.cpu_count() or 1
        n = 2
        t0 = time.time()
        oracle.forward(x[:n], W, wl.top_k)
        dt = time.time() - t0
        n = int(min(wl.T, max(n, n * budget_s / max(dt, 1e-3))))
        passes, tokens = 0, 0
        t0 = time.time()
        while passes == 0 or time.time() - t0 < budget_s / 1.5:
            oracle.forward(x[:n], W, wl.top_k)
            passes += 1
            tokens += n
        dt = time.time() - t0
    return {"value": tokens / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": "first %d of the %d tokens of the %s batch x %d passes, fp64 numpy, %.1f s"
                      % (n, wl.T, wl.name, passes, dt)}


def stored_mfma(kernel, workload):
    """MFMA counters of the expert GEMMs stored for this workload (profiles/),
    while the kernel's sources are those the counters were taken on."""
    path = os.path.join(PROFILES, "mfma_%s_%s.json" % (kernel, workload))
    if not os.path.exists(path):
        return None
    d = json.load(open(path))
    if d.get("source_sha") != source_sha(kernel):
        return None
    return {k: d[k] for k in ("mfma_busy_frac", "executed_over_algorithmic", "executed_tflop_per_launch",
                              "algorithmic_tflop_per_launch") if k in d}


def stored_traffic(kernel, workload, stage=None):
    """HBM traffic counters stored for a kernel's launch (of a layer stage), if taken
    on the current sources."""
    name = "traffic_%s_%s.json" % (kernel, workload) if stage is None else \
        "traffic_%s_%s_%s.json" % (kernel, workload, stage)
    path = os.path.join(PROFILES, name)
    if not os.path.exists(path):
        return None
    d = json.load(open(path))
    if d.get("source_sha") != source_sha(kernel):
        return None    # the kernel changed since the counters were taken
    if stage is not None and d.get("stage") != stage:
        return None
    return d


EXTRA_WORKLOADS = ("super_prefill", "ultra", "super_fp4")   # reported beside the headline


def measure(name, args, steps, warmup, tokens=0, cpu_budget=15.0, cpu_1thread=False):
    """One workload: graph-replayed timed steps (per-step HIP events for the
    spread), eager steps with stage events for the roofline, and the oracle on
    the host.  Returns the JSON fields of that workload."""
    import torch

    from sparse_moe_layer_logits_amd import binding, synth

    wl = synth.WORKLOADS[name]
    redraw_from = wl.name
    if tokens:
        # the same layer at another batch size: token rows are drawn per row, so
        # a smaller T is a prefix of the batch; super_verify's redraw table
        # covers the decode router up to 512 rows
        import dataclasses
        if tokens > wl.T and wl.name == "super_decode":
            redraw_from = "super_verify"
        elif tokens > wl.T:
            raise SystemExit("--tokens above %d needs a workload whose batch has that many rows" % wl.T)
        wl = dataclasses.replace(wl, T=tokens)
    t0 = time.time()
    redraws = {t: a for t, a in synth.load_redraws(redraw_from, args.seed).items() if t < wl.T}
    x, W = synth.make(wl, args.seed, redraws=redraws)
    log("generated %s inputs in %.1fs" % (wl.name, time.time() - t0))
    torch.cuda.set_device(0)
    Wd = binding.upload_weights(W)
    xd = binding.to_device(x)
    stream = torch.cuda.current_stream()
    layer = binding.LatentMoE(wl, Wd, max_tokens=wl.T, stream=stream)
    y = torch.empty((wl.T, wl.d), dtype=torch.float32, device="cuda")
    idx = torch.empty((wl.T, wl.top_k), dtype=torch.int32, device="cuda")
    gates = torch.empty((wl.T, wl.top_k), dtype=torch.float32, device="cuda")

    for _ in range(warmup):
        layer.forward(xd, y, idx, gates)
    torch.cuda.synchronize()
    counts = layer.intermediate("counts", (wl.n_experts,), torch.int32).cpu().numpy()
    touched = int((counts > 0).sum())
    log("%s: warmup done; %d experts touched" % (wl.name, touched))

    # timed region 1: the step as a serving loop runs it (graph replay of the
    # forward), with an event on the stream between steps for the per-step spread
    for _ in range(3):
        layer.forward(xd, y, idx, gates, graph=True)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(steps):
        layer.forward(xd, y, idx, gates, graph=True)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    per_step = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)])
    ms_per_step = 1e3 * elapsed / steps
    tokens_per_s = wl.T * steps / elapsed
    log("%s: timed %d graph-replayed steps: %.4f ms/step (p10 %.4f, median %.4f, p90 %.4f)"
        % (wl.name, steps, ms_per_step, *np.percentile(per_step, [10, 50, 90])))

    # timed region 2: the same steps launched eagerly with HIP events around
    # each stage; stage-timed forwards run every stage in program order on one
    # stream, so each stage's time is its own kernels' (durations for the roofline)
    layer.profile_begin(steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        layer.forward(xd, y, idx, gates)
    torch.cuda.synchronize()
    eager_ms = 1e3 * (time.perf_counter() - t0) / steps
    stage_ms, calls = layer.profile_end()
    log("%s: timed %d eager steps with stage events: %.4f ms/step" % (wl.name, steps, eager_ms))
    for k, v in stage_ms.items():
        log("  stage %-12s %.4f ms" % (k, v / max(calls, 1)))

    alg_bytes, alg_flops = algorithmic(wl, touched)
    step_s = ms_per_step / 1e3
    hbm_bound = alg_flops / alg_bytes < 1e3 * BF16_PEAK_TFLOPS / HBM_PEAK_GBS
    dom = max(("expert_up", "expert_down"), key=lambda s: stage_ms[s])
    dom_s = stage_ms[dom] / calls / 1e3
    kb, kf = expert_kernel_units(wl, touched, dom)
    kernel = expert_kernel(wl)
    if hbm_bound:
        achieved, peak, unit, bound = kb / dom_s / 1e9, HBM_PEAK_GBS, "GB/s", "hbm"
    else:
        achieved, peak, unit, bound = kf / dom_s / 1e12, BF16_PEAK_TFLOPS, "TFLOP/s", "mfma"
    # counter data is stored for the workloads' own batch sizes only
    tr = None if tokens else stored_traffic(kernel, wl.name, dom)
    traffic = None if tr is None else tr["hbm_bytes_per_launch"]
    roofline = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4), "traffic": traffic,
                "kernel": "%s (%s)" % (kernel, dom), "launch_ms": round(dom_s * 1e3, 5),
                "source_sha": source_sha(kernel),
                "alg_bytes_per_launch": int(kb), "alg_flops_per_launch": kf}
    mf = None if tokens else stored_mfma(kernel, wl.name)
    if mf is not None:
        roofline["mfma_counters"] = mf
    res = {
        "value": round(tokens_per_s, 1), "ms_per_step": round(ms_per_step, 5),
        "step_ms_p10": round(float(np.percentile(per_step, 10)), 5),
        "step_ms_median": round(float(np.median(per_step)), 5),
        "step_ms_p90": round(float(np.percentile(per_step, 90)), 5),
        "config": {"workload": wl.name, "T": wl.T, "d": wl.d, "latent": wl.latent,
                   "n_experts": wl.n_experts, "top_k": wl.top_k, "expert_hidden": wl.expert_hidden,
                   "shared_hidden": wl.shared_hidden, "experts": wl.experts, "shared": wl.shared,
                   "projections": wl.proj, "router": wl.router,
                   "seed": args.seed, "parallelism": "single GPU"},
        "roofline": roofline,
        "layer": {"alg_bytes": int(alg_bytes), "alg_flops": alg_flops, "experts_touched": touched,
                  "bound": "hbm" if hbm_bound else "mfma",
                  "eager_ms_per_step_with_events": round(eager_ms, 5),
                  "hbm_frac": round(alg_bytes / step_s / 1e9 / HBM_PEAK_GBS, 4),
                  "mfma_frac": round(alg_flops / step_s / 1e12 / BF16_PEAK_TFLOPS, 4),
                  "stage_ms": {k: round(v / max(calls, 1), 5) for k, v in stage_ms.items()}},
    }
    layer.close()
    del Wd, xd, y, idx, gates
    torch.cuda.empty_cache()
    if cpu_budget > 0:
        log("%s: timing the fp64 oracle on the host" % wl.name)
        res["cpu_baseline"] = cpu_baseline(wl, x, W, budget_s=cpu_budget)
        if cpu_1thread:
            res["cpu_baseline_1thread"] = cpu_baseline(wl, x, W, budget_s=cpu_budget / 2, threads=1)
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="super_decode")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--tokens", type=int, default=0,
                    help="batch size T instead of the workload's (e.g. speculative-verify sweeps)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-workloads", action="store_true",
                    help="measure the headline workload only (no prefill / Ultra / FP4 entries)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run a plain fp32 copy kernel of this size (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: there is no multi-GPU path (expert-parallel "
              "sharding is not built); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    from sparse_moe_layer_logits_amd import synth as _synth
    if args.workload in _synth.SSM_WORKLOADS:
        return bench_ssm(args)

    cpu = 0.0 if args.no_cpu_baseline else 15.0
    # the headline: the decode step (one 1-thread oracle run beside it, as for tiny and Ultra)
    head = measure(args.workload, args, args.steps, args.warmup, tokens=args.tokens, cpu_budget=cpu,
                   cpu_1thread=bool(cpu) and args.workload in ("tiny", "super_decode", "ultra"))
    result = {
        "metric": METRIC, "value": head["value"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": head["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded normal weights and tokens, N(0, 1/fan_in))",
    }
    result.update({k: v for k, v in head.items() if k not in ("value", "ms_per_step")})
    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib)
    if not args.no_workloads and not args.tokens and args.workload == "super_decode":
        # the other configurations the metric names, each with its own roofline: the
        # prefill chunk (MFMA-bound), the Ultra shape and FP4 experts (HBM-bound)
        result["workloads"] = {}
        for name in EXTRA_WORKLOADS:
            result["workloads"][name] = measure(name, args, args.steps, args.warmup,
                                                cpu_budget=cpu / 2, cpu_1thread=bool(cpu) and name == "ultra")
        if cpu:
            from sparse_moe_layer_logits_amd import synth
            wl = synth.WORKLOADS["tiny"]
            x, W = synth.make(wl, args.seed, redraws=synth.load_redraws("tiny", args.seed))
            result["cpu_baseline_tiny_1thread"] = cpu_baseline(wl, x, W, budget_s=4.0, threads=1)
    print(json.dumps(result), flush=True)


def copy_probe(mib):
    """Elementwise copy that reads and writes exactly mib MiB per launch (counter
    calibration for the FETCH_SIZE / WRITE_SIZE runs)."""
    import torch
    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(5):
        torch.mul(a, 1.0, out=b)
    torch.cuda.synchronize()
    log("copy probe: 5 launches of %d MiB read + %d MiB write" % (mib, mib))


SSM_METRIC = "Mamba-2 speculative-verify tokens/s (checkpoint + replay); % HBM peak"


def ssm_bytes(wl, lens):
    """Algorithmic HBM bytes of one checkpoint + replay verify launch: every head's
    checkpoint once, the buffered and new records, the outputs and the appended
    records."""
    R, T, H, G, P, N = wl.R, wl.T, wl.H, wl.G, wl.P, wl.N
    n = int(np.sum(lens))
    state = R * H * P * N * 2
    reads = (n + 2 * R * T) * G * N * 2 + (n + R * T) * (H * P * 2 + H * 4)
    writes = R * T * H * P * 4 + R * T * (G * N * 2 + H * P * 2 + H * 4)
    return state + reads + writes


def bench_ssm(args):
    import torch

    from sparse_moe_layer_logits_amd import binding, synth

    wl = synth.SSM_WORKLOADS[args.workload]
    d = synth.make_ssm(wl, args.seed)
    torch.cuda.set_device(0)
    dev = {k: binding.to_device(v) for k, v in d.items()}
    shape = binding.ssm_shape(wl.H, wl.G, wl.P, wl.N, wl.cap)
    st = torch.cuda.current_stream()
    y = torch.empty((wl.R, wl.T, wl.H, wl.P), dtype=torch.float32, device="cuda")
    states = torch.empty((wl.R, wl.T, wl.H, wl.P, wl.N), dtype=torch.int16, device="cuda")
    lens0 = dev["buf_len"].clone()

    def verify():
        binding.ssm_replay_verify(shape, wl.R, wl.T, dev["ckpt"].data_ptr(), dev["buf_k"].data_ptr(),
                                  dev["buf_v"].data_ptr(), dev["buf_a"].data_ptr(), dev["buf_len"].data_ptr(),
                                  dev["draft_q"].data_ptr(), dev["draft_k"].data_ptr(),
                                  dev["draft_v"].data_ptr(), dev["draft_a"].data_ptr(), y.data_ptr(),
                                  st.cuda_stream)

    def states_scheme():
        binding.ssm_states_verify(shape, wl.R, wl.T, dev["ckpt"].data_ptr(), dev["draft_q"].data_ptr(),
                                  dev["draft_k"].data_ptr(), dev["draft_v"].data_ptr(),
                                  dev["draft_a"].data_ptr(), states.data_ptr(), y.data_ptr(), st.cuda_stream)

    def timed(fn, steps, before=None):
        """Mean ms per call, HIP events on the calls' stream around each call."""
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for e0, e1 in ev:
            if before:
                before()
            e0.record(st)
            fn()
            e1.record(st)
        torch.cuda.synchronize()
        return sum(e0.elapsed_time(e1) for e0, e1 in ev) / steps

    for _ in range(args.warmup):
        verify()
        states_scheme()
    torch.cuda.synchronize()
    # timed region: K verify steps back to back (the buffer counters are not advanced,
    # so every step appends to the same slots and reads the same records)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        verify()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = 1e3 * elapsed / args.steps
    verify_ms = timed(verify, args.steps)
    states_ms = timed(states_scheme, args.steps)
    ckpt0 = dev["ckpt"].clone()

    def restore():
        dev["buf_len"].copy_(lens0)
        dev["ckpt"].copy_(ckpt0)

    def flush():
        binding.ssm_replay_flush(shape, wl.R, dev["ckpt"].data_ptr(), dev["buf_k"].data_ptr(),
                                 dev["buf_v"].data_ptr(), dev["buf_a"].data_ptr(), dev["buf_len"].data_ptr(),
                                 st.cuda_stream)
    flush_ms = timed(flush, max(1, args.steps // 4), before=restore)
    restore()
    torch.cuda.synchronize()

    lens = d["buf_len"]
    kb = ssm_bytes(wl, lens)
    tr = stored_traffic("ssm_verify_kernel", wl.name)
    traffic = None if tr is None else tr["hbm_bytes_per_launch"]
    states_bytes = wl.R * wl.H * wl.P * wl.N * 2 * (1 + wl.T) + wl.R * wl.T * wl.H * wl.P * 4
    achieved = kb / (verify_ms * 1e-3) / 1e9
    tokens = wl.R * wl.T
    log("verify %.4f ms (events) / %.4f ms (wall), state-writing scheme %.4f ms, flush %.4f ms"
        % (verify_ms, ms_per_step, states_ms, flush_ms))
    result = {
        "metric": SSM_METRIC, "value": round(tokens / (ms_per_step * 1e-3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded normal states, keys, values, queries; Mamba-2 decay ranges)",
        "config": {"workload": wl.name, "requests": wl.R, "tokens_per_request": wl.T, "heads": wl.H,
                   "groups": wl.G, "head_dim": wl.P, "state_dim": wl.N, "buffer_capacity": wl.cap,
                   "buffered_records_mean": float(np.mean(lens)), "seed": args.seed,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "ssm_verify_kernel", "launch_ms": round(verify_ms, 5),
                     "source_sha": source_sha("ssm_verify_kernel"),
                     "alg_bytes_per_launch": int(kb)},
        "state_writing_scheme": {"launch_ms": round(states_ms, 5), "alg_bytes_per_launch": int(states_bytes),
                                 "achieved_GBs": round(states_bytes / (states_ms * 1e-3) / 1e9, 2),
                                 "replay_speedup": round(states_ms / verify_ms, 3)},
        "flush": {"launch_ms": round(flush_ms, 5),
                  "alg_bytes_per_launch": int(wl.R * wl.H * wl.P * wl.N * 4)},
    }
    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib)
    if not args.no_cpu_baseline:
        log("timing the fp64 oracle on the host")
        result["cpu_baseline"] = ssm_cpu_baseline(wl, d)
    print(json.dumps(result), flush=True)


def ssm_cpu_baseline(wl, d, budget_s=10.0):
    """The fp64 recurrence oracle on the host cores over whole requests, repeated
    for about budget_s."""
    import oracle
    from oracle.formats import bf16_to_f64 as f
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count() or 1
    t0 = time.time()
    tokens, r = 0, 0
    while time.time() - t0 < budget_s or tokens == 0:
        n = int(d["buf_len"][r % wl.R])
        rr = r % wl.R
        oracle.ssm.verify_outputs(f(d["ckpt"][rr]), f(d["buf_k"][rr]), f(d["buf_v"][rr]),
                                  d["buf_a"][rr].astype(np.float64), n, f(d["draft_q"][rr]),
                                  f(d["draft_k"][rr]), f(d["draft_v"][rr]), d["draft_a"][rr].astype(np.float64))
        tokens += wl.T
        r += 1
    dt = time.time() - t0
    return {"value": tokens / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": "%d whole requests (%d tokens each) of the %s batch, fp64 numpy recurrence, %.1f s"
                      % (r, wl.T, wl.name, dt)}


if __name__ == "__main__":
    main()
