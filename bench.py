"""Benchmark of the WKV-7 hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--quick]

One timed step = one whole-sequence prefill of the D4096-long layer workload (the
largest single-GPU prefill shape: B=4, T=16384, H=64, N=64, bfloat16 inputs, float32
state carried in and out) through the C ABI with the library's automatic algorithm.
Every step is timed on its own with HIP events on the launch stream; before each one
a 1 GiB device buffer is written (outside the events), so no step finds the previous
one's data in the L2 or last-level caches. "value" is B*T*H over the median step time;
the minimum is reported beside it.

The same run also times, each under its own key: the other prefill shapes (L12-D768,
L24-D1024 in one pass and as four 1024-token calls with the state carried), every
chunked algorithm at each prefill shape, the batched decode step (D2048: B=512, H=32,
256 consecutive in-place steps; and at B=2048, a 1 GiB state four times the size of
the last-level cache), the step with a bfloat16 / float16 stored state, the fused
time-mix step, the backward and the multi-layer stack. Inputs are seeded synthetic
tensors resident in HBM before timing starts.

Prints one JSON line. "roofline" relates the headline kernel's algorithmic bytes per
launch to its median launch time and to MI355X's published HBM peak, and gives the
same launch's matrix-core rate against the dense float16 peak. "cpu_baseline" is the
float64 oracle timed on this host's cores over the whole headline workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

N = 64
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, GB/s
PEAK_MFMA_F16_TFLOPS = 2500.0  # dense bf16 / fp16
PEAK_FP32_VECTOR_TFLOPS = 157.3
FLOP_REC = 9 * N * N  # per token*head: S a (2N^2), update (5N^2), S r (2N^2)
# backward per token*head: the forward state rebuilt (S a 2N^2, update 6N^2) and the
# reverse step (G += dy r^T, dr, dk, dw, dv, G b, da, db: 2N^2 each; G update 4N^2)
FLOP_BWD = 26 * N * N
# matrix-core work of the chunked prefill per 16-token chunk of one head, as issued
# (dense count, identity transposes included): the prep's four Grams as bf16 hi/lo
# products (24 MFMAs 16x16x32), its 22 16x16x16 transposes and products, and the
# scan's 4 waves x 10 MFMAs 16x16x32
FLOP_CHUNK16 = 24 * 2 * 16 * 16 * 32 + 22 * 2 * 16 * 16 * 16 + 40 * 2 * 16 * 16 * 32
METRIC = "WKV7 tokens*heads/sec (prefill & decode step) + % of HBM/MFMA roofline"
UNIT = "tokens*heads/s"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
FLUSH_BYTES = 1 << 30
ALGO_NAMES = {1: "sequential", 2: "chunked (one kernel per head)", 3: "chunked (split prep / scan)"}
KERNELS = {  # algorithm -> (kernel names in a trace, source files whose hash keys the counter table)
    1: ("wkv7_seq_kernel", ["linear_rnn_amd/csrc/wkv7_seq.hip", "linear_rnn_amd/csrc/wkv7_device.hpp"]),
    2: ("wkv7_fused_kernel", ["linear_rnn_amd/csrc/wkv7_fused.hip", "linear_rnn_amd/csrc/wkv7_fused.hpp",
                              "linear_rnn_amd/csrc/wkv7_chunk_ops.hpp", "linear_rnn_amd/csrc/wkv7_device.hpp"]),
    3: ("wkv7_prep_kernel+wkv7_scan_kernel", ["linear_rnn_amd/csrc/wkv7_split.hip",
                                               "linear_rnn_amd/csrc/wkv7_chunk_ops.hpp",
                                               "linear_rnn_amd/csrc/wkv7_device.hpp"]),
}


def algo_bytes(B, T, H, in_bytes=2, state_bytes=4):
    """Algorithmic HBM bytes of one call: six inputs and fp32 y per token*head, the state in and out."""
    return B * T * H * (6 * N * in_bytes + N * 4) + 2 * B * H * N * N * state_bytes


def source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel_key, src_files):
    """HBM bytes per launch from the committed counter runs, or None if absent or stale."""
    try:
        with open(TRAFFIC_FILE) as fh:
            tab = json.load(fh)
    except (OSError, ValueError):
        return None
    ent = tab.get(kernel_key)
    if not ent or ent.get("src_sha") != source_hash(src_files):
        return None
    return ent.get("bytes_per_launch")


def to_dev(x, torch):
    import numpy as np
    out = {}
    for n in "rwkvab":
        a = x[n]
        out[n] = torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16) if a.dtype == np.uint16 \
            else torch.from_numpy(a).cuda()
    return out


def time_region(torch, fn, reps):
    """Mean ms per call of `fn` over `reps` back-to-back calls, HIP events on the current stream."""
    st = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(st)
    for _ in range(reps):
        fn()
    e1.record(st)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def time_steps(torch, fn, reps, flush, before=None):
    """ms of each of `reps` calls of `fn`, each between its own HIP events on the current stream (the
    library launches on that stream). Before each call, outside its events: `before()` if given, then
    a write of the whole `flush` buffer, which evicts the previous call's data from the caches."""
    st = torch.cuda.current_stream()
    evs = []
    torch.cuda.synchronize()
    for _ in range(reps):
        if before is not None:
            before()
        flush.fill_(1.0)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(st)
        fn()
        e1.record(st)
        evs.append((e0, e1))
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def med(xs):
    s = sorted(xs)
    return s[len(s) // 2] if len(s) % 2 else 0.5 * (s[len(s) // 2 - 1] + s[len(s) // 2])


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def prefill_roofline(wkv, B, T, H, algo, ms, name):
    """HBM roofline of one prefill call (and its matrix-core rate for the chunked algorithms)."""
    nbytes = algo_bytes(B, T, H)
    kname, src = KERNELS[algo]
    roof = {"bound": "hbm", "achieved": nbytes / (ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(kname + ":" + name, src)
    roof["kernel"] = kname
    roof["algorithmic_bytes"] = nbytes
    if algo in (2, 3):
        flops = B * H * ((T + 15) // 16) * FLOP_CHUNK16
        roof["mfma_flops"] = flops
        roof["mfma_tflops"] = flops / (ms * 1e-3) / 1e12
        roof["mfma_frac"] = roof["mfma_tflops"] / PEAK_MFMA_F16_TFLOPS
    else:
        roof["valu_tflops"] = FLOP_REC * B * T * H / (ms * 1e-3) / 1e12
        roof["valu_frac"] = roof["valu_tflops"] / PEAK_FP32_VECTOR_TFLOPS
    return roof


def prefill_leg(torch, wkv, cfg, d, s_in, steps, warmup, flush, other_algos=True, reps_alt=10, algo=0):
    """Time the prefill of one workload (state in and out) with `algo` (0: the automatic choice), and
    each chunked algorithm."""
    B, T, H = cfg.B, cfg.T, cfg.H
    y = torch.empty((B, T, H, N), dtype=torch.float32, device="cuda")
    s_out = torch.empty((B, H, N, N), dtype=torch.float32, device="cuda")
    chosen = algo
    algo = algo or wkv.rwkv7_wkv_prefill_algo(B, T, H)

    def call(a=chosen):
        return lambda: wkv.rwkv7_wkv_prefill_ex(d["r"], d["w"], d["k"], d["v"], d["a"], d["b"], s_in, y, s_out,
                                                algo=a)

    if warmup:  # the timed pattern (flush, call), so clocks and power settle into the timed loop's state
        time_steps(torch, call(), warmup, flush)
    t0 = time.perf_counter()
    ms_all = time_steps(torch, call(), steps, flush)
    wall = time.perf_counter() - t0
    ms = med(ms_all)
    res = {"value": B * T * H / (ms * 1e-3), "unit": UNIT, "ms_median": ms, "ms_min": min(ms_all),
           "ms_all": ms_all, "steps": steps, "algo": ALGO_NAMES[algo], "timed_wall_s": wall,
           "config": {"workload": "%s: B=%d T=%d H=%d N=%d, bf16 inputs, fp32 state in and out"
                      % (cfg.name, B, T, H, N), "B": B, "T": T, "H": H, "N": N},
           "roofline": prefill_roofline(wkv, B, T, H, algo, ms, cfg.name)}
    if other_algos:
        alt = {}
        for a in (wkv.RWKV7_ALGO_CHUNKED, wkv.RWKV7_ALGO_CHUNKED_SPLIT):
            time_steps(torch, call(a), 10, flush)
            t = time_steps(torch, call(a), reps_alt, flush)
            alt[ALGO_NAMES[a]] = {"ms_median": med(t), "ms_min": min(t),
                                  "hbm_frac": algo_bytes(B, T, H) / (med(t) * 1e-3) / 1e9 / PEAK_HBM_GBS}
        res["by_algorithm"] = alt
    return res


def resume_leg(torch, wkv, cfg, d, s_in, steps, flush, segments=4, warmup=10):
    """The sequence as `segments` consecutive calls with the state carried in place (one step = all calls)."""
    B, T, H = cfg.B, cfg.T, cfg.H
    L = T // segments
    parts = [{n: d[n][:, i * L:(i + 1) * L].contiguous() for n in "rwkvab"} for i in range(segments)]
    ys = [torch.empty((B, L, H, N), dtype=torch.float32, device="cuda") for _ in range(segments)]
    st = torch.empty_like(s_in)

    def reset():
        st.copy_(s_in)

    def run():
        for p, y in zip(parts, ys):
            wkv.rwkv7_wkv_prefill(p["r"], p["w"], p["k"], p["v"], p["a"], p["b"], st, y, st)

    time_steps(torch, run, warmup, flush, before=reset)
    ms_all = time_steps(torch, run, steps, flush, before=reset)
    ms = med(ms_all)
    nbytes = algo_bytes(B, T, H) + 2 * (segments - 1) * B * H * N * N * 4
    return {"value": B * T * H / (ms * 1e-3), "unit": UNIT, "ms_median": ms, "ms_min": min(ms_all),
            "ms_all": ms_all, "algo": ALGO_NAMES[wkv.rwkv7_wkv_prefill_algo(B, L, H)],
            "config": {"workload": "%s as %d calls of %d tokens, state carried in place" % (cfg.name, segments, L),
                       "B": B, "T": T, "H": H, "N": N, "segments": segments},
            "roofline": {"bound": "hbm", "achieved": nbytes / (ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                         "algorithmic_bytes": nbytes, "traffic": None}}


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--algo", type=int, default=0,
                    help="headline algorithm: 0 automatic, 1 sequential, 2 chunked (one kernel), 3 chunked (split)")
    ap.add_argument("--workload", default="D4096-long-prefill",
                    help="prefill workload of the headline (default: the largest single-GPU one)")
    ap.add_argument("--decode-steps", type=int, default=256)
    ap.add_argument("--decode-reps", type=int, default=3)
    ap.add_argument("--quick", action="store_true", help="headline only (for profiling runs)")
    ap.add_argument("--no-shapes", action="store_true", help="skip the other prefill shapes")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-decode-16bit", action="store_true", help="skip the bf16 / f16 stored-state decode legs")
    ap.add_argument("--no-decode-fused", action="store_true", help="skip the fused time-mix decode leg")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward leg")
    ap.add_argument("--no-stack", action="store_true", help="skip the multi-layer prompt-then-steps leg")
    ap.add_argument("--stack-steps", type=int, default=32)
    ap.add_argument("--backward-reps", type=int, default=20)
    ap.add_argument("--backward-warmup", type=int, default=40,
                    help="untimed backward calls first (the clock settles over the first tens of calls)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (reference for HBM byte counters)")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the WKV-7 units (batch, head) are independent, so a "
              "multi-GPU run would shard batch or heads with no communication; run with --gpus 1.",
              file=sys.stderr)
        return 2
    if args.quick:
        args.no_shapes = args.no_decode = args.no_backward = args.no_stack = args.no_cpu_baseline = True

    import torch

    from linear_rnn_amd import wkv
    from linear_rnn_amd.inputs import CONFIGS, make_inputs

    wkv.lib()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev_name = torch.cuda.get_device_name(0)
    flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")

    def log(msg):
        print("[bench] " + msg, file=sys.stderr, flush=True)

    # ------------------------------------------------------------------ headline prefill
    cfg = CONFIGS[args.workload]
    log("generating %s inputs" % cfg.name)
    x = make_inputs(cfg)
    d = to_dev(x, torch)
    s_in = torch.from_numpy(x["state_in"]).cuda()
    log("timing %s prefill" % cfg.name)
    head = prefill_leg(torch, wkv, cfg, d, s_in, args.steps, args.warmup, flush, other_algos=not args.quick,
                       algo=args.algo)
    out = {
        "metric": METRIC, "value": head["value"], "unit": UNIT, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": head["ms_median"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; RWKV-7 layer-shaped distributions, bf16 inputs, fp32 state)",
        "config": dict(head["config"], algo=head["algo"]),
        "roofline": head["roofline"],
        "timing": {"ms_median": head["ms_median"], "ms_min": head["ms_min"], "ms_all": head["ms_all"],
                   "flush_bytes_between_steps": FLUSH_BYTES, "events": "HIP events on the launch stream, per step"},
        "device": dev_name, "timed_wall_s": head["timed_wall_s"],
    }
    if "by_algorithm" in head:
        out["prefill_by_algorithm"] = head["by_algorithm"]
    if not args.no_cpu_baseline:
        log("timing the float64 oracle on the host")
        out["cpu_baseline"] = cpu_baseline(x, cfg)
    del d, x
    torch.cuda.empty_cache()

    # ------------------------------------------------------------------ other prefill shapes
    if not args.no_shapes:
        shapes = {}
        for name in ("D4096-long-prefill", "L12-D768-prefill", "L24-D1024-prefill-resume"):
            if name == cfg.name:
                continue
            c = CONFIGS[name]
            log("timing %s prefill" % name)
            xs = make_inputs(c)
            ds = to_dev(xs, torch)
            si = torch.from_numpy(xs["state_in"]).cuda()
            shapes[name] = prefill_leg(torch, wkv, c, ds, si, args.steps, args.warmup, flush)
            if name.startswith("L24"):
                shapes[name + ":4x1024"] = resume_leg(torch, wkv, c, ds, si, args.steps, flush, warmup=args.warmup)
            del ds, xs
        out["prefill_shapes"] = shapes

    # ------------------------------------------------------------------ decode
    if not args.no_decode:
        log("timing decode steps")
        out["decode"] = bench_decode(torch, wkv, make_inputs, CONFIGS["D2048-decode"], args)
        out["decode_large_state"] = bench_decode_large(torch, wkv, args)
        if not args.no_decode_16bit:
            for fmt in ("bf16", "f16"):
                out["decode_state_" + fmt] = bench_decode(torch, wkv, make_inputs, CONFIGS["D2048-decode"], args, fmt)

    if not args.no_decode and not args.no_decode_fused:
        out["decode_fused"] = bench_decode_fused(torch, wkv, CONFIGS["D2048-decode"], args)

    if not args.no_backward:
        log("timing the backward")
        c = CONFIGS["L12-D768-prefill"]
        xb = make_inputs(c)
        out["backward"] = bench_backward(torch, wkv, xb, to_dev(xb, torch), torch.from_numpy(xb["state_in"]).cuda(),
                                         c, args, flush)

    if not args.no_stack:
        log("timing the layer stack")
        out["stack"] = bench_stack(torch, wkv, args)

    if args.copy_calibration:
        a = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        bcopy = torch.empty_like(a)
        for _ in range(3):
            bcopy.copy_(a)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = {"read": a.numel() * 4, "write": a.numel() * 4}

    print(json.dumps(out), flush=True)
    return 0


def device_decode_inputs(torch, B, H, seed):
    """Decode-step inputs drawn on the device with the distributions of the shared generator
    (r, v ~ N(0,1); k ~ N(0,1)/8; unit removal key; a_lr = sigmoid(N(0,1)); w = exp(-exp(U(-5,-0.5))),
    a = -kk, b = kk a_lr), bfloat16. Used where no oracle comparison needs host copies."""
    g = torch.Generator("cuda").manual_seed(seed)
    sh = (B, 1, H, N)
    r = torch.randn(sh, device="cuda", generator=g)
    v = torch.randn(sh, device="cuda", generator=g)
    k = torch.randn(sh, device="cuda", generator=g) / 8
    kk = torch.randn(sh, device="cuda", generator=g)
    kk = kk / kk.norm(dim=-1, keepdim=True)
    alr = torch.sigmoid(torch.randn(sh, device="cuda", generator=g))
    w = torch.exp(-torch.exp(torch.rand(sh, device="cuda", generator=g) * 4.5 - 5.0))
    bf = lambda t: t.to(torch.bfloat16).contiguous()  # noqa: E731
    return {"r": bf(r), "w": bf(w), "k": bf(k), "v": bf(v), "a": bf(-kk), "b": bf(kk * alr)}


def bench_decode_large(torch, wkv, args, B=2048, H=32, S=64, distinct=16):
    """The float32-state step at B=2048, H=32: a 1 GiB state, four times the 256 MB last-level cache, so
    the state cannot stay cache-resident between steps. `distinct` input sets (50 MB each) cycle over
    S consecutive in-place steps."""
    sets = [device_decode_inputs(torch, B, H, 9000 + i) for i in range(distinct)]
    g = torch.Generator("cuda").manual_seed(9100)
    state = torch.randn((B, H, N, N), device="cuda", generator=g) * 0.1
    y = torch.empty((B, 1, H, N), dtype=torch.float32, device="cuda")

    def run_all():
        for i in range(S):
            dd = sets[i % distinct]
            wkv.rwkv7_wkv_step(dd["r"], dd["w"], dd["k"], dd["v"], dd["a"], dd["b"], state, y, state)

    run_all()
    torch.cuda.synchronize()
    per_step = [time_region(torch, run_all, 1) / S for _ in range(args.decode_reps)]
    ms = med(per_step)
    nbytes = algo_bytes(B, 1, H)
    return {
        "value": B * H / (ms * 1e-3), "unit": UNIT, "ms_per_step": ms, "steps_per_rep": S,
        "reps": args.decode_reps, "ms_per_step_all_reps": per_step,
        "config": {"workload": "D2048 decode at B=%d H=%d N=%d: 1 GiB float32 state (4x the last-level cache), "
                               "%d consecutive in-place steps, bf16 inputs (device-drawn, %d sets cycled)"
                               % (B, H, N, S, distinct), "B": B, "H": H, "N": N, "state": "f32"},
        "roofline": {"bound": "hbm", "achieved": nbytes / (ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                     "kernel": "wkv7_seq_kernel (step tiling, non-temporal state)", "algorithmic_bytes": nbytes,
                     "traffic": measured_traffic("wkv7_seq_kernel:D2048-decode-large-state",
                                                 ["linear_rnn_amd/csrc/wkv7_seq.hip",
                                                  "linear_rnn_amd/csrc/wkv7_device.hpp"])},
    }


def bench_decode(torch, wkv, make_inputs, cfg, args, fmt="f32"):
    """Consecutive in-place single-token steps; fmt is the stored-state format (f32, bf16, f16)."""
    B, H, S = cfg.B, cfg.H, args.decode_steps
    steps = []
    for s in range(S):
        xs = make_inputs(cfg, step=s, with_state=(s == 0))
        if s == 0:
            state = torch.from_numpy(xs["state_in"]).cuda()
            if fmt != "f32":
                state = state.to({"bf16": torch.bfloat16, "f16": torch.float16}[fmt])
        steps.append(to_dev(xs, torch))
    y = torch.empty((B, 1, H, N), dtype=torch.float32, device="cuda")
    step = wkv.rwkv7_wkv_step if fmt == "f32" else wkv.rwkv7_wkv_step_q

    def run_all():
        for dd in steps:
            step(dd["r"], dd["w"], dd["k"], dd["v"], dd["a"], dd["b"], state, y, state)

    run_all()  # warm-up pass
    torch.cuda.synchronize()
    per_step = []
    for _ in range(args.decode_reps):
        per_step.append(time_region(torch, run_all, 1) / S)
    ms = float(sorted(per_step)[len(per_step) // 2])
    nbytes = algo_bytes(B, 1, H, state_bytes=4 if fmt == "f32" else 2)
    src = ["linear_rnn_amd/csrc/wkv7_seq.hip", "linear_rnn_amd/csrc/wkv7_device.hpp"]
    kern = "wkv7_seq_kernel" if fmt == "f32" else "wkv7_step_kernel"
    key = kern + ":" + cfg.name + ("" if fmt == "f32" else ":state-" + fmt)
    return {
        "value": B * H / (ms * 1e-3), "unit": UNIT, "ms_per_step": ms, "steps_per_rep": S,
        "reps": args.decode_reps, "ms_per_step_all_reps": per_step,
        "config": {"workload": "%s: B=%d H=%d N=%d, %d consecutive in-place steps, bf16 inputs, %s stored state"
                   % (cfg.name, B, H, N, S, fmt), "B": B, "H": H, "N": N, "state": fmt},
        "roofline": {"bound": "hbm", "achieved": nbytes / (ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                     "traffic": measured_traffic(key, src),
                     "kernel": "%s (%s state)" % (kern, fmt), "algorithmic_bytes": nbytes},
    }


def bench_decode_fused(torch, wkv, cfg, args, distinct=32):
    """Consecutive in-place steps of the fused time-mix operator (prologue, recurrence, ln_x) at the
    decode shape. `distinct` seeded input sets are resident and cycled over the steps."""
    import numpy as np
    from linear_rnn_amd.inputs import make_tmix_inputs
    B, H, S = cfg.B, cfg.H, args.decode_steps
    names = ("r", "w_raw", "k", "v", "kk", "a_lr")
    sets = []
    for s in range(min(distinct, S)):
        x = make_tmix_inputs(cfg, step=s, with_state=(s == 0))
        if s == 0:
            state = torch.from_numpy(x["state_in"]).cuda()
            ln_w = torch.from_numpy(x["ln_w"]).cuda()
            ln_b = torch.from_numpy(x["ln_b"]).cuda()
        d = {}
        for n in names:
            a = x[n]
            d[n] = torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16) if a.dtype == np.uint16 \
                else torch.from_numpy(a).cuda()
        sets.append(d)
    o = torch.empty((B, 1, H, N), dtype=torch.float32, device="cuda")

    def run_all():
        for i in range(S):
            d = sets[i % len(sets)]
            wkv.rwkv7_tmix_step(*(d[n] for n in names), ln_w, ln_b, state, o, state)

    run_all()
    torch.cuda.synchronize()
    per_step = [time_region(torch, run_all, 1) / S for _ in range(args.decode_reps)]
    ms = float(sorted(per_step)[len(per_step) // 2])
    # per (b, h): state in and out (fp32), five bf16 inputs and fp32 w_raw, fp32 output; ln_w / ln_b once
    nbytes = B * H * (2 * N * N * 4 + N * (5 * 2 + 4) + N * 4) + 2 * H * N * 4
    src = ["linear_rnn_amd/csrc/wkv7_tmix.hip", "linear_rnn_amd/csrc/wkv7_device.hpp"]
    return {
        "value": B * H / (ms * 1e-3), "unit": UNIT, "ms_per_step": ms, "steps_per_rep": S,
        "reps": args.decode_reps, "ms_per_step_all_reps": per_step,
        "config": {"workload": "%s: B=%d H=%d N=%d, %d consecutive in-place fused steps (decay, normalised "
                               "removal key, slots, recurrence, ln_x), bf16 inputs, fp32 w_raw and state"
                               % (cfg.name, B, H, N, S), "B": B, "H": H, "N": N, "state": "f32",
                   "distinct_input_sets": len(sets)},
        "roofline": {"bound": "hbm", "achieved": nbytes / (ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                     "traffic": measured_traffic("wkv7_tmix_kernel:" + cfg.name, src),
                     "kernel": "wkv7_tmix_kernel (TB=1)", "algorithmic_bytes": nbytes},
    }


BWD_SRC = ["linear_rnn_amd/csrc/wkv7_bwd_chunk.hip", "linear_rnn_amd/csrc/wkv7_fused.hpp",
           "linear_rnn_amd/csrc/wkv7_chunk_ops.hpp", "linear_rnn_amd/csrc/wkv7_device.hpp"]


def bench_backward(torch, wkv, x, d, s_in, cfg, args, flush=None):
    """Gradients of the recurrence (dr, dw, dk, dv, da, db, dstate_in) at the prefill shape, from seeded
    dy and dstate_out. The default (AUTO, bfloat16 inputs) is the chunked backward on MFMA: one launch
    runs the checkpoint forward and the chain of state gradients side by side, a second forms the input
    gradients; after untimed warm-up calls, each call between its own HIP events, after a write of
    `flush` (median and min). The
    token-by-token backward (float32 throughout) is timed beside it."""
    from linear_rnn_amd.inputs import make_cotangents
    B, T, H = cfg.B, cfg.T, cfg.H
    ct = make_cotangents(B, T, H, seed=cfg.seed)
    dy = torch.from_numpy(ct["dy"]).cuda()
    ds = torch.from_numpy(ct["dstate_out"]).cuda()
    grads = [torch.empty((B, T, H, N), dtype=torch.float32, device="cuda") for _ in range(6)]
    dsi = torch.empty_like(ds)
    if flush is None:
        flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")

    def bwd(algo):
        wkv.rwkv7_wkv_backward_ex(d["r"], d["w"], d["k"], d["v"], d["a"], d["b"], s_in, dy, ds, *grads, dsi,
                                  algo=algo)

    algo = wkv.RWKV7_ALGO_AUTO
    ts = time_steps(torch, lambda: bwd(algo), args.backward_warmup + args.backward_reps, flush)[args.backward_warmup:]
    ms, ms_min = med(ts), min(ts)
    tseq = time_steps(torch, lambda: bwd(wkv.RWKV7_ALGO_SEQUENTIAL), 3, flush)[1:]
    tok_heads = B * T * H
    # inputs (bf16) and dy read, six float32 gradients written, state_in and dstate_out read, dstate_in written
    nbytes = tok_heads * N * (6 * 2 + 4 + 6 * 4) + 3 * B * H * N * N * 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {
        "value": tok_heads / (ms * 1e-3), "unit": UNIT, "ms_per_call": ms, "ms_min": ms_min, "reps": len(ts),
        "warmup": args.backward_warmup, "ms_all": ts,
        "algo": "chunked (MFMA)" if d["r"].dtype == torch.bfloat16 else "sequential",
        "config": {"workload": "%s: B=%d T=%d H=%d N=%d bf16 inputs, fp32 state_in, dy, dstate_out; fp32 "
                               "gradients" % (cfg.name, B, T, H, N), "B": B, "T": T, "H": H, "N": N},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": gbs / PEAK_HBM_GBS,
                     "traffic": measured_traffic("wkv7_bpass_kernel+wkv7_bgrad_kernel:" + cfg.name, BWD_SRC),
                     "kernel": "wkv7_bpass_kernel+wkv7_bgrad_kernel", "algorithmic_bytes": nbytes},
        "by_algorithm": {
            "sequential": {"ms": med(tseq), "alu_frac": FLOP_BWD * tok_heads / (med(tseq) * 1e-3) / 1e12 /
                           PEAK_FP32_VECTOR_TFLOPS, "note": "float32 throughout; 26 N^2 flop per token*head"}},
    }


def bench_stack(torch, wkv, args, L=12, H=12, B=8, T=1024):
    """The hybrid mode end to end on a 12-layer stack at the 0.1B width (D=768): a T-token prompt
    through every layer in one call, then single-token calls with the per-layer states carried.
    Synthetic bfloat16 weights. The fused time-mix prefill is also timed alone at the prompt shape,
    both as the chunked prefill (what the stack's prompt runs) and token by token."""
    import numpy as np
    from linear_rnn_amd.inputs import make_stack_inputs
    z = make_stack_inputs(L, B, T, H, "bf16", seed=7100, with_state=False)
    d = {}
    for n, a in z.items():
        d[n] = torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16) if a.dtype == np.uint16 \
            else torch.from_numpy(np.ascontiguousarray(a)).cuda()
    D = H * N
    x = torch.empty_like(d["x"])
    st = torch.empty_like(d["states"])
    xs = torch.randn((B, 1, D), dtype=torch.float32, device="cuda", generator=torch.Generator("cuda").manual_seed(1))

    def prompt():
        x.copy_(d["x"])
        st.zero_()
        wkv.rwkv7_stack_forward(d["w_in"], d["w_out"], d["vecs"], x, st)

    def step():
        wkv.rwkv7_stack_forward(d["w_in"], d["w_out"], d["vecs"], xs, st)

    prompt()
    ms_prompt = time_region(torch, prompt, 3)
    prompt()
    step()
    ms_step = time_region(torch, step, args.stack_steps)
    # the same single-token call captured once in a HIP graph (after the warm-up calls above, so
    # the workspace and the library handles exist) and replayed: launch latency mostly removed
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    with torch.cuda.stream(cap):
        step()  # the workspace and the rocBLAS handle are per stream: create them before capture
        cap.synchronize()
        with torch.cuda.graph(g, stream=cap):
            step()
    torch.cuda.synchronize()
    ms_graph = time_region(torch, g.replay, args.stack_steps)
    # the fused operator alone at the prompt shape (inputs from the first layer's projection scale)
    from linear_rnn_amd.inputs import CONFIGS, make_tmix_inputs
    xt = make_tmix_inputs(CONFIGS["L12-D768-prefill"], B=B, T=T, H=H, seed=7101)
    dt = {n: (torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16) if a.dtype == np.uint16
              else torch.from_numpy(a).cuda()) for n, a in xt.items() if a is not None}
    o = torch.empty((B, T, H, N), dtype=torch.float32, device="cuda")
    so = torch.empty((B, H, N, N), dtype=torch.float32, device="cuda")
    names = ("r", "w_raw", "k", "v", "kk", "a_lr")

    def tm():
        wkv.rwkv7_tmix_prefill(*(dt[n] for n in names), dt["ln_w"], dt["ln_b"], dt["state_in"], o, so)

    tm()
    ms_tmix = time_region(torch, tm, 5)

    # the chunked form the stack's prompt runs at this shape, and the other one beside it
    stack_algo = wkv.rwkv7_wkv_prefill_algo(B, T, H)
    ms_by_algo = {}
    for a in (wkv.RWKV7_ALGO_CHUNKED, wkv.RWKV7_ALGO_CHUNKED_SPLIT):
        def tmc(a=a):
            wkv.rwkv7_tmix_prefill_ex(*(dt[n] for n in names), dt["ln_w"], dt["ln_b"], dt["state_in"], o, so,
                                      algo=a)

        tmc()
        ms_by_algo[a] = time_region(torch, tmc, 5)
    ms_tmix_ch = ms_by_algo[stack_algo]
    # (kernel names as traced, sources keying the counter table); ln_x runs inside the scan in both
    tm_kernel = {wkv.RWKV7_ALGO_CHUNKED: ("wkv7_fused_kernel<1>", KERNELS[2][1]),
                 wkv.RWKV7_ALGO_CHUNKED_SPLIT: ("wkv7_prep_kernel<1>+wkv7_scan_kernel<4, true>", KERNELS[3][1])}
    tm_key = "%s:tmix-B%d-T%d-H%d" % (tm_kernel[stack_algo][0], B, T, H)
    # algorithmic bytes: r, k, v, kk, a_lr (bf16), w_raw and out (float32) per element, the state in and out
    tm_bytes = B * T * H * N * (5 * 2 + 4 + 4) + 2 * B * H * N * N * 4
    flops = FLOP_REC * B * T * H
    return {
        "prompt_tokens_per_s": B * T / (ms_prompt * 1e-3), "ms_per_prompt": ms_prompt,
        "step_tokens_per_s": B / (ms_step * 1e-3), "ms_per_step": ms_step, "steps": args.stack_steps,
        "graph_step_tokens_per_s": B / (ms_graph * 1e-3), "ms_per_graph_step": ms_graph,
        "config": {"workload": "12-layer stack, D=768 (H=12), B=%d, %d-token prompt then single-token calls, "
                               "synthetic bf16 weights, fp32 residual stream and states" % (B, T),
                   "L": L, "B": B, "T": T, "H": H, "N": N},
        "tmix_prefill_chunked": {
            "ms": ms_tmix_ch, "algo": ALGO_NAMES[stack_algo], "share_of_prompt": ms_tmix_ch * L / ms_prompt,
            "by_algorithm": {ALGO_NAMES[a]: {"ms": t} for a, t in ms_by_algo.items()},
            "roofline": {"bound": "hbm", "achieved": tm_bytes / (ms_tmix_ch * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": tm_bytes / (ms_tmix_ch * 1e-3) / 1e9 / PEAK_HBM_GBS,
                         "kernel": tm_kernel[stack_algo][0], "algorithmic_bytes": tm_bytes,
                         "traffic": measured_traffic(tm_key, tm_kernel[stack_algo][1])}},
        "tmix_prefill_sequential": {
            "ms": ms_tmix,
            "roofline": {"bound": "alu", "achieved": flops / (ms_tmix * 1e-3) / 1e12,
                         "peak": PEAK_FP32_VECTOR_TFLOPS, "unit": "TFLOP/s",
                         "frac": flops / (ms_tmix * 1e-3) / 1e12 / PEAK_FP32_VECTOR_TFLOPS,
                         "kernel": "wkv7_tmix_kernel (TB=16)", "traffic": None}},
    }


def cpu_baseline(x, cfg, budget_s=20.0):
    """Time the float64 oracle (as it stands) on the whole headline workload, on every host core, up to
    three runs within about `budget_s`; and on one thread over four (b, h) units of the same workload."""
    import numpy as np

    import oracle
    oracle.build(force=False)
    th = oracle.default_threads()
    B, T, H = x["r"].shape[:3]
    times = []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        oracle.wkv7(*(x[n] for n in "rwkvab"), state_in=x["state_in"], nthreads=th)
        times.append(time.perf_counter() - t0)
        if len(times) >= 3 or time.perf_counter() - t_start > budget_s / 2:
            break
    sec = med(times)
    units = [(0, h) for h in range(min(4, H))]
    sl = {n: np.ascontiguousarray(x[n][:1, :, :len(units)]) for n in "rwkvab"}
    t0 = time.perf_counter()
    oracle.wkv7(*(sl[n] for n in "rwkvab"), state_in=np.ascontiguousarray(x["state_in"][:1, :len(units)]),
                nthreads=1)
    sec1 = time.perf_counter() - t0
    return {"value": B * T * H / sec, "unit": UNIT, "cores": th, "kind": "oracle",
            "sample": "the whole %s prefill (B=%d T=%d H=%d), float64, median of %d runs, %.2f s each"
                      % (cfg.name, B, T, H, len(times), sec),
            "one_thread": {"value": len(units) * T / sec1, "unit": UNIT, "seconds": sec1,
                           "sample": "%d (b, h) units x %d tokens on one thread" % (len(units), T)},
            "cpu_model": cpu_model()}


if __name__ == "__main__":
    sys.exit(main())
