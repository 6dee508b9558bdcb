"""Benchmark of the WKV-7 hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--decode-steps S] [--no-cpu-baseline]

One timed step = one whole-sequence prefill of the L12-D768 layer workload
(B=8, T=4096, H=12, N=64, bfloat16 inputs, float32 state carried in and out)
through the C ABI with the library's default algorithm. The batched decode
step (D2048 shape: B=512, H=32, 256 consecutive in-place steps) is timed in the
same run and reported under "decode", and again with the state stored as
bfloat16 and as float16 ("decode_state_bf16", "decode_state_f16"); the fused
time-mix step under "decode_fused"; and the backward (gradients of the
recurrence) at the prefill shape under "backward". Inputs are seeded synthetic
tensors, resident in HBM before timing starts.

Prints one JSON line. "value" is prefill tokens*heads per second. "roofline"
relates the dominant kernel's algorithmic bytes (or flops) per launch to its
mean launch time (HIP events on the launch stream) and to MI355X's published
peak. "cpu_baseline" is the float64 oracle timed on this host's cores.
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
PEAK_MFMA_BF16_TFLOPS = 2500.0  # dense
PEAK_FP32_VECTOR_TFLOPS = 157.3
FLOP_REC = 9 * N * N  # per token*head: S a (2N^2), update (5N^2), S r (2N^2)
# backward per token*head: the forward state rebuilt (S a 2N^2, update 6N^2) and the
# reverse step (G += dy r^T, dr, dk, dw, dv, G b, da, db: 2N^2 each; G update 4N^2)
FLOP_BWD = 26 * N * N
METRIC = "WKV7 tokens*heads/sec (prefill & decode step) + % of HBM/MFMA roofline"
UNIT = "tokens*heads/s"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


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


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=256)
    ap.add_argument("--decode-reps", type=int, default=3)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-decode-16bit", action="store_true", help="skip the bf16 / f16 stored-state decode legs")
    ap.add_argument("--no-decode-fused", action="store_true", help="skip the fused time-mix decode leg")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward leg")
    ap.add_argument("--no-stack", action="store_true", help="skip the multi-layer prompt-then-steps leg")
    ap.add_argument("--stack-steps", type=int, default=32)
    ap.add_argument("--backward-reps", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--algo", type=int, default=0, help="0 auto, 1 sequential, 2 chunked (fused), 3 chunked (split)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (reference for HBM byte counters)")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the WKV-7 units (batch, head) are independent, so a "
              "multi-GPU run would shard batch or heads with no communication; run with --gpus 1.",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from linear_rnn_amd import wkv
    from linear_rnn_amd.inputs import CONFIGS, make_inputs

    wkv.lib()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev_name = torch.cuda.get_device_name(0)

    # ------------------------------------------------------------------ prefill
    cfg = CONFIGS["L12-D768-prefill"]
    B, T, H = cfg.B, cfg.T, cfg.H
    x = make_inputs(cfg)
    d = to_dev(x, torch)
    s_in = torch.from_numpy(x["state_in"]).cuda()
    y = torch.empty((B, T, H, N), dtype=torch.float32, device="cuda")
    s_out = torch.empty((B, H, N, N), dtype=torch.float32, device="cuda")
    # the library's default for bfloat16 inputs is the split chunked algorithm
    algo = args.algo if args.algo else wkv.RWKV7_ALGO_CHUNKED_SPLIT

    def prefill():
        wkv.rwkv7_wkv_prefill_ex(d["r"], d["w"], d["k"], d["v"], d["a"], d["b"], s_in, y, s_out, algo=algo)

    for _ in range(args.warmup):
        prefill()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms = time_region(torch, prefill, args.steps)
    wall = time.perf_counter() - t0
    tok_heads = B * T * H
    value = tok_heads / (ms * 1e-3)

    nbytes = algo_bytes(B, T, H)
    if algo == wkv.RWKV7_ALGO_SEQUENTIAL:
        kname, src = "wkv7_seq_kernel", ["linear_rnn_amd/csrc/wkv7_seq.hip", "linear_rnn_amd/csrc/wkv7_device.hpp"]
        flops = FLOP_REC * tok_heads
        roof = {"bound": "alu", "achieved": flops / (ms * 1e-3) / 1e12, "peak": PEAK_FP32_VECTOR_TFLOPS,
                "unit": "TFLOP/s"}
    elif algo == wkv.RWKV7_ALGO_CHUNKED:
        kname, src = "wkv7_chunk_kernel", ["linear_rnn_amd/csrc/wkv7_chunk.hip",
                                           "linear_rnn_amd/csrc/wkv7_device.hpp"]
        roof = {"bound": "hbm", "achieved": nbytes / (ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    else:
        kname, src = "wkv7_prep_kernel+wkv7_scan_kernel", ["linear_rnn_amd/csrc/wkv7_split.hip",
                                                           "linear_rnn_amd/csrc/wkv7_device.hpp"]
        roof = {"bound": "hbm", "achieved": nbytes / (ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(kname + ":" + cfg.name, src)
    roof["kernel"] = kname
    roof["algorithmic_bytes"] = nbytes
    roof["hbm_frac_of_peak"] = nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS

    out = {
        "metric": METRIC, "value": value, "unit": UNIT, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32" if algo == wkv.RWKV7_ALGO_SEQUENTIAL else "bf16",
        "data": "synthetic (seeded; RWKV-7 layer-shaped distributions)",
        "config": {"workload": "%s: B=%d T=%d H=%d N=%d bf16 inputs, fp32 state in/out" % (cfg.name, B, T, H, N),
                   "B": B, "T": T, "H": H, "N": N, "algo": {1: "sequential", 2: "chunked-fused", 3: "chunked-split"}[algo]},
        "roofline": roof, "device": dev_name, "timed_wall_s": wall,
    }

    # ------------------------------------------------------------------ decode
    if not args.no_decode:
        out["decode"] = bench_decode(torch, wkv, make_inputs, CONFIGS["D2048-decode"], args)
        if not args.no_decode_16bit:
            for fmt in ("bf16", "f16"):
                out["decode_state_" + fmt] = bench_decode(torch, wkv, make_inputs, CONFIGS["D2048-decode"], args, fmt)

    if not args.no_decode and not args.no_decode_fused:
        out["decode_fused"] = bench_decode_fused(torch, wkv, CONFIGS["D2048-decode"], args)

    if not args.no_backward:
        out["backward"] = bench_backward(torch, wkv, x, d, s_in, cfg, args)

    if not args.no_stack:
        out["stack"] = bench_stack(torch, wkv, args)

    if args.copy_calibration:
        a = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        bcopy = torch.empty_like(a)
        for _ in range(3):
            bcopy.copy_(a)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = {"read": a.numel() * 4, "write": a.numel() * 4}

    # ------------------------------------------------------------------ CPU oracle
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(x)

    print(json.dumps(out), flush=True)
    return 0


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


def bench_backward(torch, wkv, x, d, s_in, cfg, args):
    """Gradients of the recurrence (dr, dw, dk, dv, da, db, dstate_in) at the prefill shape, from seeded
    dy and dstate_out; one call = checkpoint forward, reverse pass and (two row blocks) column-sum add."""
    from linear_rnn_amd.inputs import make_cotangents
    B, T, H = cfg.B, cfg.T, cfg.H
    ct = make_cotangents(B, T, H, seed=cfg.seed)
    dy = torch.from_numpy(ct["dy"]).cuda()
    ds = torch.from_numpy(ct["dstate_out"]).cuda()
    grads = [torch.empty((B, T, H, N), dtype=torch.float32, device="cuda") for _ in range(6)]
    dsi = torch.empty_like(ds)

    def bwd():
        wkv.rwkv7_wkv_backward(d["r"], d["w"], d["k"], d["v"], d["a"], d["b"], s_in, dy, ds, *grads, dsi)

    for _ in range(2):
        bwd()
    ms = time_region(torch, bwd, args.backward_reps)
    tok_heads = B * T * H
    flops = FLOP_BWD * tok_heads
    # inputs (bf16) and dy read, six float32 gradients written, states in and out
    nbytes = tok_heads * N * (6 * 2 + 4 + 6 * 4) + 3 * B * H * N * N * 4
    return {
        "value": tok_heads / (ms * 1e-3), "unit": UNIT, "ms_per_call": ms, "reps": args.backward_reps,
        "config": {"workload": "%s: B=%d T=%d H=%d N=%d bf16 inputs, fp32 state_in, dy, dstate_out; fp32 "
                               "gradients" % (cfg.name, B, T, H, N), "B": B, "T": T, "H": H, "N": N},
        "roofline": {"bound": "alu", "achieved": flops / (ms * 1e-3) / 1e12, "peak": PEAK_FP32_VECTOR_TFLOPS,
                     "unit": "TFLOP/s", "frac": flops / (ms * 1e-3) / 1e12 / PEAK_FP32_VECTOR_TFLOPS,
                     "traffic": measured_traffic("wkv7_ckpt_kernel+wkv7_bwd_kernel+wkv7_colsum_kernel:" + cfg.name,
                                                 ["linear_rnn_amd/csrc/wkv7_bwd.hip",
                                                  "linear_rnn_amd/csrc/wkv7_device.hpp"]),
                     "kernel": "wkv7_ckpt_kernel+wkv7_bwd_kernel+wkv7_colsum_kernel",
                     "algorithmic_flops": flops, "algorithmic_bytes": nbytes,
                     "hbm_frac_of_peak": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS},
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

    def tmc():
        wkv.rwkv7_tmix_prefill_ex(*(dt[n] for n in names), dt["ln_w"], dt["ln_b"], dt["state_in"], o, so,
                                  algo=wkv.RWKV7_ALGO_CHUNKED_SPLIT)

    tmc()
    ms_tmix_ch = time_region(torch, tmc, 5)
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
            "ms": ms_tmix_ch, "share_of_prompt": ms_tmix_ch * L / ms_prompt,
            "roofline": {"bound": "hbm", "achieved": tm_bytes / (ms_tmix_ch * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": tm_bytes / (ms_tmix_ch * 1e-3) / 1e9 / PEAK_HBM_GBS,
                         "kernel": "wkv7_prep_kernel<time-mix> + wkv7_scan_kernel + tmix_ln_kernel",
                         "algorithmic_bytes": tm_bytes, "traffic": None}},
        "tmix_prefill_sequential": {
            "ms": ms_tmix,
            "roofline": {"bound": "alu", "achieved": flops / (ms_tmix * 1e-3) / 1e12,
                         "peak": PEAK_FP32_VECTOR_TFLOPS, "unit": "TFLOP/s",
                         "frac": flops / (ms_tmix * 1e-3) / 1e12 / PEAK_FP32_VECTOR_TFLOPS,
                         "kernel": "wkv7_tmix_kernel (TB=16)", "traffic": None}},
    }


def cpu_baseline(x):
    """Time the float64 oracle (as it stands) on the prefill workload, on every host core."""
    import oracle
    oracle.build(force=False)
    th = oracle.default_threads()
    B, T, H = x["r"].shape[:3]
    times = []
    budget = 20.0
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        oracle.wkv7(*(x[n] for n in "rwkvab"), state_in=x["state_in"], nthreads=th)
        times.append(time.perf_counter() - t0)
        if len(times) >= 5 or time.perf_counter() - t_start > budget / 2:
            break
    sec = sorted(times)[len(times) // 2]
    return {"value": B * T * H / sec, "unit": UNIT, "cores": th, "kind": "oracle",
            "sample": "whole prefill workload (B=%d T=%d H=%d), float64, median of %d runs, %.3f s each"
                      % (B, T, H, len(times), sec),
            "cpu_model": cpu_model()}


if __name__ == "__main__":
    sys.exit(main())
