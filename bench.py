"""Benchmark of the w4 hot path on one MI355X.

Headline (the JSON line's `value`): the batch-1 decode GEMV at model size,
x fp16 [1, 2048] times two group-affine 4-bit matrices, K = 2048 x N = 8192
(a fused projection) and K = 2048 x N = 151552 (the vocabulary head).  One
step is both GEMVs.  `value` is the effective HBM bandwidth: algorithmic
bytes (codes + scales + biases + x + y) per step divided by the step time,
with every input already resident in HBM.  Weight copies are rotated so the
working set between two uses of one copy exceeds the 256 MB Infinity Cache.
`stats` adds the spread: the median step time over 30 event-bracketed
rounds of 10 steps, with a 2,000-resample bootstrap 95% interval of that
median, measured after the timed regions.

Also measured and reported under "workloads" (same run, same rules): the
small GEMV (K = N = 512), the prefill GEMM (M = 4096, K = 2048, N = 8192 and
the M sweep), the few-row GEMM, the bf16 variant, the FP8 / NVFP4 codecs,
the decode fusions, the decode MoE layer (one token, 8 of 256 experts +
shared; moe_decode and the three-call path) and the prefill MoE layer (4096
tokens, Zipf-skewed expert loads, two token sets alternating; w4, bf16, FP8
and NVFP4 experts).  "read_probe" gives the chip's measured HBM read rate
(the GEMV's code-load pattern and a plain streaming read, libqlprobe) beside
the 8 TB/s specification; "workloads.lds_probe" the LDS read and write rates
of one CU that bound the GEMM tiles' staging; "cpu_baseline" times the oracle on the host cores
on bounded samples of every workload; "meta" records the device, software,
clocks, seeds and hashes of the inputs and of the sources.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--only-primary]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "w4 GEMV eff. HBM GB/s; w4 GEMM/MoE TFLOP/s; both as % of MI355X peak"
HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0
ROTATE_BYTES = 600e6  # > 2 x 256 MB Infinity Cache
# Untimed settling run before each measurement (after the W warmup steps):
# the clocks reach their sustained level under the measured load within a
# fraction of a second.
SETTLE_S = 0.5
KERNEL_GEMV = "gemv_w4_chunked_kernel<64,1,8,0,0>"  # the K = 2048 vocabulary-head launch


def w4_bytes(K, N):
    return N * K // 2 + 4 * N * (K // 64)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--eager", action="store_true",
                    help="launch graph-timed sections eagerly (for counter collection)")
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--only-primary", action="store_true")
    ap.add_argument("--workload", choices=["all", "gemm", "gemm_prefill", "decode", "bf16", "codecs",
                                           "moe_decode", "moe_prefill", "latency"],
                    default="all",
                    help="secondary workloads to run after the headline (default: all)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pmc-calibration", action="store_true",
                    help="also run a plain copy of known size (for HBM counter calibration)")
    ap.add_argument("--ingest-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter CSVs (FETCH_SIZE, WRITE_SIZE) of "
                         "`bench.py --only-primary --pmc-calibration` into profiles/traffic.json")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------
# timing helpers (events on torch's current stream, which the library uses)
# ----------------------------------------------------------------------------
def timed_steps(step_fn, steps, warmup, settle_s=0.0):
    """Run `warmup` untimed steps (and, with settle_s, keep running untimed
    steps for that many seconds so that the clocks reach their sustained
    level under this load), then time exactly `steps` steps between two
    events on torch's current stream (the stream the library launches on),
    with a synchronize on both sides.  Returns ms per step."""
    import torch
    for i in range(warmup):
        step_fn(i)
    torch.cuda.synchronize()
    t0 = time.time()
    while time.time() - t0 < settle_s:
        for i in range(8):
            step_fn(i)
        torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        step_fn(warmup + i)
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps


def stage_times(stage_fns, steps, warmup, settle_s=0.0):
    """Per-stage time: each stage alone, `steps` back-to-back launches between
    two events (inputs of later stages are left from a full warm-up pass)."""
    out = []
    for fn in stage_fns:
        out.append(timed_steps(fn, steps, warmup, settle_s))
    return out


def round_stats(step_fn, rounds=30, per_round=10, resamples=2000, seed=0):
    """Distribution of the step time: `rounds` event-bracketed rounds of
    `per_round` back-to-back steps (after the main timed region, so that it
    is not perturbed); returns the median ms per step over rounds and a
    bootstrap 95% confidence interval of that median (`resamples` draws of
    the rounds with replacement, percentile interval)."""
    import torch
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(rounds + 1)]
    evs[0].record()
    i = 0
    for r in range(rounds):
        for _ in range(per_round):
            step_fn(i)
            i += 1
        evs[r + 1].record()
    torch.cuda.synchronize()
    per = np.array([evs[r].elapsed_time(evs[r + 1]) / per_round for r in range(rounds)])
    rng = np.random.default_rng(seed)
    boot = np.median(per[rng.integers(0, rounds, size=(resamples, rounds))], axis=1)
    lo, hi = np.percentile(boot, [2.5, 97.5])
    return {"rounds": rounds, "steps_per_round": per_round, "median_ms": float(np.median(per)),
            "ci95_ms": [float(lo), float(hi)], "resamples": resamples}


USE_GRAPHS = True


def graph_time(step_fn, ng, replays):
    """Capture `ng` calls of step_fn(i) in one HIP graph, replay it `replays`
    times between two events; returns ms per call.  With --eager the same
    calls are launched directly instead (for profilers that do not follow
    graph launches)."""
    import torch
    if not USE_GRAPHS:
        return timed_steps(lambda i: step_fn(i % ng), ng * replays, ng)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(ng):
            step_fn(i)
    g.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(replays):
        g.replay()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / (replays * ng)


def source_sha(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "bit_group_quantized_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


INPUTS = {}


def note_inputs(name, seed, *arrays):
    """Record the seed and a SHA-256 of the bytes of a workload's inputs."""
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).view(np.uint8).tobytes())
    INPUTS[name] = {"seed": seed, "sha256_16": h.hexdigest()[:16]}


def w4_arrays(W):
    return (W["qweight"], W["scales"], W["biases"])


def traffic_for(kernel_key, sha):
    """Measured HBM traffic per launch (FETCH_SIZE + WRITE_SIZE, scaled by the
    copy-kernel calibration), if the counters were taken on this source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    ent = d.get(kernel_key)
    if not ent or ent.get("source_sha") != sha:
        return None
    return ent.get("bytes_per_launch")


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------
def dev_w4(W, dev):
    import torch
    return {"qweight": torch.from_numpy(np.ascontiguousarray(W["qweight"]).view(np.int32)).to(dev),
            "scales": torch.from_numpy(W["scales"]).to(dev),
            "biases": torch.from_numpy(W["biases"]).to(dev), "K": W["K"], "N": W["N"]}


def clone_w4(W):
    return {k: (v.clone() if hasattr(v, "clone") else v) for k, v in W.items()}


def bench_gemv(args, dev):
    import torch
    import bit_group_quantized_amd as ql
    import synth
    K = 2048
    Ns = (8192, synth.VOCAB)
    cases = [synth.gemv_case(s, K, N) for s, N in zip((0, 1), Ns)]
    note_inputs("gemv_K2048_N8192", 0, cases[0]["x"], *w4_arrays(cases[0]["W"]))
    note_inputs("gemv_K2048_N151552", 1, cases[1]["x"], *w4_arrays(cases[1]["W"]))
    step_bytes = sum(w4_bytes(K, N) + 2 * K + 2 * N for N in Ns)
    copies = max(2, int(np.ceil(ROTATE_BYTES / step_bytes)))
    base = [dev_w4(c["W"], dev) for c in cases]
    Ws = [base] + [[clone_w4(w) for w in base] for _ in range(copies - 1)]
    x = torch.from_numpy(cases[0]["x"][0]).to(dev)
    ys = [torch.empty(N, dtype=torch.float16, device=dev) for N in Ns]

    def step(i):
        Wc = Ws[i % copies]
        ql.qlinear_gemv(Wc[0], x, ys[0])
        ql.qlinear_gemv(Wc[1], x, ys[1])

    ms = timed_steps(step, args.steps, args.warmup, settle_s=SETTLE_S)
    gbs = step_bytes / (ms * 1e-3) / 1e9
    launch_bytes = [w4_bytes(K, N) + 2 * K + 2 * N for N in Ns]
    # Each matrix alone: back-to-back launches with rotation.  The vocabulary
    # head (the dominant launch) runs the kernel the roofline reports; its
    # timed region holds only launches of that kernel, so its average launch
    # duration is region time / launches.
    kern_ms = []
    for j in range(2):
        kern_ms.append(timed_steps(lambda i, j=j: ql.qlinear_gemv(Ws[i % copies][j], x, ys[j]),
                                   args.steps, args.warmup, settle_s=SETTLE_S / 2))
    kern_ms = np.asarray(kern_ms)
    avg_launch_ms = kern_ms[1]
    avg_launch_bytes = launch_bytes[1]
    achieved = avg_launch_bytes / (avg_launch_ms * 1e-3) / 1e9
    # Spread of the step time (median over rounds and its bootstrap 95%
    # interval), after the timed regions above.
    st_step = round_stats(step)
    to_gbs = lambda b, ms: b / (ms * 1e-3) / 1e9
    stats = {
        "step": dict(st_step, **{"GB/s_median": to_gbs(step_bytes, st_step["median_ms"]),
                                 "GB/s_ci95": [to_gbs(step_bytes, st_step["ci95_ms"][1]),
                                               to_gbs(step_bytes, st_step["ci95_ms"][0])]}),
    }
    # The same step as a replayed HIP graph (launch overhead removed), for context.
    graph_ms = graph_time(step, copies * 2, 20) if copies * 2 <= 64 else None
    # The same two matrices in one launch (qlinear_gemv_multi: they share x),
    # and the projection alone in a graph of back-to-back launches.
    def step_multi(i):
        Wc = Ws[i % copies]
        ql.qlinear_gemv_multi([Wc[0], Wc[1]], x, ys)

    ms_multi = timed_steps(step_multi, args.steps, args.warmup, settle_s=SETTLE_S / 2)
    # (a graph of 64 launches over 64 copies, 605 MB: past the Infinity
    # Cache, and long enough that the replay's own overhead is amortized)
    pc = 64
    Wp = [base[0]] + [clone_w4(base[0]) for _ in range(pc - 1)]
    proj_graph_ms = graph_time(lambda i: ql.qlinear_gemv(Wp[i % pc], x, ys[0]), pc, 20)
    del Wp
    sha = source_sha("gemv.hip", "ql_device.h")
    traffic = traffic_for(KERNEL_GEMV, sha)
    return {
        "value": gbs, "ms_per_step": ms, "step_bytes": step_bytes, "rotation_copies": copies,
        "stats": stats,
        "graph": None if graph_ms is None else {"ms_per_step": graph_ms,
                                                 "GB/s": step_bytes / (graph_ms * 1e-3) / 1e9},
        "per_matrix": {f"N={N}": {"us": float(kern_ms[j] * 1e3),
                                  "GB/s": launch_bytes[j] / (kern_ms[j] * 1e-3) / 1e9}
                       for j, N in enumerate(Ns)},
        "projection_in_graph": {"us": float(proj_graph_ms * 1e3),
                                "GB/s": launch_bytes[0] / (proj_graph_ms * 1e-3) / 1e9,
                                "note": "N=8192 alone: 64 back-to-back launches over 64 weight copies, replayed from a HIP graph"},
        "step_one_launch": {"ms_per_step": ms_multi, "GB/s": step_bytes / (ms_multi * 1e-3) / 1e9,
                            "note": "both matrices in one qlinear_gemv_multi launch (same x)"},
        "roofline": {"bound": "hbm", "kernel": KERNEL_GEMV, "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic, "algorithmic_bytes_per_launch": avg_launch_bytes,
                     "avg_launch_us": float(avg_launch_ms * 1e3), "source_sha": sha},
    }


def bench_gemv_small(args, dev):
    """The small GEMV (x fp16 [1, 512], K = N = 512): 149,504 bytes, which
    stay in the L2 cache from one call to the next, so the call is bound by
    launch and memory latency, not by HBM bandwidth (a correctness-sized
    workload; its GB/s is reported with no roofline claim).  Timed eagerly
    (back-to-back launches between events) and from a replayed HIP graph of
    64 launches (no host launch cost)."""
    import torch
    import bit_group_quantized_amd as ql
    import synth
    K = N = 512
    case = synth.gemv_case(0, K, N)
    note_inputs("gemv_K512_N512", 0, case["x"], *w4_arrays(case["W"]))
    W = dev_w4(case["W"], dev)
    x = torch.from_numpy(case["x"][0]).to(dev)
    y = torch.empty(N, dtype=torch.float16, device=dev)
    step = lambda i: ql.qlinear_gemv(W, x, y)
    ms = timed_steps(step, max(args.steps, 100), args.warmup)
    gms = graph_time(step, 64, 20)
    nbytes = w4_bytes(K, N) + 2 * K + 2 * N
    return {"bytes": nbytes, "eager_us": ms * 1e3, "graph_us": gms * 1e3,
            "GB/s_graph": nbytes / (gms * 1e-3) / 1e9, "GB/s_eager": nbytes / (ms * 1e-3) / 1e9,
            "bound": "latency (L2-resident weights)"}


def bench_gemm(args, dev):
    import torch
    import bit_group_quantized_amd as ql
    import synth
    K, N = 2048, 8192
    out = {}
    for M in (4096, 256, 1024, 16384):
        case = synth.gemm_case(0, M, K, N)
        note_inputs(f"gemm_M{M}_K2048_N8192", 0, case["X"], *w4_arrays(case["W"]))
        W = dev_w4(case["W"], dev)
        X = torch.from_numpy(case["X"]).to(dev)
        Xs = [X] + [X.clone() for _ in range(1 if M >= 4096 else 3)]
        Y = torch.empty((M, N), dtype=torch.float16, device=dev)

        def step(i):
            ql.qlinear_gemm(W, Xs[i % len(Xs)], Y)

        steps = 20 if M <= 4096 else 8
        ms = timed_steps(step, steps, 3, settle_s=SETTLE_S)
        flops = 2.0 * M * N * K
        tf = flops / (ms * 1e-3) / 1e12
        out[f"M={M}"] = {"us": float(ms * 1e3), "TFLOP/s": tf, "frac_mfma_f16": tf / MFMA_F16_PEAK_TFLOPS}
        if M <= 1024:
            # The K-split entry point (K in two halves per workgroup; its own
            # rounding), for the caller who trades qlinear_gemm's bits for speed.
            def step_ks(i):
                ql.qlinear_gemm_ksplit(W, Xs[i % len(Xs)], Y)

            ms_ks = timed_steps(step_ks, steps, 3, settle_s=SETTLE_S / 2)
            tf_ks = flops / (ms_ks * 1e-3) / 1e12
            out[f"M={M}"]["ksplit"] = {"us": float(ms_ks * 1e3), "TFLOP/s": tf_ks,
                                      "frac_mfma_f16": tf_ks / MFMA_F16_PEAK_TFLOPS,
                                      "entry": "qlinear_gemm_ksplit"}
        del Xs, Y, X, W
        torch.cuda.empty_cache()
    return out


def bench_few_rows(args, dev):
    """Few activation rows (verify-sized groups, lightly loaded experts): the
    weight-stationary qlinear_gemm_few_rows next to the tiled qlinear_gemm
    (and qlinear_gemv at one row).  Calls are replayed from a HIP graph (the
    per-call Python path is slower than these kernels) over enough weight
    copies that more than 256 MB pass between two uses of one copy, so the
    weights come from HBM as they would layer after layer."""
    import torch
    import bit_group_quantized_amd as ql
    import synth
    out = {}
    for K, N in ((2048, 8192), (2048, 1024), (512, 2048)):
        case = synth.gemm_case(0, 256, K, N)
        W0 = dev_w4(case["W"], dev)
        ncopy = max(2, -(-300_000_000 // w4_bytes(K, N)))
        Ws = [W0] + [clone_w4(W0) for _ in range(ncopy - 1)]
        Xall = torch.from_numpy(case["X"]).to(dev)
        shape = {}
        for M in (1, 2, 4, 8, 16, 32, 64, 128, 256):
            X = Xall[:M].contiguous()
            Y = torch.empty((M, N), dtype=torch.float16, device=dev)
            flops = 2.0 * M * N * K
            fns = [("few_rows", ql.qlinear_gemm_few_rows), ("tiled", ql.qlinear_gemm)]
            if M == 1:
                fns.append(("gemv", lambda W, X, Y: ql.qlinear_gemv(W, X[0], Y[0])))
            row = {}
            for name, fn in fns:
                step = (lambda i, fn=fn: fn(Ws[i % ncopy], X, Y))
                for i in range(2 * ncopy):
                    step(i)
                ms = graph_time(step, ncopy, 20)
                row[name] = {"us": round(ms * 1e3, 2), "TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 2),
                             "weight_GB/s": round(w4_bytes(K, N) / (ms * 1e-3) / 1e9, 1)}
            shape[f"M={M}"] = row
        out[f"K{K}_N{N}"] = shape
        del Ws, W0
        torch.cuda.empty_cache()
    return out


def bench_decode_fusions(args, dev):
    """The decode steps beside the GEMV, each timed from HIP graphs over
    rotated weight copies (more than 600 MB between two uses of a copy):
    the vocabulary head plain, with the on-GPU token choice, and with the
    token choice plus fp16 logits; the K = 2048, N = 8192 projection plain
    and with its RMSNorm prologue; the embedding row of the token; and one
    chained decode tail (normalized projection, head with token choice,
    embedding row of the chosen token)."""
    import torch
    import bit_group_quantized_amd as ql
    import synth
    K, V, N = 2048, synth.VOCAB, 8192
    head = synth.gemv_case(1, K, V)
    proj = synth.decode_norm_case(2, K, N)
    emb = synth.w4_matrix(synth.rng_for(3), K, V)
    hb, pb, eb = w4_bytes(K, V), w4_bytes(K, N), w4_bytes(K, V)
    copies = max(2, int(np.ceil(ROTATE_BYTES / hb)))
    Hs = [dev_w4(head["W"], dev)]
    Hs += [clone_w4(Hs[0]) for _ in range(copies - 1)]
    pc = max(2, int(np.ceil(ROTATE_BYTES / pb)))
    Ps = [dev_w4(proj["W"], dev)]
    Ps += [clone_w4(Ps[0]) for _ in range(pc - 1)]
    E = dev_w4(emb, dev)
    x = torch.from_numpy(head["x"][0]).to(dev)
    xp = torch.from_numpy(proj["x"][0]).to(dev)
    gamma = torch.from_numpy(proj["gamma"]).to(dev)
    logits = torch.empty(V, dtype=torch.float16, device=dev)
    yp = torch.empty(N, dtype=torch.float16, device=dev)
    tok = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = ql.gemv_argmax_workspace(V, dev)
    xe = torch.empty(K, dtype=torch.float16, device=dev)
    cases = {
        "head_gemv": (copies, hb + 2 * K + 2 * V, lambda i: ql.qlinear_gemv(Hs[i % copies], x, logits)),
        "head_argmax": (copies, hb + 2 * K + 4,
                        lambda i: ql.qlinear_gemv_argmax(Hs[i % copies], x, token=tok, workspace=ws)),
        "head_argmax_and_logits": (copies, hb + 2 * K + 2 * V + 4,
                                   lambda i: ql.qlinear_gemv_argmax(Hs[i % copies], x, token=tok,
                                                                    logits=logits, workspace=ws)),
        "proj_gemv": (pc, pb + 2 * K + 2 * N, lambda i: ql.qlinear_gemv(Ps[i % pc], xp, yp)),
        "proj_rmsnorm_gemv": (pc, pb + 4 * K + 2 * N,
                              lambda i: ql.qlinear_gemv_rmsnorm(Ps[i % pc], xp, gamma, 1e-6, yp)),
        "embed_row": (8, K // 2 + K // 16 + 2 * K + 4, lambda i: ql.qlinear_embed_token(E, tok, xe)),
    }
    # Interleaved rounds, median per case (a case timed right after another
    # can inherit its cache and clock state).
    times = {name: [] for name in cases}
    for _ in range(3):
        for name, (ng, nbytes, fn) in cases.items():
            for i in range(2 * ng):
                fn(i)
            times[name].append(graph_time(fn, ng, 20))
    out = {}
    for name, (ng, nbytes, fn) in cases.items():
        ms = float(np.median(times[name]))
        out[name] = {"us": round(ms * 1e3, 2), "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
                     "bytes": nbytes}

    def tail(i):
        ql.qlinear_gemv_rmsnorm(Ps[i % pc], xp, gamma, 1e-6, yp)
        ql.qlinear_gemv_argmax(Hs[i % copies], x, token=tok, workspace=ws)
        ql.qlinear_embed_token(E, tok, xe)
    ng = max(copies, pc)
    for i in range(ng):
        tail(i)
    ms = graph_time(tail, ng, 20)
    out["decode_tail_chain"] = {"us": round(ms * 1e3, 2),
                                "GB/s": round((hb + pb) / (ms * 1e-3) / 1e9, 1),
                                "what": "rmsnorm projection K2048 N8192, head with token choice and embedding row, back to back in one graph (no data dependency between the projection and the head here)"}
    return out


def dev_w4_bits(W, dev):
    """w4 dict whose scales and biases are 16-bit patterns (bf16)."""
    import torch
    return {"qweight": torch.from_numpy(np.ascontiguousarray(W["qweight"]).view(np.int32)).to(dev),
            "scales": torch.from_numpy(W["scales"].view(np.int16)).to(dev),
            "biases": torch.from_numpy(W["biases"].view(np.int16)).to(dev), "K": W["K"], "N": W["N"]}


def bench_bf16(args, dev):
    """The bf16 variant on the headline shapes: the two decode GEMVs (K = 2048,
    N = 8192 and 151552, rotated weight copies as in the headline) and the
    prefill GEMM at M = 4096 and 16384 (K = 2048, N = 8192)."""
    import torch
    import bit_group_quantized_amd as ql
    import synth
    K = 2048
    Ns = (8192, synth.VOCAB)
    cases = [synth.gemm_case_bf16(s, 1, K, N) for s, N in zip((0, 1), Ns)]
    step_bytes = sum(w4_bytes(K, N) + 2 * K + 2 * N for N in Ns)
    copies = max(2, int(np.ceil(ROTATE_BYTES / step_bytes)))
    base = [dev_w4_bits(c["W"], dev) for c in cases]
    Ws = [base] + [[clone_w4(w) for w in base] for _ in range(copies - 1)]
    x = torch.from_numpy(cases[0]["X"][0].view(np.int16)).to(dev)
    ys = [torch.empty(N, dtype=torch.bfloat16, device=dev) for N in Ns]

    def step(i):
        Wc = Ws[i % copies]
        ql.qlinear_gemv_bf16(Wc[0], x, ys[0])
        ql.qlinear_gemv_bf16(Wc[1], x, ys[1])

    ms = timed_steps(step, args.steps, args.warmup, settle_s=SETTLE_S)
    head_ms = timed_steps(lambda i: ql.qlinear_gemv_bf16(Ws[i % copies][1], x, ys[1]), args.steps, args.warmup,
                          settle_s=SETTLE_S / 2)
    out = {"gemv_step": {"us": float(ms * 1e3), "GB/s": step_bytes / (ms * 1e-3) / 1e9,
                         "frac_hbm": step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
           "gemv_head": {"us": float(head_ms * 1e3),
                         "GB/s": (w4_bytes(K, Ns[1]) + 2 * K + 2 * Ns[1]) / (head_ms * 1e-3) / 1e9}}
    del Ws, base
    torch.cuda.empty_cache()
    N = 8192
    for M in (4096, 16384):
        c = synth.gemm_case_bf16(0, M, K, N)
        W = dev_w4_bits(c["W"], dev)
        X = torch.from_numpy(c["X"].view(np.int16)).to(dev)
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        ms = timed_steps(lambda i: ql.qlinear_gemm_bf16(W, X, Y), 20 if M == 4096 else 8, 3, settle_s=SETTLE_S)
        tf = 2.0 * M * N * K / (ms * 1e-3) / 1e12
        out[f"gemm_M={M}"] = {"us": float(ms * 1e3), "TFLOP/s": tf, "frac_mfma_bf16": tf / MFMA_F16_PEAK_TFLOPS}
        del W, X, Y
        torch.cuda.empty_cache()
    return out


def bench_codecs(args, dev):
    """The second weight codecs on the headline decode shapes: FP8-E4M3 (1
    byte per weight + an fp16 scale per 64) and NVFP4 (half a byte + an E4M3
    scale per 16) GEMVs at K = 2048, N = 8192 and 151552, rotated weight
    copies as in the headline; bytes = codes + scales + x + y.  Then the FP8
    and NVFP4 GEMMs (fp16 MFMA on the staged weights) on the prefill shape."""
    import torch
    import bit_group_quantized_amd as ql
    import synth
    K = 2048
    Ns = (8192, synth.VOCAB)
    out = {}
    for codec in ("fp8", "nvfp4"):
        mats, nbytes = [], []
        for seed, N in zip((0, 1), Ns):
            rng = synth.rng_for(seed)
            if codec == "fp8":
                W = synth.fp8_matrix(rng, K, N)
                mats.append({"codes": torch.from_numpy(W["codes"]).to(dev),
                             "scales": torch.from_numpy(W["scales"]).to(dev), "K": K, "N": N})
                nbytes.append(N * K + 2 * N * (K // 64) + 2 * K + 2 * N)
            else:
                W = synth.nvfp4_matrix(rng, K, N)
                mats.append({"qweight": torch.from_numpy(W["qweight"].view(np.int32)).to(dev),
                             "block_scales": torch.from_numpy(W["block_scales"]).to(dev),
                             "global_scale": float(W["global_scale"]), "K": K, "N": N})
                nbytes.append(N * K // 2 + N * (K // 16) + 2 * K + 2 * N)
        step_bytes = sum(nbytes)
        copies = max(2, int(np.ceil(ROTATE_BYTES / step_bytes)))
        Ws = [mats] + [[{k: (v.clone() if hasattr(v, "clone") else v) for k, v in m.items()} for m in mats]
                       for _ in range(copies - 1)]
        fn = ql.qlinear_gemv_fp8 if codec == "fp8" else ql.qlinear_gemv_nvfp4
        x = torch.from_numpy(synth.activations(synth.rng_for(5), 1, K)[0]).to(dev)
        ys = [torch.empty(N, dtype=torch.float16, device=dev) for N in Ns]

        def step(i):
            fn(Ws[i % copies][0], x, ys[0])
            fn(Ws[i % copies][1], x, ys[1])

        ms = timed_steps(step, args.steps, args.warmup, settle_s=SETTLE_S)
        head_ms = timed_steps(lambda i: fn(Ws[i % copies][1], x, ys[1]), args.steps, args.warmup,
                              settle_s=SETTLE_S / 2)
        out[codec] = {"step_us": float(ms * 1e3), "step_GB/s": step_bytes / (ms * 1e-3) / 1e9,
                      "frac_hbm": step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                      "head_us": float(head_ms * 1e3), "head_GB/s": nbytes[1] / (head_ms * 1e-3) / 1e9,
                      "step_bytes": step_bytes}
        del Ws, mats
        torch.cuda.empty_cache()
    # FP8 weights on the prefill GEMM shape (K 2048, N 8192), M = 4096 and 16384.
    rng = synth.rng_for(3)
    W = synth.fp8_matrix(rng, K, 8192)
    Wd = {"codes": torch.from_numpy(W["codes"]).to(dev), "scales": torch.from_numpy(W["scales"]).to(dev),
          "K": K, "N": 8192}
    out["fp8_gemm"] = {}
    for M in (4096, 16384):
        X = torch.from_numpy(synth.activations(rng, M, K)).to(dev)
        Y = torch.empty((M, 8192), dtype=torch.float16, device=dev)
        ms = timed_steps(lambda i: ql.qlinear_gemm_fp8(Wd, X, Y), 20 if M == 4096 else 6, 3,
                         settle_s=SETTLE_S)
        tf = 2.0 * M * K * 8192 / (ms * 1e-3) / 1e12
        out["fp8_gemm"][f"M={M}"] = {"us": float(ms * 1e3), "TFLOP/s": tf,
                                      "frac_mfma_f16": tf / MFMA_F16_PEAK_TFLOPS}
    W = synth.nvfp4_matrix(rng, K, 8192)
    Wd = {"qweight": torch.from_numpy(W["qweight"].view(np.int32)).to(dev),
          "block_scales": torch.from_numpy(W["block_scales"]).to(dev),
          "global_scale": float(W["global_scale"]), "K": K, "N": 8192}
    out["nvfp4_gemm"] = {}
    for M in (4096, 16384):
        X = torch.from_numpy(synth.activations(rng, M, K)).to(dev)
        Y = torch.empty((M, 8192), dtype=torch.float16, device=dev)
        ms = timed_steps(lambda i: ql.qlinear_gemm_nvfp4(Wd, X, Y), 20 if M == 4096 else 6, 3,
                         settle_s=SETTLE_S)
        tf = 2.0 * M * K * 8192 / (ms * 1e-3) / 1e12
        out["nvfp4_gemm"][f"M={M}"] = {"us": float(ms * 1e3), "TFLOP/s": tf,
                                        "frac_mfma_f16": tf / MFMA_F16_PEAK_TFLOPS}
    return out


def moe_dev_weights(w, dev):
    import torch
    return {"Wr": torch.from_numpy(w["Wr"]).to(dev), "gate_up": dev_w4(w["gate_up"], dev),
            "down": dev_w4(w["down"], dev), "shared_gate_up": dev_w4(w["shared_gate_up"], dev),
            "shared_down": dev_w4(w["shared_down"], dev)}


def bench_moe_decode(args, dev, w):
    import torch
    import bit_group_quantized_amd as ql
    import synth
    base = moe_dev_weights(w, dev)
    copies = [base, {k: (clone_w4(v) if isinstance(v, dict) else v.clone()) for k, v in base.items()}]
    htoks = [synth.moe_tokens(2000 + i, 1)["H"] for i in range(32)]
    note_inputs("moe_decode_tokens_seeds2000-2031", list(range(2000, 2032)), *htoks)
    toks = [torch.from_numpy(h).to(dev) for h in htoks]
    route_buf = ql.alloc_route_outputs(1, 256, 8, dev)
    act = torch.empty((9, 512), dtype=torch.float16, device=dev)
    out = torch.empty((1, 2048), dtype=torch.float16, device=dev)

    def route(i):
        ql.moe_route(toks[i % len(toks)], copies[i % 2]["Wr"], None, 8, route_buf)

    def gate_up(i):
        dw = copies[i % 2]
        ql.moe_grouped_gemm(dw["gate_up"], dw["shared_gate_up"], toks[i % len(toks)], 1, 8,
                            ql.QL_OP_GATE_UP_SILU, route_buf, act)

    def down(i):
        dw = copies[i % 2]
        ql.moe_grouped_gemm(dw["down"], dw["shared_down"], act, 1, 8, ql.QL_OP_DOWN_COMBINE,
                            route_buf, out)

    def step3(i):
        route(i)
        gate_up(i)
        down(i)

    dec_buf = ql.alloc_decode_outputs(1, 256, 8, 2048, 512, dev)

    def layer(i):
        dw = copies[i % 2]
        ql.moe_decode(toks[i % len(toks)], dw["Wr"], None, 8, dw["gate_up"], dw["down"],
                      dw["shared_gate_up"], dw["shared_down"], out=dec_buf)

    # The per-call host path (Python, ctypes) is slower than these short
    # kernels, so the decode layer is timed as HIP graphs: NG steps captured
    # once (tokens and weight copies rotating), replayed back to back.
    NG = 16
    for i in range(3):
        step3(i)
        layer(i)
    torch.cuda.synchronize()
    ms = graph_time(layer, NG, 30)
    ms3 = graph_time(step3, NG, 30)

    # The same layer without the shared expert: what the shared expert costs
    # in this launch chain at all (an upper bound on what moving its rows
    # to an earlier launch could save).
    def layer_ns(i):
        dw = copies[i % 2]
        ql.moe_decode(toks[i % len(toks)], dw["Wr"], None, 8, dw["gate_up"], dw["down"], None, None,
                      out=dec_buf)

    for i in range(3):
        layer_ns(i)
    torch.cuda.synchronize()
    ms_ns = graph_time(layer_ns, NG, 30)
    # The bf16 layer (moe_decode_bf16), same rotation of tokens and weights.
    wb = synth.moe_weights_bf16(0)
    as_dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16 if a.dtype == np.uint16 else np.int32)).to(dev)
    wd = lambda W: {"qweight": as_dev(W["qweight"]), "scales": as_dev(W["scales"]),
                    "biases": as_dev(W["biases"]), "K": W["K"], "N": W["N"]}
    bcopies = []
    for c in range(2):
        d = {k: wd(wb[k]) for k in ("gate_up", "down", "shared_gate_up", "shared_down")}
        d["Wr"] = as_dev(wb["Wr"])
        bcopies.append(d)
    btoks = [as_dev(synth.moe_tokens_bf16(2000 + i, 1)["H"]) for i in range(32)]
    bbuf = ql.alloc_decode_outputs(1, 256, 8, 2048, 512, dev)
    bbuf["out"] = torch.empty((1, 2048), dtype=torch.bfloat16, device=dev)

    def layer_bf16(i):
        dw = bcopies[i % 2]
        ql.moe_decode(btoks[i % len(btoks)], dw["Wr"], None, 8, dw["gate_up"], dw["down"],
                      dw["shared_gate_up"], dw["shared_down"], out=bbuf, bf16=True)

    for i in range(3):
        layer_bf16(i)
    torch.cuda.synchronize()
    ms_bf = graph_time(layer_bf16, NG, 30)
    k = [graph_time(fn, NG, 30) for fn in (route, gate_up, down)]
    algo = 2048 * 256 * 2 + 9 * (w4_bytes(2048, 1024) + w4_bytes(512, 2048)) + 2 * 2048 * 2
    # FP8 and NVFP4 experts (moe_decode_fp8 / moe_decode_nvfp4), same tokens.
    codec = {}
    to_dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    for name in ("fp8", "nvfp4"):
        wc = synth.moe_weights_fp8(0) if name == "fp8" else synth.moe_weights_nvfp4(0)
        ccopies = []
        for c in range(2):
            d = {}
            for key in ("gate_up", "down", "shared_gate_up", "shared_down"):
                d[key] = {kk: (to_dev(v) if isinstance(v, np.ndarray) and v.ndim > 0 else v)
                          for kk, v in wc[key].items()}
                if "global_scale" in d[key] and not torch.is_tensor(d[key]["global_scale"]):
                    d[key]["global_scale"] = float(d[key]["global_scale"])
            d["Wr"] = to_dev(wc["Wr"])
            ccopies.append(d)
        cbuf = ql.alloc_decode_outputs(1, 256, 8, 2048, 512, dev)

        def layer_c(i, ccopies=ccopies, cbuf=cbuf, name=name):
            dw = ccopies[i % 2]
            ql.moe_decode_codec(name, toks[i % len(toks)], dw["Wr"], None, 8, dw["gate_up"], dw["down"],
                                dw["shared_gate_up"], dw["shared_down"], out=cbuf)

        for i in range(3):
            layer_c(i)
        torch.cuda.synchronize()
        msc = graph_time(layer_c, NG, 30)
        if name == "fp8":
            mat = lambda K, N: N * K + 2 * N * (K // 64)
        else:
            mat = lambda K, N: N * K // 2 + N * (K // 16)
        cb = 2048 * 256 * 2 + 9 * (mat(2048, 1024) + mat(512, 2048)) + 2 * 2048 * 2
        codec[name] = {"us_per_token": msc * 1e3, "algorithmic_bytes": cb,
                       "GB/s": cb / (msc * 1e-3) / 1e9, "entry": f"moe_decode_{name}"}
        del ccopies
    return {"tokens/s": 1e3 / ms, "us_per_token": ms * 1e3, "algorithmic_bytes": algo,
            "codec_experts": codec,
            "GB/s": algo / (ms * 1e-3) / 1e9, "frac_hbm": algo / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "entry": "moe_decode (router partials; routing fused into gate/up; down + combine)",
            "three_call_us_per_token": ms3 * 1e3,
            "no_shared_expert_us_per_token": ms_ns * 1e3,
            "bf16_us_per_token": ms_bf * 1e3,
            "three_call_stage_us": {"route": k[0] * 1e3, "gate_up_silu": k[1] * 1e3,
                                    "down_combine": k[2] * 1e3},
            "timing": "HIP graph of 16 decode steps, replayed" if USE_GRAPHS else "eager launches"}


def bench_moe_prefill(args, dev, w):
    """The 4096-token prefill layer (route, gate/up + SiLU, down, combine);
    two token sets (the first two screened seeds, each with its own Zipf
    logit bias) alternate from step to step, so the routing and the expert
    loads change between consecutive steps."""
    import torch
    import bit_group_quantized_amd as ql
    import synth
    T = 4096
    seeds = json.load(open(os.path.join(ROOT, "tests", "golden", "prefill_seeds.json")))["kept_seeds_by_gap"][:2]
    dw = moe_dev_weights(w, dev)
    toks = [synth.moe_tokens(sd, T, skewed=True) for sd in seeds]
    for sd, tk in zip(seeds, toks):
        note_inputs(f"moe_prefill_tokens_seed{sd}", sd, tk["H"], tk["logit_bias"])
    Hs = [torch.from_numpy(tk["H"]).to(dev) for tk in toks]
    biases = [torch.from_numpy(tk["logit_bias"]).to(dev) for tk in toks]
    routes = [ql.alloc_route_outputs(T, 256, 8, dev) for _ in toks]
    act = torch.empty((9 * T, 512), dtype=torch.float16, device=dev)
    yd = torch.empty((9 * T, 2048), dtype=torch.float16, device=dev)
    out = torch.empty((T, 2048), dtype=torch.float16, device=dev)

    def r_(i):
        ql.moe_route(Hs[i % 2], dw["Wr"], biases[i % 2], 8, routes[i % 2])

    def gu(i):
        ql.moe_grouped_gemm(dw["gate_up"], dw["shared_gate_up"], Hs[i % 2], T, 8, ql.QL_OP_GATE_UP_SILU,
                            routes[i % 2], act)

    def dn(i):
        ql.moe_grouped_gemm(dw["down"], dw["shared_down"], act, T, 8, ql.QL_OP_DOWN, routes[i % 2], yd)

    def cb(i):
        ql.moe_combine(yd, routes[i % 2]["gates"], routes[i % 2]["pos"], T, 8, True, out)

    SO = ql.QL_OP_SHARED_ONLY
    split = (lambda i: ql.moe_grouped_gemm(dw["gate_up"], None, Hs[i % 2], T, 8, ql.QL_OP_GATE_UP_SILU,
                                           routes[i % 2], act),
             lambda i: ql.moe_grouped_gemm(dw["down"], None, act, T, 8, ql.QL_OP_DOWN, routes[i % 2], yd),
             lambda i, st: ql.moe_grouped_gemm(dw["gate_up"], dw["shared_gate_up"], Hs[i % 2], T, 8,
                                               ql.QL_OP_GATE_UP_SILU | SO, None, act, stream=st),
             lambda i, st: ql.moe_grouped_gemm(dw["down"], dw["shared_down"], act, T, 8, ql.QL_OP_DOWN | SO,
                                               None, yd, stream=st))
    return prefill_timing(T, r_, gu, dn, cb, seeds, split)


def prefill_timing(T, r_, gu, dn, cb, seeds, split=None):
    """Time the four prefill stages as one step (20 steps) and each stage
    alone (10 launches); the stage functions take the step index, whose
    parity selects the token set.  With split = (gu_routed, dn_routed,
    gu_shared, dn_shared) the step that sets the reported rate runs the
    shared expert (which needs no routing) on a second stream beside the
    route and the routed projections, joined before the combine; the
    single-stream step is reported beside it."""
    import torch

    def step(i):
        r_(i)
        gu(i)
        dn(i)
        cb(i)

    ms_single = timed_steps(step, 20, 4, settle_s=SETTLE_S)
    ms = ms_single
    if split is not None:
        gu_r, dn_r, gu_s, dn_s = split
        side = torch.cuda.Stream()  # default priority
        forks = [torch.cuda.Event() for _ in range(2)]
        joins = [torch.cuda.Event() for _ in range(2)]

        def step2(i):
            main = torch.cuda.current_stream()
            forks[i % 2].record(main)
            side.wait_event(forks[i % 2])
            with torch.cuda.stream(side):
                gu_s(i, side)
                dn_s(i, side)
            joins[i % 2].record(side)
            r_(i)
            gu_r(i)
            dn_r(i)
            main.wait_event(joins[i % 2])
            cb(i)

        ms = timed_steps(step2, 20, 4, settle_s=SETTLE_S)
    k = np.asarray(stage_times([r_, gu, dn, cb], 10, 2, settle_s=SETTLE_S / 4))
    routed_rows = T * 8
    flops = (2.0 * routed_rows * 2048 * 1024 + 2.0 * routed_rows * 512 * 2048
             + 2.0 * T * 2048 * 1024 + 2.0 * T * 512 * 2048 + 2.0 * T * 2048 * 256)
    res = {"tokens/s": T / (ms * 1e-3), "ms_per_step": ms, "flops": flops,
           "TFLOP/s": flops / (ms * 1e-3) / 1e12,
           "frac_mfma_f16": flops / (ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS,
           "stage_us": {"route": float(k[0] * 1e3), "gate_up_silu": float(k[1] * 1e3),
                        "down": float(k[2] * 1e3), "combine": float(k[3] * 1e3)},
           "token_seeds": [int(sd) for sd in seeds]}
    if split is not None:
        res["streams"] = ("2: shared expert (QL_OP_SHARED_ONLY) on a second stream beside the route "
                          "and the routed rows")
        res["single_stream_ms_per_step"] = ms_single
        res["single_stream_TFLOP/s"] = flops / (ms_single * 1e-3) / 1e12
    return res


def bench_moe_prefill_bf16(args, dev):
    """The same 4096-token layer with bf16 tokens, router weight, scales,
    biases and outputs (moe_route_bf16 / moe_grouped_gemm_bf16 /
    moe_combine_bf16); two token sets alternate."""
    import torch
    import bit_group_quantized_amd as ql
    import synth
    T = 4096
    seeds = [4, 5]
    w = synth.moe_weights_bf16(0)
    toks = [synth.moe_tokens_bf16(sd, T, skewed=True) for sd in seeds]
    as_dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16 if a.dtype == np.uint16 else np.int32)).to(dev)
    wd = lambda W: {"qweight": as_dev(W["qweight"]), "scales": as_dev(W["scales"]),
                    "biases": as_dev(W["biases"]), "K": W["K"], "N": W["N"]}
    dw = {k: wd(w[k]) for k in ("gate_up", "down", "shared_gate_up", "shared_down")}
    Wr = as_dev(w["Wr"])
    Hs = [as_dev(tk["H"]) for tk in toks]
    biases = [torch.from_numpy(tk["logit_bias"]).to(dev) for tk in toks]
    routes = [ql.alloc_route_outputs(T, 256, 8, dev) for _ in toks]
    act = torch.empty((9 * T, 512), dtype=torch.bfloat16, device=dev)
    yd = torch.empty((9 * T, 2048), dtype=torch.bfloat16, device=dev)
    out = torch.empty((T, 2048), dtype=torch.bfloat16, device=dev)

    def r_(i):
        ql.moe_route_bf16(Hs[i % 2], Wr, biases[i % 2], 8, routes[i % 2])

    def gu(i):
        ql.moe_grouped_gemm_bf16(dw["gate_up"], dw["shared_gate_up"], Hs[i % 2], T, 8, ql.QL_OP_GATE_UP_SILU,
                                 routes[i % 2], act)

    def dn(i):
        ql.moe_grouped_gemm_bf16(dw["down"], dw["shared_down"], act, T, 8, ql.QL_OP_DOWN, routes[i % 2], yd)

    def cb(i):
        ql.moe_combine_bf16(yd, routes[i % 2]["gates"], routes[i % 2]["pos"], T, 8, True, out)

    SO = ql.QL_OP_SHARED_ONLY
    g = ql.moe_grouped_gemm_bf16
    split = (lambda i: g(dw["gate_up"], None, Hs[i % 2], T, 8, ql.QL_OP_GATE_UP_SILU, routes[i % 2], act),
             lambda i: g(dw["down"], None, act, T, 8, ql.QL_OP_DOWN, routes[i % 2], yd),
             lambda i, st: g(dw["gate_up"], dw["shared_gate_up"], Hs[i % 2], T, 8, ql.QL_OP_GATE_UP_SILU | SO,
                             None, act, stream=st),
             lambda i, st: g(dw["down"], dw["shared_down"], act, T, 8, ql.QL_OP_DOWN | SO, None, yd, stream=st))
    r = prefill_timing(T, r_, gu, dn, cb, seeds, split)
    r["frac_mfma_bf16"] = r.pop("frac_mfma_f16")
    return r


def bench_moe_prefill_codec(args, dev, codec: str):
    """The same 4096-token layer with FP8-E4M3 or NVFP4 experts (moe_route /
    moe_grouped_gemm_fp8 or _nvfp4 / moe_combine; fp16 tokens and outputs);
    two token sets alternate."""
    import torch
    import bit_group_quantized_amd as ql
    import synth
    T = 4096
    seeds = json.load(open(os.path.join(ROOT, "tests", "golden", "prefill_seeds.json")))["kept_seeds_by_gap"][:2]
    w = synth.moe_weights_fp8(0) if codec == "fp8" else synth.moe_weights_nvfp4(0)
    toks = [synth.moe_tokens(sd, T, skewed=True) for sd in seeds]
    to_dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    def wd(W):
        d = {k: (to_dev(v) if isinstance(v, np.ndarray) and v.ndim > 0 else v) for k, v in W.items()}
        if "global_scale" in d and not torch.is_tensor(d["global_scale"]):
            d["global_scale"] = float(d["global_scale"])
        return d

    dw = {k: wd(w[k]) for k in ("gate_up", "down", "shared_gate_up", "shared_down")}
    gemm = ql.moe_grouped_gemm_fp8 if codec == "fp8" else ql.moe_grouped_gemm_nvfp4
    Wr = to_dev(w["Wr"])
    Hs = [to_dev(tk["H"]) for tk in toks]
    biases = [torch.from_numpy(tk["logit_bias"]).to(dev) for tk in toks]
    routes = [ql.alloc_route_outputs(T, 256, 8, dev) for _ in toks]
    act = torch.empty((9 * T, 512), dtype=torch.float16, device=dev)
    yd = torch.empty((9 * T, 2048), dtype=torch.float16, device=dev)
    out = torch.empty((T, 2048), dtype=torch.float16, device=dev)

    def r_(i):
        ql.moe_route(Hs[i % 2], Wr, biases[i % 2], 8, routes[i % 2])

    def gu(i):
        gemm(dw["gate_up"], dw["shared_gate_up"], Hs[i % 2], T, 8, ql.QL_OP_GATE_UP_SILU, routes[i % 2], act)

    def dn(i):
        gemm(dw["down"], dw["shared_down"], act, T, 8, ql.QL_OP_DOWN, routes[i % 2], yd)

    def cb(i):
        ql.moe_combine(yd, routes[i % 2]["gates"], routes[i % 2]["pos"], T, 8, True, out)

    SO = ql.QL_OP_SHARED_ONLY
    split = (lambda i: gemm(dw["gate_up"], None, Hs[i % 2], T, 8, ql.QL_OP_GATE_UP_SILU, routes[i % 2], act),
             lambda i: gemm(dw["down"], None, act, T, 8, ql.QL_OP_DOWN, routes[i % 2], yd),
             lambda i, st: gemm(dw["gate_up"], dw["shared_gate_up"], Hs[i % 2], T, 8,
                                ql.QL_OP_GATE_UP_SILU | SO, None, act, stream=st),
             lambda i, st: gemm(dw["down"], dw["shared_down"], act, T, 8, ql.QL_OP_DOWN | SO, None, yd,
                                stream=st))
    return prefill_timing(T, r_, gu, dn, cb, seeds, split)


CALIB_BYTES = 256 * 1024 * 1024


def pmc_calibration(dev):
    """A plain elementwise copy (negation) of CALIB_BYTES of fp16: it reads
    and writes exactly CALIB_BYTES, which calibrates FETCH_SIZE and WRITE_SIZE."""
    import torch
    src = torch.randn(CALIB_BYTES // 2, dtype=torch.float16, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()


def ingest_pmc(fetch_csv, write_csv):
    import csv
    def per_kernel(path, counter):
        # Per kernel name: (grid size, bytes) of every dispatch, in dispatch order.
        out = {}
        with open(path) as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") != counter:
                    continue
                name = row.get("Kernel_Name", "")
                out.setdefault(name, []).append((int(row["Grid_Size"]),
                                                 float(row["Counter_Value"]) * 1024.0))  # KiB
        return out
    fetch = per_kernel(fetch_csv, "FETCH_SIZE")
    write = per_kernel(write_csv, "WRITE_SIZE")

    def pick(d, pattern):
        keys = [k for k in d if pattern in k]
        if not keys:
            raise SystemExit(f"no kernel matching {pattern!r} in the counter file")
        return keys[0]
    def values(rows, largest_grid=False):
        # The N = 8192 matrix runs the same kernel instantiation with a smaller
        # grid; the vocabulary head is the dispatch with the largest grid.
        g = max(r[0] for r in rows)
        return np.asarray([v for gs, v in rows if gs == g or not largest_grid])
    f_read = CALIB_BYTES / np.median(values(fetch[pick(fetch, "neg_kernel")]))
    f_write = CALIB_BYTES / np.median(values(write[pick(write, "neg_kernel")]))
    fr = values(fetch[pick(fetch, "gemv_w4_chunked_kernel<64, 1, 8, 0, 0>")], largest_grid=True) * f_read
    wr = values(write[pick(write, "gemv_w4_chunked_kernel<64, 1, 8, 0, 0>")], largest_grid=True) * f_write
    n = min(len(fr), len(wr))
    per_launch = float(np.mean(fr[:n] + wr[:n]))
    algo = w4_bytes(2048, 151552) + 2 * 2048 + 2 * 151552
    path = os.path.join(ROOT, "profiles", "traffic.json")
    d = json.load(open(path)) if os.path.exists(path) else {}
    d[KERNEL_GEMV] = {
        "source_sha": source_sha("gemv.hip", "ql_device.h"),
        "bytes_per_launch": per_launch,
        "algorithmic_bytes_per_launch": algo,
        "ratio_to_algorithmic": per_launch / algo,
        "fetch_scale": f_read, "write_scale": f_write,
        "calibration": f"torch.neg on {CALIB_BYTES} bytes of fp16: expected reads = writes = {CALIB_BYTES}",
        "dispatches": n,
    }
    with open(path, "w") as f:
        json.dump(d, f, indent=1)
    print(json.dumps(d[KERNEL_GEMV], indent=1))


PROBE_BYTES = 2 << 30  # 2 GiB: far beyond the 256 MB Infinity Cache


def read_probe(dev):
    """Measured HBM read rate (libqlprobe, built with the library): 2 GiB
    read once per launch, 10 launches between two events, median and best
    of 5 rounds.  Pattern "rows" is the vocabulary-head GEMV's code-load
    pattern (1 KB rows, 8 per wave, 16-byte non-temporal loads, all issued
    before use); "stream" a grid-stride streaming read."""
    import ctypes
    import torch
    path = os.path.join(ROOT, "bit_group_quantized_amd", "libqlprobe.so")
    L = ctypes.CDLL(path)
    L.ql_read_probe.restype = ctypes.c_int
    L.ql_read_probe.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    L.ql_probe_out_words.restype = ctypes.c_size_t
    L.ql_probe_out_words.argtypes = [ctypes.c_int, ctypes.c_size_t]
    buf = torch.randint(0, 255, (PROBE_BYTES,), dtype=torch.uint8, device=dev)
    out = {}
    for pattern, name in ((0, "rows"), (1, "stream")):
        words = torch.empty(int(L.ql_probe_out_words(pattern, PROBE_BYTES)), dtype=torch.int32, device=dev)
        st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

        def launch():
            rc = L.ql_read_probe(pattern, buf.data_ptr(), PROBE_BYTES, words.data_ptr(), st)
            if rc != 0:
                raise RuntimeError(f"ql_read_probe failed with status {rc}")

        for _ in range(3):
            launch()
        torch.cuda.synchronize()
        rates = []
        for _ in range(5):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(10):
                launch()
            b.record()
            torch.cuda.synchronize()
            rates.append(10 * PROBE_BYTES / (a.elapsed_time(b) * 1e-3) / 1e9)
        out[name] = {"GB/s_median": float(np.median(rates)), "GB/s_best": float(np.max(rates)),
                     "frac_of_spec_median": float(np.median(rates)) / HBM_PEAK_GBS}
    del buf
    torch.cuda.empty_cache()
    out["bytes_per_launch"] = PROBE_BYTES
    out["short_reads"] = short_reads(dev, L)
    out["spec_peak_GB/s"] = HBM_PEAK_GBS
    return out


def short_reads(dev, L):
    """Reads of a few MB with the "rows" pattern, one launch per HIP-graph
    node (64 nodes, replayed), each launch on a buffer of its own (together
    more than the 256 MB Infinity Cache), beside the K 2048 x N 8192
    projection GEMV timed the same way over rotated weight copies: the read
    floor of a launch of that size.  The fit over the sizes gives the fixed
    cost of a launch and the marginal read rate."""
    import ctypes
    import torch
    import bit_group_quantized_amd as ql
    import synth
    proj = w4_bytes(2048, 8192)  # 9,457,664 B, a multiple of 1024
    sizes = [proj, 2 * proj, 4 * proj]
    res = {"projection_bytes": proj, "reads": []}
    for nbytes in sizes:
        nbuf = max(4, (700 << 20) // nbytes)
        bufs = [torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1) for _ in range(nbuf)]
        words = torch.empty(int(L.ql_probe_out_words(0, nbytes)), dtype=torch.int32, device=dev)

        def rd(i, bufs=bufs, words=words, nbytes=nbytes):
            # the current stream: the capture stream while a graph is recorded
            st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
            rc = L.ql_read_probe(0, bufs[i % len(bufs)].data_ptr(), nbytes, words.data_ptr(), st)
            if rc != 0:
                raise RuntimeError(f"ql_read_probe failed with status {rc}")

        for i in range(3):
            rd(i)
        torch.cuda.synchronize()
        ms = graph_time(rd, 64, 20)
        res["reads"].append({"bytes": nbytes, "us_per_launch": ms * 1e3, "GB/s": nbytes / (ms * 1e-3) / 1e9})
        del bufs
    torch.cuda.empty_cache()
    xs = np.array([r["bytes"] for r in res["reads"]], dtype=np.float64)
    ys = np.array([r["us_per_launch"] for r in res["reads"]], dtype=np.float64)
    slope, icpt = np.polyfit(xs, ys, 1)
    res["fit_fixed_us"] = float(icpt)
    res["fit_marginal_GB/s"] = float(1e-3 / slope)
    case = synth.gemv_case(0, 2048, 8192)
    base = {"qweight": torch.from_numpy(case["W"]["qweight"].view(np.int32)).to(dev),
            "scales": torch.from_numpy(case["W"]["scales"]).to(dev),
            "biases": torch.from_numpy(case["W"]["biases"]).to(dev), "K": 2048, "N": 8192}
    ncopy = max(4, (700 << 20) // proj)
    copies = [base] + [clone_w4(base) for _ in range(ncopy - 1)]
    x = torch.from_numpy(case["x"][0]).to(dev)
    y = torch.empty(8192, dtype=torch.float16, device=dev)

    def gv(i):
        ql.qlinear_gemv(copies[i % ncopy], x, y)

    for i in range(3):
        gv(i)
    torch.cuda.synchronize()
    ms = graph_time(gv, 64, 20)
    res["projection_gemv_us"] = ms * 1e3
    res["projection_gemv_over_read"] = ms * 1e3 / res["reads"][0]["us_per_launch"]
    del copies
    torch.cuda.empty_cache()
    return res


def probe_lib():
    import ctypes
    L = ctypes.CDLL(os.path.join(ROOT, "bit_group_quantized_amd", "libqlprobe.so"))
    L.ql_probe_empty.restype = ctypes.c_int
    L.ql_probe_empty.argtypes = [ctypes.c_void_p]
    L.ql_probe_chase.restype = ctypes.c_int
    L.ql_probe_chase.argtypes = [ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_int,
                                 ctypes.c_void_p, ctypes.c_void_p]
    L.ql_probe_lds_blocks.restype = ctypes.c_int
    L.ql_probe_lds_blocks.argtypes = []
    L.ql_probe_lds_bytes.restype = ctypes.c_double
    L.ql_probe_lds_bytes.argtypes = [ctypes.c_int, ctypes.c_int]
    L.ql_probe_lds.restype = ctypes.c_int
    L.ql_probe_lds.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    return L


LDS_PROBE_MODES = ((0, "read_b128_contiguous"), (1, "read_b128_mfma_fragment_rows"),
                   (2, "write_b128_staging_rows"), (3, "write_b64_contiguous"))


def lds_probe(dev):
    """LDS throughput of one CU (libqlprobe): 8 waves of one workgroup per CU
    issue back-to-back 16- or 8-byte LDS accesses; bytes per shader clock
    (s_memtime in the kernel), median over the 256 workgroups of the second
    of two launches, for reads in the contiguous and the matrix-fragment
    pattern and for writes in the staging pattern."""
    import ctypes
    import torch
    L = probe_lib()
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    blocks = int(L.ql_probe_lds_blocks())
    cyc = torch.empty(blocks, dtype=torch.int64, device=dev)
    out = torch.empty(blocks * 512, dtype=torch.int32, device=dev)
    iters = 4096
    res = {}
    for mode, name in LDS_PROBE_MODES:
        for _ in range(2):
            if L.ql_probe_lds(mode, iters, ctypes.c_void_p(cyc.data_ptr()), ctypes.c_void_p(out.data_ptr()), st) != 0:
                raise RuntimeError("ql_probe_lds failed")
        torch.cuda.synchronize()
        c = cyc.cpu().numpy().astype(np.float64)
        res[name] = {"bytes_per_clock_per_CU": float(L.ql_probe_lds_bytes(mode, iters) / np.median(c))}
    return res


def latency_budget(dev):
    """The fixed costs a short dependent chain of launches pays (libqlprobe):
    the gap one node of a replayed HIP graph adds (a graph of 64 empty
    kernels on one stream), the cost of an eager launch of an empty kernel,
    and the round trip of one load that depends on the previous one, as one
    thread follows a random cycle with a 128-byte stride: "warm" repeats one
    segment of 2,000 loads of a 2 MB buffer (every line already in L2),
    "cold" walks fresh segments of a 2 GB buffer (every line missing every
    cache); median of 5 launches of 2,000 loads."""
    import ctypes
    import torch
    L = probe_lib()
    st = lambda: ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    out = {}

    def empty(i):
        if L.ql_probe_empty(st()) != 0:
            raise RuntimeError("ql_probe_empty failed")
    for i in range(10):
        empty(i)
    torch.cuda.synchronize()
    out["graph_node_us"] = graph_time(empty, 64, 20) * 1e3
    out["eager_launch_us"] = timed_steps(empty, 200, 10) * 1e3
    res = torch.empty(1, dtype=torch.int32, device=dev)
    rng = np.random.default_rng(0)
    steps = 2000
    for name, nbytes, warm in (("warm_L2_2MB", 2 << 20, True), ("cold_2GB", 2 << 30, False)):
        n = nbytes // 4
        slots = n // 32                        # one element per 128 bytes
        perm = rng.permutation(slots).astype(np.int64) * 32
        nxt = np.zeros(n, dtype=np.uint32)
        nxt[perm] = np.roll(perm, -1).astype(np.uint32)  # one cycle through every slot
        buf = torch.from_numpy(nxt.view(np.int32)).to(dev)
        times = []
        for rep in range(6):
            start = int(perm[0 if warm else (rep + 1) * 3 * steps])
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            if L.ql_probe_chase(buf.data_ptr(), n, start, steps, res.data_ptr(), st()) != 0:
                raise RuntimeError("ql_probe_chase failed")
            b.record()
            torch.cuda.synchronize()
            if rep > 0:
                times.append(a.elapsed_time(b) * 1e6 / steps)
        out[f"dependent_load_ns_{name}"] = float(np.median(times))
        del buf
    torch.cuda.empty_cache()
    return out


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        return int(os.environ.get("OMP_NUM_THREADS", "1"))


def _repeat(fn, budget_s):
    """Run fn until budget_s seconds have passed (at least once); returns
    (repetitions, seconds)."""
    reps = 0
    t0 = time.perf_counter()
    while True:
        fn()
        reps += 1
        if time.perf_counter() - t0 > budget_s:
            break
    return reps, time.perf_counter() - t0


def cpu_baseline():
    """The oracle as it stands, timed on the host cores on a bounded sample
    of every workload (about 25 s in all; inputs drawn before the clocks
    start).  The headline entry (config 1, in the headline's unit) keeps the
    contract keys; "per_config" has all five workloads in their own units."""
    import oracle
    import synth
    threads = _blas_threads()
    per = {}
    K = 2048
    # config 0: the whole 512 x 512 GEMV
    c0 = synth.gemv_case(0, 512, 512)
    reps, dt = _repeat(lambda: oracle.linear(c0["x"], c0["W"]), 2.0)
    b0 = w4_bytes(512, 512) + 2 * 512 * 2
    per["gemv_K512_N512"] = {"GB/s": reps * b0 / dt / 1e9, "s_per_call": dt / reps,
                                     "sample": f"whole workload, {reps} calls in {dt:.1f} s"}
    # config 1: the 8192-row projection and the first 16384 rows of the head
    small = synth.gemv_case(0, K, 8192)
    head = synth.gemv_case(1, K, 16384)
    b1 = sum(w4_bytes(K, N) + 2 * K + 2 * N for N in (8192, 16384))
    reps, dt = _repeat(lambda: (oracle.linear(small["x"], small["W"]), oracle.linear(head["x"], head["W"])), 8.0)
    g1 = reps * b1 / dt / 1e9
    per["gemv_K2048_N8192_and_N151552"] = {
        "GB/s": g1, "s_per_step_extrapolated": (w4_bytes(K, 8192) + w4_bytes(K, 151552)) / (g1 * 1e9),
        "sample": f"the 2048x8192 matrix and 16384 of the head's 151552 rows, {reps} repetitions in {dt:.1f} s"}
    # config 2: 64 of the 4096 rows of X through the whole 2048 x 8192 matrix
    c2 = synth.gemm_case(0, 64, K, 8192)
    reps, dt = _repeat(lambda: oracle.linear(c2["X"], c2["W"]), 4.0)
    f2 = 2.0 * 64 * K * 8192
    per["gemm_K2048_N8192"] = {"GFLOP/s": reps * f2 / dt / 1e9, "rows_per_s": reps * 64 / dt,
                                      "sample": f"64 rows of X, {reps} calls in {dt:.1f} s"}
    # config 3: one decode token through the whole layer
    w = synth.moe_weights(0)
    tok = synth.moe_tokens(2000, 1)
    reps, dt = _repeat(lambda: oracle.moe_layer(tok["H"], w, None, 8), 4.0)
    b3 = 2048 * 256 * 2 + 9 * (w4_bytes(2048, 1024) + w4_bytes(512, 2048)) + 2 * 2048 * 2
    per["moe_decode_1tok"] = {"tokens/s": reps / dt, "GB/s": reps * b3 / dt / 1e9,
                                      "sample": f"one token, {reps} calls in {dt:.1f} s"}
    # config 4: 64 of the 4096 Zipf-biased prefill tokens through the layer
    seed = json.load(open(os.path.join(ROOT, "tests", "golden", "prefill_seeds.json")))["kept_seeds_by_gap"][0]
    t4 = synth.moe_tokens(seed, 4096, skewed=True)
    H4 = t4["H"][:64]
    reps, dt = _repeat(lambda: oracle.moe_layer(H4, w, t4["logit_bias"], 8), 4.0)
    f4 = 64 * (2.0 * 8 * 2048 * 1024 + 2.0 * 8 * 512 * 2048 + 2.0 * 2048 * 1024 + 2.0 * 512 * 2048
               + 2.0 * 2048 * 256)
    per["moe_prefill_4096tok"] = {"tokens/s": reps * 64 / dt, "GFLOP/s": reps * f4 / dt / 1e9,
                                  "sample": f"64 of the 4096 tokens (seed {seed}), {reps} calls in {dt:.1f} s"}
    return {"value": g1, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": per["gemv_K2048_N8192_and_N151552"]["sample"] +
                      f" (oracle.linear, numpy fp64); BLAS threads {threads}, host cpu_count {os.cpu_count()}, "
                      f"affinity {len(os.sched_getaffinity(0))}",
            "per_config": per}


def run_metadata():
    """Device, software, clocks, input seeds and hashes, source fingerprint."""
    import subprocess
    import torch
    p = torch.cuda.get_device_properties(0)
    meta = {"device": p.name, "arch": getattr(p, "gcnArchName", None),
            "compute_units": p.multi_processor_count, "hbm_bytes": p.total_memory,
            "torch": torch.__version__, "hip_runtime": torch.version.hip}
    try:
        meta["rocm"] = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        meta["rocm"] = None
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True, timeout=20)
        clocks = json.loads(r.stdout) if r.returncode == 0 else None
        meta["clocks"] = next(iter(clocks.values())) if isinstance(clocks, dict) and clocks else None
    except Exception:
        meta["clocks"] = None
    h = hashlib.sha256()
    for d in (os.path.join(ROOT, "bit_group_quantized_amd", "csrc"), os.path.join(ROOT, "include")):
        for n in sorted(os.listdir(d)):
            with open(os.path.join(d, n), "rb") as f:
                h.update(n.encode() + f.read())
    meta["source_sha256_16"] = h.hexdigest()[:16]
    lib = os.path.join(ROOT, "bit_group_quantized_amd", "libqlinear.so")
    with open(lib, "rb") as f:
        meta["library_sha256_16"] = hashlib.sha256(f.read()).hexdigest()[:16]
    meta["inputs"] = dict(INPUTS)
    return meta


def main():
    args = parse()
    global USE_GRAPHS
    USE_GRAPHS = not args.eager
    if args.ingest_pmc:
        ingest_pmc(*args.ingest_pmc)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(this library has no multi-GPU path: it runs on one GPU's share of the work)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import bit_group_quantized_amd as ql
    ql.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    log("bench: GEMV (headline)")
    g = bench_gemv(args, dev)
    res = {
        "metric": METRIC, "value": g["value"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": g["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": "batch-1 decode w4 GEMV: x fp16[1,2048] times K=2048 x N=8192 and "
                               "K=2048 x N=151552 (g=64, fp16 scale/bias), one step = both",
                   "K": 2048, "N": [8192, 151552], "rotation_copies": g["rotation_copies"],
                   "step_bytes": g["step_bytes"]},
        "roofline": g["roofline"],
        "per_matrix": g["per_matrix"],
        "projection_in_graph": g["projection_in_graph"],
        "step_one_launch": g["step_one_launch"],
        "graph_step": g["graph"],
        "stats": g["stats"],
    }
    if args.pmc_calibration:
        pmc_calibration(dev)
    if not args.only_primary:
        import synth
        log("bench: read-bandwidth probe")
        res["read_probe"] = read_probe(dev)
        res["roofline"]["measured_read_ceiling_GB/s"] = res["read_probe"]["rows"]["GB/s_median"]
        res["roofline"]["frac_of_measured_ceiling"] = (res["roofline"]["achieved"] /
                                                       res["read_probe"]["rows"]["GB/s_median"])
        wl = res.setdefault("workloads", {})
        log("bench: small GEMV")
        wl["gemv_K512_N512"] = bench_gemv_small(args, dev)
        if args.workload in ("all", "gemm", "gemm_prefill", "latency"):
            log("bench: LDS probe")
            wl["lds_probe"] = lds_probe(dev)
        if args.workload in ("all", "gemm", "gemm_prefill"):
            log("bench: GEMM")
            wl["prefill_gemm_K2048_N8192"] = bench_gemm(args, dev)
        if args.workload in ("all", "gemm"):
            log("bench: few-row GEMM")
            wl["few_rows_gemm"] = bench_few_rows(args, dev)
        if args.workload in ("all", "bf16"):
            log("bench: bf16 variant")
            wl["bf16"] = bench_bf16(args, dev)
        if args.workload in ("all", "codecs"):
            log("bench: second codecs")
            wl["codecs"] = bench_codecs(args, dev)
        if args.workload in ("all", "decode"):
            log("bench: decode fusions")
            wl["decode_fusions"] = bench_decode_fusions(args, dev)
        if args.workload in ("all", "latency", "moe_decode"):
            log("bench: latency budget")
            wl["latency_budget"] = latency_budget(dev)
        if args.workload in ("all", "moe_decode", "moe_prefill"):
            w = synth.moe_weights(0)
            note_inputs("moe_weights_seed0", 0, w["Wr"], *w4_arrays(w["gate_up"]), *w4_arrays(w["down"]),
                        *w4_arrays(w["shared_gate_up"]), *w4_arrays(w["shared_down"]))
            if args.workload in ("all", "moe_decode"):
                log("bench: MoE decode")
                wl["moe_decode_1tok"] = bench_moe_decode(args, dev, w)
            if args.workload in ("all", "moe_prefill"):
                log("bench: MoE prefill")
                wl["moe_prefill_4096tok"] = bench_moe_prefill(args, dev, w)
                log("bench: MoE prefill, bf16")
                wl["moe_prefill_4096tok_bf16"] = bench_moe_prefill_bf16(args, dev)
                log("bench: MoE prefill, FP8 experts")
                wl["moe_prefill_4096tok_fp8"] = bench_moe_prefill_codec(args, dev, "fp8")
                log("bench: MoE prefill, NVFP4 experts")
                wl["moe_prefill_4096tok_nvfp4"] = bench_moe_prefill_codec(args, dev, "nvfp4")
    if not args.no_cpu_baseline:
        log("bench: CPU baseline (oracle)")
        res["cpu_baseline"] = cpu_baseline()
    res["meta"] = run_metadata()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
