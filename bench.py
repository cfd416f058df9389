"""Benchmark of the MoE dispatch/combine hot path on one MI355X.

One step = the whole path on one batch: routing plan and FP8 dispatch
(OCP E4M3, one fp32 scale per 128 columns) through the fused
mep_plan_dispatch, bf16 combine, then reset, for
4096 tokens x 7168 hidden, top-8 of 256 experts on 8 virtual ranks -- the
shape of the MORI README bandwidth table ("4096 tokens, 7168 hidden, top-8,
FP8 dispatch + BF16 combine").  Inputs are synthetic and already resident in
HBM; the expert outputs combine reads are produced once, before timing, by
the dequantise-times-0.5 stand-in.  Several buffer sets rotate so that no step
finds its data in the 256 MB Infinity Cache.

value = algorithmic HBM bytes of the step / step time (GB/s).  The JSON line
also carries the decode latency (128 tokens, bf16 both ways), the roofline of
the dominant kernel (achieved bytes per launch / its HIP-event duration on
the library's stream) and the CPU oracle's rate on a bounded sample.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
METRIC = "dispatch & combine effective HBM GB/s (% of peak) at 4096×7168 top-8; µs at 128 tok"


# --------------------------------------------------------------------------
# algorithmic bytes: what the method must read and write, per launch
# --------------------------------------------------------------------------

def plan_bytes(T, k, R, U):
    return T * k * 4 + U * 4 + R * 4            # ids in; src_token_pos, counts out


def dispatch_bytes(T, H, k, U, fp8):
    nb = H // 128 if fp8 else 0
    b = 1 if fp8 else 2
    return T * H * 2 + T * k * 8 + U * (H * b + nb * 4 + k * 8)


def combine_bytes(T, H, k, U):
    return U * H * 2 + T * k * 8 + T * H * 2


def src_digest(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "combine_mep_plan_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def profile_traffic(kernel_file, digest):
    """HBM bytes per launch measured by rocprofv3 counters for the current kernel
    source, or None if no summary matches this source."""
    p = os.path.join(ROOT, "profiles", kernel_file)
    if not os.path.exists(p):
        return None
    vals = {}
    with open(p) as f:
        for line in f:
            if ":" in line:
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("source_digest") != digest:
        return None
    try:
        return int(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# --------------------------------------------------------------------------

def setup_prefill(M, torch, wl, inp, nsets):
    """Device buffers for `nsets` independent copies of the workload."""
    T, H, R, cap, k = wl.tokens, wl.hidden, wl.ranks, wl.cap, wl.topk
    m = M.Mep(H, wl.experts_per_rank, k, cap, R, fp8=True)
    sets = []
    for _ in range(nsets):
        s = {
            "x": torch.from_numpy(inp["x"].view(np.int16)).cuda(),
            "w": torch.from_numpy(inp["weights"]).cuda(),
            "idx": torch.from_numpy(inp["indices"]).cuda(),
            "counts": torch.zeros(R, dtype=torch.int32, device="cuda"),
            "spos": torch.zeros((R, cap), dtype=torch.int32, device="cuda"),
            "rx": torch.zeros((R, cap, H), dtype=torch.uint8, device="cuda"),
            "rs": torch.zeros((R, cap, H // 128), dtype=torch.float32, device="cuda"),
            "rw": torch.zeros((R, cap, k), dtype=torch.float32, device="cuda"),
            "ri": torch.zeros((R, cap, k), dtype=torch.int32, device="cuda"),
            "out": torch.empty((T, H), dtype=torch.int16, device="cuda"),
        }
        # expert outputs (harness, untimed): bf16(decode(q) * scale * 0.5) of this
        # set's own dispatch
        M.mep_plan(m.h, s["idx"], T, s["counts"], s["spos"])
        M.mep_dispatch(m.h, s["x"], s["w"], s["idx"], s["rx"], s["rs"], s["rw"], s["ri"])
        q = s["rx"].view(torch.float8_e4m3fn).float()
        y = (q * s["rs"].repeat_interleave(128, dim=-1)) * 0.5
        s["y"] = y.to(torch.bfloat16).view(torch.int16)
        del q, y
        M.mep_reset(m.h)
        sets.append(s)
    torch.cuda.synchronize()
    U = int(sets[0]["counts"].sum().item())
    return m, sets, U


def _loop_ms(torch, stream, fn, n):
    """Average ms per call of fn(i) over n back-to-back calls on `stream`,
    timed by two HIP events (none inside the loop)."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for i in range(n):
        fn(i)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n


def time_prefill(M, torch, m, sets, wl, steps, warmup):
    """Headline loop: whole steps back to back.  Then one loop per kernel
    (same rotation of buffer sets) for its average launch duration.  Every set
    has the same routing, so the plan in the handle serves any set."""
    T = wl.tokens
    stream = torch.cuda.current_stream()
    n = len(sets)

    def plan(i):
        s = sets[i % n]
        M.mep_plan(m.h, s["idx"], T, s["counts"], s["spos"], stream)

    def dispatch(i):
        s = sets[i % n]
        M.mep_dispatch(m.h, s["x"], s["w"], s["idx"], s["rx"], s["rs"], s["rw"], s["ri"], stream)

    def combine(i):
        s = sets[i % n]
        M.mep_combine(m.h, M.MEP_RANK_MAJOR, s["y"], s["w"], s["out"], stream)

    def plan_dispatch(i):
        s = sets[i % n]
        M.mep_plan_dispatch(m.h, s["idx"], T, s["counts"], s["spos"], s["x"], s["w"], s["rx"],
                            s["rs"], s["rw"], s["ri"], stream)

    def step(i):
        plan_dispatch(i)
        combine(i)
        M.mep_reset(m.h, stream)

    for i in range(warmup):
        step(i)
    step_ms = _loop_ms(torch, stream, step, steps)
    assert M.mep_get_status(m.h, stream) == 0
    times = {
        "plan_dispatch": _loop_ms(torch, stream, plan_dispatch, steps),
        "combine": _loop_ms(torch, stream, combine, steps),
        "plan": _loop_ms(torch, stream, plan, steps),
        "dispatch": _loop_ms(torch, stream, dispatch, steps),
    }
    M.mep_reset(m.h, stream)
    return step_ms, times


def time_decode(M, torch, wl, inp, reps, warmup):
    """128-token latency, bf16 both ways, identity expert (combine reads the
    receive buffers): plan+dispatch as one call sequence, and combine, each
    between its own pair of events with the GPU idle before it."""
    T, H, R, cap, k = wl.tokens, wl.hidden, wl.ranks, wl.cap, wl.topk
    m = M.Mep(H, wl.experts_per_rank, k, cap, R, fp8=False)
    nsets = 4
    sets = []
    for _ in range(nsets):
        sets.append({
            "x": torch.from_numpy(inp["x"].view(np.int16)).cuda(),
            "w": torch.from_numpy(inp["weights"]).cuda(),
            "idx": torch.from_numpy(inp["indices"]).cuda(),
            "counts": torch.zeros(R, dtype=torch.int32, device="cuda"),
            "spos": torch.zeros((R, cap), dtype=torch.int32, device="cuda"),
            "rx": torch.zeros((R, cap, H), dtype=torch.int16, device="cuda"),
            "rw": torch.zeros((R, cap, k), dtype=torch.float32, device="cuda"),
            "ri": torch.zeros((R, cap, k), dtype=torch.int32, device="cuda"),
            "out": torch.empty((T, H), dtype=torch.int16, device="cuda"),
        })
    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    res = {"plan_dispatch": [], "combine": [], "plan": [], "dispatch": []}
    for i in range(warmup + reps):
        s = sets[i % nsets]
        e = [ev() for _ in range(8)]
        torch.cuda.synchronize()
        e[0].record(stream)
        M.mep_plan_dispatch(m.h, s["idx"], T, s["counts"], s["spos"], s["x"], s["w"], s["rx"],
                            None, s["rw"], s["ri"], stream)
        e[1].record(stream)
        torch.cuda.synchronize()
        e[2].record(stream)
        M.mep_combine(m.h, M.MEP_RANK_MAJOR, s["rx"], s["w"], s["out"], stream)
        e[3].record(stream)
        torch.cuda.synchronize()
        e[4].record(stream)
        M.mep_plan(m.h, s["idx"], T, s["counts"], s["spos"], stream)
        e[5].record(stream)
        torch.cuda.synchronize()
        e[6].record(stream)
        M.mep_dispatch(m.h, s["x"], s["w"], s["idx"], s["rx"], None, s["rw"], s["ri"], stream)
        e[7].record(stream)
        M.mep_reset(m.h, stream)
        torch.cuda.synchronize()
        if i >= warmup:
            res["plan_dispatch"].append(e[0].elapsed_time(e[1]) * 1e3)
            res["combine"].append(e[2].elapsed_time(e[3]) * 1e3)
            res["plan"].append(e[4].elapsed_time(e[5]) * 1e3)
            res["dispatch"].append(e[6].elapsed_time(e[7]) * 1e3)
    U = int(sets[0]["counts"].sum().item())
    out = {f"{k}_us": round(statistics.median(v), 2) for k, v in res.items()}
    out["tokens"] = T
    out["U"] = U
    out["dispatch_bytes"] = dispatch_bytes(T, H, k, U, False) + plan_bytes(T, k, R, U)
    out["combine_bytes"] = combine_bytes(T, H, k, U)
    return out


def copy_ceiling(torch, nbytes=512 << 20, reps=20):
    """Read+write rate of a plain device-to-device copy (torch's copy kernel) over
    rotating 512 MiB buffers: the practical HBM ceiling for streaming traffic."""
    n = 3
    src = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(n)]
    dst = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(n)]
    stream = torch.cuda.current_stream()
    for i in range(3):
        dst[i % n].copy_(src[i % n])
    ms = _loop_ms(torch, stream, lambda i: dst[i % n].copy_(src[(i + 1) % n]), reps)
    del src, dst
    return round(2 * nbytes / (ms * 1e-3) / 1e9, 1)


def cpu_baseline(wl, inp, budget_s=20.0):
    """The CPU oracle, single-threaded, on a bounded token sample of the same
    workload: plan + FP8 dispatch + combine of the first `ts` tokens."""
    from oracle import oracle as O
    ts = 512
    sub = {"x": inp["x"][:ts], "indices": inp["indices"][:ts], "weights": inp["weights"][:ts]}
    R, epr, cap, H, k = wl.ranks, wl.experts_per_rank, wl.cap, wl.hidden, wl.topk
    # expert outputs for the sample, prepared untimed
    pl = O.plan(sub["indices"], R, epr, cap)
    d = O.dispatch(sub["x"], sub["weights"], sub["indices"], pl, R, epr, cap, True)
    y = O.expert_dequant(d["recv_x"], d["recv_scales"], 0.5)
    U = int(pl["recv_counts"].sum())
    nbytes = (plan_bytes(ts, k, R, U) + dispatch_bytes(ts, H, k, U, True)
              + combine_bytes(ts, H, k, U))
    times = []
    t_end = time.perf_counter() + budget_s
    while time.perf_counter() < t_end or len(times) < 2:
        t0 = time.perf_counter()
        pl = O.plan(sub["indices"], R, epr, cap)
        d = O.dispatch(sub["x"], sub["weights"], sub["indices"], pl, R, epr, cap, True)
        O.combine(y, sub["weights"], sub["indices"], pl, epr, cap)
        times.append(time.perf_counter() - t0)
        if len(times) >= 20:
            break
    t = statistics.median(times)
    return {"value": round(nbytes / t / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"first {ts} of {wl.tokens} tokens of the prefill workload, plan + FP8 "
                      f"dispatch + combine, single thread, median of {len(times)} runs "
                      f"({t * 1e3:.0f} ms each; expert outputs prepared untimed)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--sets", type=int, default=4)
    ap.add_argument("--decode-reps", type=int, default=200)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(this build has no multi-GPU path)", file=sys.stderr)
        return 2

    import torch
    import combine_mep_plan_amd as M
    from synthetic import WORKLOADS, make_inputs

    wl = WORKLOADS["prefill"]
    inp = make_inputs(wl, 0)
    print(f"[bench] prefill setup: T={wl.tokens} H={wl.hidden} R={wl.ranks} "
          f"epr={wl.experts_per_rank} k={wl.topk} sets={args.sets}", file=sys.stderr, flush=True)
    m, sets, U = setup_prefill(M, torch, wl, inp, args.sets)
    T, H, k, R = wl.tokens, wl.hidden, wl.topk, wl.ranks
    ms_step, times = time_prefill(M, torch, m, sets, wl, args.steps, args.warmup)
    b_plan, b_disp, b_comb = (plan_bytes(T, k, R, U), dispatch_bytes(T, H, k, U, True),
                              combine_bytes(T, H, k, U))
    step_bytes = b_plan + b_disp + b_comb
    value = step_bytes / (ms_step * 1e-3) / 1e9
    print(f"[bench] prefill done: {ms_step * 1e3:.1f} us/step", file=sys.stderr, flush=True)

    nbytes = {"plan_dispatch": b_plan + b_disp, "combine": b_comb, "plan": b_plan,
              "dispatch": b_disp}
    ops = {}
    for name, ms in times.items():
        o = {"us": round(ms * 1e3, 2), "bytes": nbytes[name]}
        o["GBps"] = round(o["bytes"] / (ms * 1e-3) / 1e9, 1)
        o["frac"] = round(o["GBps"] / HBM_PEAK_GBS, 4)
        ops[name] = o
    dom = max(("plan_dispatch", "combine"), key=lambda n: ops[n]["us"])
    kernel_file = {"plan_dispatch": "dispatch.hip", "combine": "combine.hip"}[dom]
    achieved = ops[dom]["bytes"] / (ops[dom]["us"] * 1e-6) / 1e9
    traffic = profile_traffic(f"{dom}_prefill_pmc.txt", src_digest(kernel_file))
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic, "algorithmic_bytes": ops[dom]["bytes"]}

    copy_gbs = copy_ceiling(torch)
    roofline["copy_ceiling_GBps"] = copy_gbs
    dwl = WORKLOADS["decode"]
    print("[bench] decode latency", file=sys.stderr, flush=True)
    decode = time_decode(M, torch, dwl, make_inputs(dwl, 0), args.decode_reps, 20)

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl, inp)

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "prefill: 4096 tokens x 7168 hidden, top-8 of 256 experts on 8 "
                               "virtual ranks x 32, FP8 E4M3 dispatch (fp32 scale per 128 "
                               "columns), bf16 combine with fp32 accumulation",
                   "tokens": T, "hidden": H, "ranks": R, "experts_per_rank": wl.experts_per_rank,
                   "topk": k, "unique_rows": U, "step_bytes": step_bytes,
                   "buffer_sets": args.sets, "hbm_frac": round(value / HBM_PEAK_GBS, 4)},
        "ops": ops,
        "decode_128": decode,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
