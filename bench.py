"""Benchmark of the MoE dispatch/combine hot path on one MI355X.

Headline step (`value`): the whole path on one batch of the prefill workload
-- routing plan + FP8 dispatch through the fused mep_plan_dispatch (OCP E4M3,
one fp32 scale per 128 columns), bf16 combine, reset -- for 4096 tokens x
7168 hidden, top-8 of 256 experts on 8 virtual ranks: the shape and dtypes of
the MORI README's bandwidth table.  The timed steps rotate over buffer sets
whose inputs come from seeds 0, 1 and 2.  value = the algorithmic HBM bytes
of the timed steps / their time.

Also measured, each on its own buffers: decode latency (128 tokens, bf16 both
ways), the skewed-routing workload (Zipf 1.2, 16 ranks) and the standard-MoE
workload (FP8 dispatch, expert-major conversion, combine from it; the
single-call standard-MoE dispatch followed by the same combine; and the
conversion of the expert outputs back to rank rows followed by their
combine), and the prefill shape with an MXFP4 dispatch payload and with the
FP8 direct-cast combine payload.  Inputs are synthetic and resident in HBM;
expert outputs are produced once, before timing, by the stand-in expert.
Buffer sets rotate so no step finds its data in the 256 MB Infinity Cache.
Kernel durations come from back-to-back loops of one call each between two
HIP events on the library's stream.  A streaming probe gives what HBM
delivers for each kernel's own mix of reads and writes (the ceilings the
roofline fractions are set against).  The oracle's own rate on the whole
prefill workload is reported beside the GPU's (cpu_baseline).

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
                    [--no-extra | --extra skew,stdmoe,prefill_mxfp4,prefill_fp8direct]
                    [--sweep 256,1024,8192] [--decode-only]
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
HEADLINE_SEEDS = (0, 1, 2)


# --------------------------------------------------------------------------
# algorithmic bytes: what the method must read and write, per launch
# --------------------------------------------------------------------------

def plan_bytes(T, k, R, U):
    return T * k * 4 + U * 4 + R * 4            # ids in; src_token_pos, counts out


def row_bytes(H, quant):
    # received row and its scales: bf16; E4M3 + fp32 per 128; E2M1 + E8M0 per 32
    return {"none": H * 2, "fp8": H + H // 128 * 4, "mxfp4": H // 2 + H // 32}[quant]


def dispatch_bytes(T, H, k, U, quant):
    return T * H * 2 + T * k * 8 + U * (row_bytes(H, quant) + k * 8)


def combine_bytes(T, H, k, U):
    return U * H * 2 + T * k * 8 + T * H * 2


def to_expert_major_bytes(T, H, k, U, quant):
    rb = row_bytes(H, quant)
    return U * (rb + k * 4) + T * k * (rb + 4)


def standard_moe_bytes(T, H, k, E, Uem, quant):
    # x and ids read once; each expert row written with its scales and source
    # position; per-expert counts and offsets
    return T * H * 2 + T * k * 4 + Uem * (row_bytes(H, quant) + 4) + E * 8


def cast_fp8_bytes(H, U):
    return U * H * 3          # bf16 rows read, E4M3 rows written


def combine_fp8_bytes(T, H, k, U):
    return U * H + T * k * 8 + T * H * 2


def combine_em_bytes(T, H, k):
    return T * k * H * 2 + T * k * 8 + T * H * 2


def convert_combine_input_bytes(T, H, k, U, Uem):
    # each expert-major row read with its dispatched weight, the route of every
    # (token, top-k position) read, each rank row written
    return Uem * (H * 2 + 4) + T * k * 8 + U * H * 2


def combine_rank_sum_bytes(T, H, k, U):
    return U * H * 2 + T * k * 4 + T * H * 2


def src_digest(name):
    """Digest of the code of a kernel source file and of every header beside it
    (a change to a shared header changes the kernel too).  Comments and blank
    space are left out, so that a comment edit keeps the counters valid."""
    import glob
    import re
    csrc = os.path.join(ROOT, "combine_mep_plan_amd", "csrc")
    h = hashlib.sha256()
    for p in [os.path.join(csrc, name)] + sorted(glob.glob(os.path.join(csrc, "*.h"))):
        with open(p) as f:
            code = re.sub(r"/\*.*?\*/|//[^\n]*", "", f.read(), flags=re.S)
        h.update(" ".join(code.split()).encode())
    return h.hexdigest()[:16]


def profile_traffic(summary_file, digest):
    """HBM bytes per launch measured by rocprofv3 counters for the current kernel
    source, or None if no summary matches this source."""
    p = os.path.join(ROOT, "profiles", summary_file)
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


def _per_call_us(torch, stream, fn, n):
    """Median, p10 and p90 of n calls of fn(i), each bracketed by its own pair
    of HIP events on `stream`; the calls still run back to back on the GPU."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(evs):
        a.record(stream)
        fn(i)
        b.record(stream)
    torch.cuda.synchronize()
    d = [a.elapsed_time(b) * 1e3 for a, b in evs]
    q = statistics.quantiles(d, n=10)
    return {"median": round(statistics.median(d), 2), "p10": round(q[0], 2),
            "p90": round(q[8], 2), "calls": n}


# --------------------------------------------------------------------------
# one workload: buffers, stand-in expert outputs, timed loops
# --------------------------------------------------------------------------

class Runner:
    """Buffer sets of one workload.  Set i holds the inputs of
    seeds[i % len(seeds)]; the per-operation loops use the sets of seeds[0]
    only, so that the plan in the handle always matches the set a call
    reads."""

    def __init__(self, M, torch, wl, seeds, nsets):
        from synthetic import make_inputs
        self.M, self.torch, self.wl = M, torch, wl
        T, H, R, cap, k = wl.tokens, wl.hidden, wl.ranks, wl.cap, wl.topk
        self.quant = wl.quant
        self.em = wl.layout == "expert_major"
        self.fp8c = wl.combine == "fp8_direct"
        qmode = {"none": M.MEP_QUANT_NONE, "fp8": M.MEP_QUANT_FP8_E4M3_BLOCK128,
                 "mxfp4": M.MEP_QUANT_MXFP4}[wl.quant]
        self.m = M.Mep(H, wl.experts_per_rank, k, cap, R, quant=qmode)
        self.stream = torch.cuda.current_stream()
        self.seeds = list(seeds)
        inputs = {sd: make_inputs(wl, sd) for sd in self.seeds}
        dev = lambda a: torch.from_numpy(a).cuda()  # noqa: E731
        # received rows: bf16 values, E4M3 bytes, or packed E2M1 bytes
        rcols, rdt = {"none": (H, torch.int16), "fp8": (H, torch.uint8),
                      "mxfp4": (H // 2, torch.uint8)}[wl.quant]
        nb = wl.scale_dim
        self.sets = []
        for i in range(nsets):
            inp = inputs[self.seeds[i % len(self.seeds)]]
            s = {
                "seed": self.seeds[i % len(self.seeds)],
                "x": dev(inp["x"].view(np.int16)), "w": dev(inp["weights"]),
                "idx": dev(inp["indices"]),
                "counts": torch.zeros(R, dtype=torch.int32, device="cuda"),
                "spos": torch.zeros((R, cap), dtype=torch.int32, device="cuda"),
                "rx": torch.zeros((R, cap, rcols), dtype=rdt, device="cuda"),
                "rs": (torch.zeros((R, cap, nb), dtype=torch.float32, device="cuda")
                       if nb else None),
                "rw": torch.zeros((R, cap, k), dtype=torch.float32, device="cuda"),
                "ri": torch.zeros((R, cap, k), dtype=torch.int32, device="cuda"),
                "out": torch.empty((T, H), dtype=torch.int16, device="cuda"),
            }
            if self.em:
                ce = wl.cap_em
                s["emx"] = torch.zeros((ce, rcols), dtype=rdt, device="cuda")
                s["ems"] = (torch.zeros((ce, nb), dtype=torch.float32, device="cuda")
                            if nb else None)
                s["emc"] = torch.zeros(wl.experts, dtype=torch.int32, device="cuda")
                s["emo"] = torch.zeros(wl.experts + 1, dtype=torch.int32, device="cuda")
                s["emp"] = torch.zeros(ce, dtype=torch.int32, device="cuda")
                s["conv"] = torch.zeros((R, cap, H), dtype=torch.int16, device="cuda")
            self.plan_dispatch(s)
            if self.em:
                self.to_em(s)
                s["y"] = self.stand_in(s["emx"], s["ems"])
            else:
                s["y"] = self.stand_in(s["rx"], s["rs"])
            if self.fp8c:
                s["y8"] = torch.zeros(s["y"].shape, dtype=torch.uint8, device="cuda")
            M.mep_reset(self.m.h, self.stream)
            self.sets.append(s)
        torch.cuda.synchronize()
        for s in self.sets:
            s["U"] = int(s["counts"].sum().item())
            s["Uem"] = int(s["emc"].sum().item()) if self.em else 0
        self.op_sets = [s for s in self.sets if s["seed"] == self.seeds[0]]
        self.U = self.op_sets[0]["U"]
        self.Uem = self.op_sets[0]["Uem"]

    def stand_in(self, x, scales):
        # expert outputs (harness, untimed): identity for bf16 payloads,
        # bf16((decode(q) * scale) * mult) for E4M3 and MX FP4 payloads
        torch = self.torch
        if scales is None:
            return x
        mult = 0.5 if self.wl.expert == "dequant_half" else 1.0
        if self.quant == "mxfp4":
            lut = torch.tensor([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6],
                               dtype=torch.float32, device=x.device)
            b = x.long()
            q = torch.stack([lut[b & 15], lut[b >> 4]], dim=-1).flatten(-2)
            e = scales.view(torch.uint8).float()
            s = torch.exp2(e - 127.0).repeat_interleave(32, dim=-1)
        else:
            q = x.view(torch.float8_e4m3fn).float()
            s = scales.repeat_interleave(128, dim=-1)
        return ((q * s) * mult).to(torch.bfloat16).view(torch.int16)

    def plan_dispatch(self, s):
        self.M.mep_plan_dispatch(self.m.h, s["idx"], self.wl.tokens, s["counts"], s["spos"],
                                 s["x"], s["w"], None, s["rx"], s["rs"], s["rw"], s["ri"],
                                 self.stream)

    def plan(self, s):
        self.M.mep_plan(self.m.h, s["idx"], self.wl.tokens, s["counts"], s["spos"], self.stream)

    def dispatch(self, s):
        self.M.mep_dispatch(self.m.h, s["x"], s["w"], None, s["idx"], s["rx"], s["rs"], s["rw"],
                            s["ri"], self.stream)

    def standard_moe(self, s):
        self.M.mep_dispatch_standard_moe(self.m.h, s["idx"], self.wl.tokens, s["x"], None,
                                         s["emx"], s["ems"], s["emc"], s["emo"], s["emp"],
                                         self.wl.cap_em, self.stream)

    def step_standard(self, s):
        self.standard_moe(s)
        self.combine(s)
        self.M.mep_reset(self.m.h, self.stream)

    def to_em(self, s):
        self.M.mep_to_expert_major(self.m.h, s["rx"], s["rs"], s["ri"], s["counts"], s["spos"],
                                   s["emx"], s["ems"], s["emc"], s["emo"], s["emp"],
                                   self.wl.cap_em, self.stream)

    def convert(self, s):
        self.M.mep_convert_combine_input(self.m.h, s["y"], s["rw"], s["conv"], self.stream)

    def combine_rank_sum(self, s):
        self.M.mep_combine(self.m.h, self.M.MEP_RANK_SUM, s["conv"], None, s["out"], self.stream)

    def step_convert(self, s):
        # dispatch, expert-major layout, experts (outputs prepared untimed),
        # back to rank rows, combine of the rank rows
        self.plan_dispatch(s)
        self.to_em(s)
        self.convert(s)
        self.combine_rank_sum(s)
        self.M.mep_reset(self.m.h, self.stream)

    def layout(self):
        return self.M.MEP_EXPERT_MAJOR if self.em else self.M.MEP_RANK_MAJOR

    def cast(self, s):
        self.M.mep_cast_fp8_direct(self.m.h, self.layout(), s["y"], s["y8"], self.stream)

    def combine_in_flight(self, s):
        self.M.mep_combine_fp8_direct(self.m.h, self.layout(), s["y"], s["w"], s["out"],
                                      self.stream)

    def step_in_flight(self, s):
        self.plan_dispatch(s)
        self.combine_in_flight(s)
        self.M.mep_reset(self.m.h, self.stream)

    def combine(self, s):
        if self.fp8c:
            self.M.mep_combine_fp8(self.m.h, self.layout(), s["y8"], s["w"], s["out"], self.stream)
        else:
            self.M.mep_combine(self.m.h, self.layout(), s["y"], s["w"], s["out"], self.stream)

    def step(self, s):
        self.plan_dispatch(s)
        if self.em:
            self.to_em(s)
        if self.fp8c:
            self.cast(s)
        self.combine(s)
        self.M.mep_reset(self.m.h, self.stream)

    def loop(self, fn, n, prime=True, sets=None):
        # one untimed call per buffer set first (prime), so that no loop pays
        # for a first launch of its kernels; the headline step loop has its own
        # warmup steps instead
        sets = self.op_sets if sets is None else sets
        if prime:
            for s in sets:
                fn(s)
        return _loop_ms(self.torch, self.stream, lambda i: fn(sets[i % len(sets)]), n)

    def per_call(self, fn, n=100):
        sets = self.op_sets
        return _per_call_us(self.torch, self.stream, lambda i: fn(sets[i % len(sets)]), n)

    def bytes(self, s=None):
        """Algorithmic bytes of every operation for the routing of set s
        (default: the sets the per-operation loops use)."""
        wl = self.wl
        U, Uem = (self.U, self.Uem) if s is None else (s["U"], s["Uem"])
        T, H, k, R = wl.tokens, wl.hidden, wl.topk, wl.ranks
        b = {"plan": plan_bytes(T, k, R, U), "dispatch": dispatch_bytes(T, H, k, U, self.quant)}
        b["plan_dispatch"] = b["plan"] + b["dispatch"]
        if self.em:
            b["to_expert_major"] = to_expert_major_bytes(T, H, k, U, self.quant)
            b["combine"] = combine_em_bytes(T, H, k)
            b["dispatch_standard_moe"] = standard_moe_bytes(T, H, k, wl.experts, Uem,
                                                            self.quant)
            b["step_standard"] = b["dispatch_standard_moe"] + b["combine"]
            b["convert_combine_input"] = convert_combine_input_bytes(T, H, k, U, Uem)
            b["combine_rank_sum"] = combine_rank_sum_bytes(T, H, k, U)
            b["step_convert"] = (b["plan_dispatch"] + b["to_expert_major"]
                                 + b["convert_combine_input"] + b["combine_rank_sum"])
        elif self.fp8c:
            b["cast_fp8_direct"] = cast_fp8_bytes(H, U)
            b["combine"] = combine_fp8_bytes(T, H, k, U)
            b["combine_in_flight"] = combine_bytes(T, H, k, U)
            b["step_in_flight"] = b["plan_dispatch"] + b["combine_in_flight"]
        else:
            b["combine"] = combine_bytes(T, H, k, U)
        b["step"] = (b["plan_dispatch"] + b["combine"] + b.get("to_expert_major", 0)
                     + b.get("cast_fp8_direct", 0))
        return b

    def measure(self, steps, warmup):
        """Step loop over every set (all seeds), then one loop per operation
        over the sets of the first seed."""
        for i in range(warmup):
            self.step(self.sets[i % len(self.sets)])
        step_ms = self.loop(self.step, steps, prime=False, sets=self.sets)
        assert self.M.mep_get_status(self.m.h, self.stream) == 0
        # the bytes of exactly the timed steps (their sets in loop order)
        step_bytes = sum(self.bytes(self.sets[i % len(self.sets)])["step"]
                         for i in range(steps)) / steps
        times = {"step": step_ms}
        # run-to-run spread: the same loop repeated (not part of `value`)
        self.step_repeats = [round(self.loop(self.step, steps, sets=self.sets) * 1e3, 2)
                             for _ in range(4)]
        # each seed alone (not part of `value`)
        by_seed = {}
        for sd in self.seeds:
            ss = [s for s in self.sets if s["seed"] == sd]
            ms = self.loop(self.step, steps, sets=ss)
            by_seed[str(sd)] = {"U": ss[0]["U"], "step_us": round(ms * 1e3, 2),
                                "GBps": round(self.bytes(ss[0])["step"] / (ms * 1e-3) / 1e9, 1)}
        times["plan_dispatch"] = self.loop(self.plan_dispatch, steps)
        if self.em:
            times["to_expert_major"] = self.loop(self.to_em, steps)
            times["convert_combine_input"] = self.loop(self.convert, steps)
            times["combine_rank_sum"] = self.loop(self.combine_rank_sum, steps)
        if self.fp8c:
            times["cast_fp8_direct"] = self.loop(self.cast, steps)
            # the same rounding applied in registers by the combine (one device)
            times["combine_in_flight"] = self.loop(self.combine_in_flight, steps)
        times["combine"] = self.loop(self.combine, steps)
        times["plan"] = self.loop(self.plan, steps)
        times["dispatch"] = self.loop(self.dispatch, steps)
        if self.fp8c:
            times["step_in_flight"] = self.loop(self.step_in_flight, steps)
        if self.em:
            times["step_convert"] = self.loop(self.step_convert, steps)
            # standard-MoE dispatch straight into the expert-major layout, then
            # the same expert-major combine
            times["step_standard"] = self.loop(self.step_standard, steps)
            assert self.M.mep_get_status(self.m.h, self.stream) == 0
            times["dispatch_standard_moe"] = self.loop(self.standard_moe, steps)
        self.M.mep_reset(self.m.h, self.stream)
        nbytes = self.bytes()
        nbytes["step"] = step_bytes
        # the pages' own bandwidth figure: payload bytes received (dispatch) or
        # sent back (combine) per second; context, not the roofline
        wl = self.wl
        payload = {"dispatch": self.U * row_bytes(wl.hidden, self.quant),
                   "combine": (self.Uem if self.em else self.U) * wl.hidden * 2}
        payload["plan_dispatch"] = payload["dispatch"]
        ops = {}
        for name, ms in times.items():
            o = {"us": round(ms * 1e3, 2), "bytes": int(round(nbytes[name]))}
            o["GBps"] = round(o["bytes"] / (ms * 1e-3) / 1e9, 1)
            o["frac"] = round(o["GBps"] / HBM_PEAK_GBS, 4)
            if name in payload:
                o["payload_GBps"] = round(payload[name] / (ms * 1e-3) / 1e9, 1)
            ops[name] = o
        ops["step"]["repeats_us"] = self.step_repeats
        ops["step"]["by_seed"] = by_seed
        # per-call spread (context; the figures above are loop averages).
        # Each call is bracketed by its own events; the calls before a
        # plan-dependent one leave the plan it needs.
        per = {"step": self.per_call(self.step),
               "plan_dispatch": self.per_call(self.plan_dispatch),
               "plan": self.per_call(self.plan)}
        per["dispatch"] = self.per_call(self.dispatch)
        if self.em:
            per["to_expert_major"] = self.per_call(self.to_em)
            per["convert_combine_input"] = self.per_call(self.convert)
        per["combine"] = self.per_call(self.combine)
        self.M.mep_reset(self.m.h, self.stream)
        for name, v in per.items():
            ops[name]["per_call_us"] = v
        return ops

    def output_of_first_set(self):
        """The combined output of the first set, computed afresh (plan,
        dispatch, combine on that set's own inputs), as host bf16 bits."""
        s = self.op_sets[0]
        self.plan_dispatch(s)
        self.combine(s)
        self.M.mep_reset(self.m.h, self.stream)
        self.torch.cuda.synchronize()
        return s["out"].cpu().numpy().view(np.uint16)


def time_decode(M, torch, wl, reps, warmup):
    """128-token latency, bf16 both ways, identity expert (combine reads the
    receive buffers).  device: the calls are queued behind a short GPU sleep, so
    the two events bracket only GPU work (launch processing included, host
    submission excluded); host: the GPU is idle when the first event is
    recorded, so host submission time is included.  graph: plan+dispatch and
    combine captured in one HIP graph and replayed (device timing).
    launch_floor: the library's smallest kernel (one workgroup converting two
    values: a load and a store) timed the same way, eager and as a graph; and
    the replay of an empty graph."""
    r = Runner(M, torch, wl, (0,), 4)
    stream = r.stream
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def timed(fns, s, queued):
        a, b = ev(), ev()
        torch.cuda.synchronize()
        if queued:
            torch.cuda._sleep(200_000)  # ~80 us of GPU spin while the host queues the calls
        a.record(stream)
        for fn in fns:
            fn(s)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3

    # launch floor: a one-workgroup kernel of the library (one load, one store)
    # queued and timed the same way, for scale
    fin = torch.zeros(64, dtype=torch.float32, device="cuda")
    fout = torch.zeros(64, dtype=torch.int16, device="cuda")
    seqs = {"plan_dispatch": [r.plan_dispatch], "combine": [r.combine], "plan": [r.plan],
            "dispatch": [r.dispatch],
            "launch_floor": [lambda s: M.mep_probe_bf16(fin, fout, 2, r.stream)]}
    res = {}
    for i in range(warmup + reps):
        s = r.sets[i % len(r.sets)]
        for name, fns in seqs.items():
            for queued in (True, False):
                t = timed(fns, s, queued)
                if i >= warmup:
                    res.setdefault(f"{name}{'' if queued else '_host'}_us", []).append(t)
        M.mep_reset(r.m.h, stream)
    out = {k: round(statistics.median(v), 2) for k, v in res.items()}
    for k, v in res.items():
        if not k.endswith("_host_us"):
            q = statistics.quantiles(v, n=10)
            out[k.replace("_us", "_p10_p90_us")] = [round(q[0], 2), round(q[8], 2)]
    s = r.sets[0]

    def graph_us(fns):
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            r.stream = torch.cuda.current_stream()  # capture stream
            for fn in fns:
                fn(s)
        r.stream = stream
        g_us = []
        for i in range(warmup + reps):
            a, b = ev(), ev()
            torch.cuda.synchronize()
            torch.cuda._sleep(200_000)
            a.record(stream)
            graph.replay()
            b.record(stream)
            torch.cuda.synchronize()
            if i >= warmup:
                g_us.append(a.elapsed_time(b) * 1e3)
        del graph
        return round(statistics.median(g_us), 2)

    # a plan+dispatch starts a round: a reset precedes each capture holding one
    M.mep_reset(r.m.h, stream)
    out["graph_plan_dispatch_us"] = graph_us([r.plan_dispatch])
    out["graph_combine_us"] = graph_us([r.combine])
    M.mep_reset(r.m.h, stream)
    out["graph_plan_dispatch_combine_us"] = graph_us([r.plan_dispatch, r.combine])
    out["graph_launch_floor_us"] = graph_us(seqs["launch_floor"])
    out["graph_empty_us"] = graph_us([])  # a replay that launches nothing
    M.mep_reset(r.m.h, stream)
    # back outside capture (the next eager plan leaves the graph's status word)
    r.plan_dispatch(r.sets[0])
    M.mep_reset(r.m.h, stream)
    nb = r.bytes()
    out.update({"tokens": wl.tokens, "U": r.U, "dispatch_bytes": nb["plan_dispatch"],
                "combine_bytes": nb["combine"]})
    return out


def env_info(torch):
    p = torch.cuda.get_device_properties(0)
    return {"device": p.name, "arch": getattr(p, "gcnArchName", ""),
            "compute_units": p.multi_processor_count, "hip": torch.version.hip,
            "torch": torch.__version__, "host_cpus": len(os.sched_getaffinity(0))}


def sets_sweep(M, torch, wl, counts, steps):
    """How the prefill loops depend on the number of rotated buffer sets (all
    seed 0): step, combine and fused plan+dispatch µs for each count.  The
    token rows of a few sets stay in the 256 MB Infinity Cache; many sets
    leave every launch cold."""
    r = Runner(M, torch, wl, (0,), max(counts))
    out = {}
    for n in counts:
        sets = r.sets[:n]
        for i in range(20):
            r.step(sets[i % n])
        st = r.loop(r.step, steps, sets=sets)
        r.plan_dispatch(sets[0])
        cb = r.loop(r.combine, steps, sets=sets)
        pd = r.loop(r.plan_dispatch, steps, sets=sets)
        r.M.mep_reset(r.m.h, r.stream)
        out[n] = {"step_us": round(st * 1e3, 2), "combine_us": round(cb * 1e3, 2),
                  "plan_dispatch_us": round(pd * 1e3, 2)}
    del r
    torch.cuda.empty_cache()
    return out


PROBE_WAVES = (28672, 57344, 86016, 114688, 172032)


def _probe_buffers(torch, units):
    """One source and one destination buffer for the streaming probe; each launch
    takes the next region of them, the regions of a cycle spanning at least
    1 GiB each way (so no launch finds its data in the 256 MB Infinity Cache)."""
    span = max(1 << 30, 3 * 1024 * max(max(r, w) for r, w in units.values()))
    return (span, torch.empty(span, dtype=torch.uint8, device="cuda"),
            torch.empty(span, dtype=torch.uint8, device="cuda"))


def _probe_ms(M, torch, bufs, ru, wu, nw, reps):
    span, src_all, dst_all = bufs
    stream = torch.cuda.current_stream()
    nreg = span // (1024 * max(ru, wu))

    def fn(i):
        j = i % nreg
        src = src_all[j * ru * 1024:(j + 1) * ru * 1024] if ru else src_all[:16]
        dst = dst_all[j * wu * 1024:(j + 1) * wu * 1024] if wu else dst_all[:16]
        M.mep_probe_stream(src, dst, nw, ru, wu, stream)
    for i in range(nreg):
        fn(i)
    return _loop_ms(torch, stream, fn, max(reps, nreg))


def _probe_entry(ru, wu, by_waves):
    best = min(by_waves, key=by_waves.get)
    ms = by_waves[best]
    out = {"GBps": round((ru + wu) * 1024 / (ms * 1e-3) / 1e9, 1), "us": round(ms * 1e3, 2),
           "read_bytes": ru * 1024, "write_bytes": wu * 1024, "waves": best}
    if len(by_waves) > 1:
        out["us_by_waves"] = {str(w): round(v * 1e3, 2) for w, v in by_waves.items()}
    return out


def stream_ceilings(M, torch, wl, U, reps=20):
    """What HBM gives plain streams with the prefill kernels' own byte mixes:
    the library's streaming probe with the same bytes read and written,
    spread evenly over the waves, non-temporal, each wave's loads before its
    stores.  The mixes are timed at several wave counts (4096 tokens x 7
    slices = 28672 is the kernels' old shape; plain streams do better with
    more, smaller waves) and the fastest is the ceiling.  Also the combine's
    reads alone and writes alone."""
    T, H, k = wl.tokens, wl.hidden, wl.topk
    waves = T * ((H // 8 + 127) // 128)
    mixes = {
        "combine_mix": (U * H * 2 + T * k * 8, T * H * 2),
        "dispatch_mix": (T * H * 2 + T * k * 8, U * (row_bytes(H, "fp8") + k * 8)),
        "combine_reads_only": (U * H * 2 + T * k * 8, 0),
        "combine_writes_only": (0, T * H * 2),
        # the shapes plain streams do best with on this GPU (one wave per
        # 2 KiB read, per 1 KiB written), for the same byte counts
        "combine_reads_2k_waves": (U * H * 2 + T * k * 8, 0),
        "dispatch_writes_1k_waves": (0, U * (row_bytes(H, "fp8") + k * 8)),
    }
    units = {n: (-(-r // 1024), -(-w // 1024)) for n, (r, w) in mixes.items()}
    wave_counts = {n: [waves] for n in mixes}
    for n in ("combine_mix", "dispatch_mix"):
        wave_counts[n] = [w for w in (waves, 2 * waves, 3 * waves, 4 * waves, 6 * waves)
                          if -(-max(units[n]) // w) <= 16]
    wave_counts["combine_reads_2k_waves"] = [-(-units["combine_reads_2k_waves"][0] // 2)]
    wave_counts["dispatch_writes_1k_waves"] = [units["dispatch_writes_1k_waves"][1]]
    bufs = _probe_buffers(torch, units)
    out = {}
    for name, (ru, wu) in units.items():
        out[name] = _probe_entry(ru, wu, {nw: _probe_ms(M, torch, bufs, ru, wu, nw, reps)
                                          for nw in wave_counts[name]})
    del bufs
    return out


def op_mixes(wl, U, Uem, quant, em, fp8c):
    """Bytes read and written by each main operation of a workload (the same
    algorithmic bytes as Runner.bytes, split by direction)."""
    T, H, k, E = wl.tokens, wl.hidden, wl.topk, wl.experts
    rb = row_bytes(H, quant)
    mixes = {"dispatch": (T * H * 2 + T * k * 8, U * (rb + k * 8))}
    if em:
        mixes["combine"] = (T * k * H * 2 + T * k * 8, T * H * 2)
        mixes["to_expert_major"] = (U * (rb + k * 4), T * k * (rb + 4))
        mixes["dispatch_standard_moe"] = (T * H * 2 + T * k * 4, Uem * (rb + 4) + E * 8)
        mixes["convert_combine_input"] = (Uem * (H * 2 + 4) + T * k * 8, U * H * 2)
        mixes["combine_rank_sum"] = (U * H * 2 + T * k * 4, T * H * 2)
    elif fp8c:
        mixes["cast_fp8_direct"] = (U * H * 2, U * H)
        mixes["combine"] = (U * H + T * k * 8, T * H * 2)
        mixes["combine_in_flight"] = (U * H * 2 + T * k * 8, T * H * 2)
    else:
        mixes["combine"] = (U * H * 2 + T * k * 8, T * H * 2)
    return mixes


def workload_ceilings(M, torch, mixes, reps=20):
    """The streaming probe at each operation's own mix of reads and writes,
    timed at several wave counts (at most 16 KiB read per wave); the fastest
    is that operation's ceiling."""
    units = {n: (-(-r // 1024), -(-w // 1024)) for n, (r, w) in mixes.items()}
    bufs = _probe_buffers(torch, units)
    out = {}
    for name, (ru, wu) in units.items():
        counts = [w for w in PROBE_WAVES if -(-ru // w) <= 16]
        out[name] = _probe_entry(ru, wu, {nw: _probe_ms(M, torch, bufs, ru, wu, nw, reps)
                                          for nw in counts})
    del bufs
    return out


def cpu_baseline(wl, inp, gpu_out=None):
    """The CPU oracle, single-threaded, on the whole prefill workload (4096
    tokens): plan + FP8 dispatch, then combine, each timed once (one pass
    takes about 13 s; the expert stand-in between them is untimed).  The
    oracle's combined rows are compared with the GPU's for the same inputs
    (`gpu_out`, bf16 bits)."""
    from oracle import oracle as O
    T, R, epr, cap, H, k = wl.tokens, wl.ranks, wl.experts_per_rank, wl.cap, wl.hidden, wl.topk
    t0 = time.perf_counter()
    pl = O.plan(inp["indices"], R, epr, cap)
    d = O.dispatch(inp["x"], inp["weights"], inp["indices"], pl, R, epr, cap, True)
    t1 = time.perf_counter()
    y = O.expert_dequant(d["recv_x"], d["recv_scales"], 0.5)
    t2 = time.perf_counter()
    out = O.combine(y, inp["weights"], inp["indices"], pl, epr, cap)
    t3 = time.perf_counter()
    U = int(pl["recv_counts"].sum())
    nbytes = plan_bytes(T, k, R, U) + dispatch_bytes(T, H, k, U, "fp8") + combine_bytes(T, H, k, U)
    t = (t1 - t0) + (t3 - t2)
    return {"value": round(nbytes / t / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"the whole prefill workload, seed 0 ({T} tokens, U = {U} rows): plan + "
                      f"FP8 dispatch + combine, single thread, one pass "
                      f"({t:.1f} s; expert outputs prepared untimed in between)",
            "phases_ms": {"plan_dispatch": round((t1 - t0) * 1e3, 1),
                          "combine": round((t3 - t2) * 1e3, 1)},
            "bytes": nbytes,
            "sample_matches_gpu": (None if gpu_out is None else
                                   bool(np.array_equal(out, gpu_out)))}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--sets", type=int, default=18,
                    help="prefill buffer sets; set i holds the inputs of seed i %% 3 (the token "
                         "rows of four or fewer sets stay in the 256 MB Infinity Cache)")
    ap.add_argument("--decode-reps", type=int, default=200)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="prefill and decode only")
    ap.add_argument("--extra", default="skew,stdmoe,prefill_mxfp4,prefill_fp8direct",
                    help="comma-separated extra workloads to measure after prefill and decode")
    ap.add_argument("--sweep", default="",
                    help="comma-separated token counts: the prefill configuration at each "
                         "(step, fused plan+dispatch, combine), reported under 'sweep'")
    ap.add_argument("--decode-only", action="store_true",
                    help="only the 128-token decode leg (for kernel traces of it)")
    ap.add_argument("--sets-sweep", default="",
                    help="comma-separated buffer-set counts: prefill step, combine and fused "
                         "plan+dispatch at each, reported under 'sets_sweep'")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the library drives one device; the sharded design is not built)", file=sys.stderr)
        return 2

    import torch
    import combine_mep_plan_amd as M
    from synthetic import WORKLOADS, make_inputs

    say = lambda s: print(f"[bench] {s}", file=sys.stderr, flush=True)  # noqa: E731
    dwl = WORKLOADS["decode"]
    if args.decode_only:
        say("decode latency only")
        print(json.dumps({"decode_128": time_decode(M, torch, dwl, args.decode_reps, 20)}),
              flush=True)
        return 0

    wl = WORKLOADS["prefill"]
    say(f"prefill: T={wl.tokens} H={wl.hidden} R={wl.ranks} epr={wl.experts_per_rank} "
        f"k={wl.topk} sets={args.sets} seeds={list(HEADLINE_SEEDS)}")
    run = Runner(M, torch, wl, HEADLINE_SEEDS, args.sets)
    ops = run.measure(args.steps, args.warmup)
    U = run.U
    gpu_out = run.output_of_first_set()
    del run
    torch.cuda.empty_cache()
    ms_step = ops["step"]["us"] * 1e-3
    step_bytes = ops["step"]["bytes"]
    value = step_bytes / (ms_step * 1e-3) / 1e9
    say(f"prefill step {ops['step']['us']} us, {value:.0f} GB/s")

    say("stream ceilings")
    ceil = stream_ceilings(M, torch, wl, U)
    dom = max(("plan_dispatch", "combine"), key=lambda n: ops[n]["us"])
    kfile = {"plan_dispatch": "dispatch.hip", "combine": "combine.hip"}[dom]
    summary = {"plan_dispatch": "dispatch_prefill_pmc.txt",
               "combine": "combine_prefill_pmc.txt"}[dom]
    mix = ceil["combine_mix" if dom == "combine" else "dispatch_mix"]["GBps"]
    achieved = ops[dom]["bytes"] / (ops[dom]["us"] * 1e-6) / 1e9
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": profile_traffic(summary, src_digest(kfile)),
                "algorithmic_bytes": ops[dom]["bytes"],
                "mix_ceiling_GBps": mix, "frac_of_mix_ceiling": round(achieved / mix, 4),
                "ceilings": ceil}
    ops["combine"]["frac_of_mix_ceiling"] = round(ops["combine"]["GBps"]
                                                  / ceil["combine_mix"]["GBps"], 4)
    ops["dispatch"]["frac_of_mix_ceiling"] = round(ops["dispatch"]["GBps"]
                                                   / ceil["dispatch_mix"]["GBps"], 4)

    say("decode latency")
    decode = time_decode(M, torch, dwl, args.decode_reps, 20)
    torch.cuda.empty_cache()

    extra = {}
    if not args.no_extra:
        for name in [n for n in args.extra.split(",") if n]:
            nsets = 6  # as for the prefill loops: no set's token rows stay cached
            xwl = WORKLOADS[name]
            say(f"{name}: T={xwl.tokens} R={xwl.ranks} epr={xwl.experts_per_rank}")
            r = Runner(M, torch, xwl, (0,), nsets)
            xops = r.measure(max(args.steps // 2, 10), 3)
            xU = r.U
            mixes = op_mixes(xwl, r.U, r.Uem, r.quant, r.em, r.fp8c)
            del r
            torch.cuda.empty_cache()
            # each operation against the probe at its own read/write mix
            xceil = workload_ceilings(M, torch, mixes)
            for op, c in xceil.items():
                xops[op]["frac_of_mix_ceiling"] = round(xops[op]["GBps"] / c["GBps"], 4)
            extra[name] = {"U": xU, "seed": 0, "ops": xops, "mix_ceilings": xceil}
            torch.cuda.empty_cache()

    ssweep = {}
    if args.sets_sweep:
        say("buffer-set sweep")
        ssweep = sets_sweep(M, torch, wl, [int(v) for v in args.sets_sweep.split(",") if v],
                            args.steps)

    sweep = {}
    for T in [int(v) for v in args.sweep.split(",") if v]:
        swl = wl.with_tokens(T, cap=max(T, wl.cap))
        say(f"sweep: T={T}")
        r = Runner(M, torch, swl, (0,), 6)
        o = r.measure(max(args.steps // 2, 10), 10)
        sweep[T] = {"U": r.U, **{n: {"us": o[n]["us"], "GBps": o[n]["GBps"]}
                                 for n in ("step", "plan_dispatch", "combine")}}
        del r
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        say("cpu baseline (oracle, whole prefill workload)")
        cpu = cpu_baseline(wl, make_inputs(wl, 0), gpu_out)

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
        "dtype": "fp8_e4m3 dispatch + bf16 combine (fp32 accumulate)",
        "data": "synthetic",
        "config": {"workload": "prefill: 4096 tokens x 7168 hidden, top-8 of 256 experts on 8 "
                               "virtual ranks x 32, FP8 E4M3 dispatch (fp32 scale per 128 "
                               "columns), bf16 combine with fp32 accumulation",
                   "tokens": wl.tokens, "hidden": wl.hidden, "ranks": wl.ranks,
                   "experts_per_rank": wl.experts_per_rank, "topk": wl.topk,
                   "seeds": list(HEADLINE_SEEDS), "unique_rows_seed0": U,
                   "step_bytes": step_bytes, "buffer_sets": args.sets,
                   "hbm_frac": round(value / HBM_PEAK_GBS, 4)},
        "ops": ops,
        "decode_128": decode,
        "roofline": roofline,
        "workloads": extra,
        **({"sweep": sweep} if sweep else {}),
        **({"sets_sweep": ssweep} if ssweep else {}),
        "cpu_baseline": cpu,
        "env": env_info(torch),
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
