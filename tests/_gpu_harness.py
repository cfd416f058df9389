"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI
on seeded synthetic inputs, run the CPU oracle on the same host arrays, and
compare.  Unwritten receive / expert-major rows are pre-filled with a sentinel
so stray writes show up."""

from __future__ import annotations

import dataclasses

import numpy as np
import torch

import combine_mep_plan_amd as M
from oracle import oracle as O
from synthetic import Workload, make_inputs

SENT8 = 0xA5
SENT16 = 0xA5A5
SENT32 = -0x5A5A5A5B  # int32 sentinel


def dev(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t: torch.Tensor, dtype=None) -> np.ndarray:
    a = t.cpu().numpy()
    if dtype is not None:
        a = a.view(dtype)
    return a


def bf16_ulp_diff(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    def ordered(b):
        b = b.astype(np.int32)
        mag = b & 0x7FFF
        return np.where(b & 0x8000, -mag, mag)
    return np.abs(ordered(a_bits) - ordered(b_bits))


def alloc_recv(wl: Workload):
    R, cap, H, k = wl.ranks, wl.cap, wl.hidden, wl.topk
    fp8 = wl.quant == "fp8"
    recv_x = torch.full((R, cap, H), SENT8 if fp8 else SENT16 - 0x10000,
                        dtype=torch.uint8 if fp8 else torch.int16, device="cuda")
    recv_s = (torch.full((R, cap, H // 128), float("nan"), dtype=torch.float32, device="cuda")
              if fp8 else None)
    recv_w = torch.full((R, cap, k), float("nan"), dtype=torch.float32, device="cuda")
    recv_i = torch.full((R, cap, k), SENT32, dtype=torch.int32, device="cuda")
    return recv_x, recv_s, recv_w, recv_i


@dataclasses.dataclass
class GpuResult:
    m: M.Mep
    x: torch.Tensor
    w: torch.Tensor
    idx: torch.Tensor
    counts: torch.Tensor
    spos: torch.Tensor
    recv_x: torch.Tensor
    recv_s: torch.Tensor | None
    recv_w: torch.Tensor
    recv_i: torch.Tensor
    route: torch.Tensor


def gpu_plan_dispatch(wl: Workload, inp: dict, src_rank: int = 0, fused: bool = False) -> GpuResult:
    """Plan + dispatch through the C ABI: mep_plan then mep_dispatch, or the
    fused mep_plan_dispatch."""
    T = inp["indices"].shape[0]
    m = M.Mep(wl.hidden, wl.experts_per_rank, wl.topk, wl.cap, wl.ranks, rank=src_rank,
              fp8=wl.quant == "fp8")
    x, w, idx = dev(inp["x"]), dev(inp["weights"]), dev(inp["indices"])
    counts = torch.full((wl.ranks,), SENT32, dtype=torch.int32, device="cuda")
    spos = torch.full((wl.ranks, wl.cap), SENT32, dtype=torch.int32, device="cuda")
    recv_x, recv_s, recv_w, recv_i = alloc_recv(wl)
    if fused:
        M.mep_plan_dispatch(m.h, idx, T, counts, spos, x, w, None, recv_x, recv_s, recv_w, recv_i)
    else:
        M.mep_plan(m.h, idx, T, counts, spos)
        M.mep_dispatch(m.h, x, w, None, idx, recv_x, recv_s, recv_w, recv_i)
    route = torch.full((max(T, 1), wl.topk), SENT32, dtype=torch.int32, device="cuda")
    M.mep_get_route(m.h, route)
    torch.cuda.synchronize()
    return GpuResult(m, x, w, idx, counts, spos, recv_x, recv_s, recv_w, recv_i, route[:T])


def oracle_plan_dispatch(wl: Workload, inp: dict, src_rank: int = 0):
    pl = O.plan(inp["indices"], wl.ranks, wl.experts_per_rank, wl.cap, src_rank)
    d = O.dispatch(inp["x"], inp["weights"], inp["indices"], pl, wl.ranks, wl.experts_per_rank,
                   wl.cap, wl.quant == "fp8")
    return pl, d


def expected_route(wl: Workload, inp: dict, pl: dict) -> np.ndarray:
    r = inp["indices"] // wl.experts_per_rank
    return np.where(pl["slot"] >= 0, r * wl.cap + pl["slot"], -1).astype(np.int32)


def check_plan_dispatch(wl: Workload, inp: dict, g: GpuResult, pl: dict, d: dict) -> None:
    """Bit-exact comparison of counts, src_token_pos, route, and every written
    receive row; unwritten rows must still hold the sentinel."""
    R, cap = wl.ranks, wl.cap
    counts = host(g.counts)
    assert np.array_equal(counts, pl["recv_counts"]), (counts, pl["recv_counts"])
    spos = host(g.spos)
    written = np.zeros((R, cap), bool)
    for r in range(R):
        n = int(counts[r])
        written[r, :n] = True
        assert np.array_equal(spos[r, :n], pl["src_token_pos"][r, :n]), f"src_token_pos rank {r}"
        assert np.all(spos[r, n:] == SENT32), f"stray src_token_pos write on rank {r}"
    assert np.array_equal(host(g.route), expected_route(wl, inp, pl))
    fp8 = wl.quant == "fp8"
    rx = host(g.recv_x, np.uint8 if fp8 else np.uint16)
    assert np.array_equal(rx[written], d["recv_x"][written]), "receive rows differ"
    sent = SENT8 if fp8 else SENT16
    assert np.all(rx[~written] == sent), "stray receive-row write"
    if fp8:
        rs = host(g.recv_s)
        assert np.array_equal(rs[written].view(np.uint32),
                              d["recv_scales"][written].view(np.uint32)), "scales differ"
        assert np.all(np.isnan(rs[~written]))
    rw = host(g.recv_w)
    assert np.array_equal(rw[written].view(np.uint32), d["recv_weights"][written].view(np.uint32))
    assert np.all(np.isnan(rw[~written]))
    ri = host(g.recv_i)
    assert np.array_equal(ri[written], d["recv_indices"][written])
    assert np.all(ri[~written] == SENT32)


def stand_in_gpu(wl: Workload, recv_x: torch.Tensor, recv_s: torch.Tensor | None,
                 mult: float) -> torch.Tensor:
    """Expert stand-in on the GPU (harness): identity for bf16 payloads;
    bf16((decode(q) * scale) * mult) for E4M3 payloads."""
    if recv_s is None:
        return recv_x
    q = recv_x.view(torch.float8_e4m3fn).float()
    s = recv_s.repeat_interleave(128, dim=-1)
    y = (q * s) * mult
    return y.to(torch.bfloat16).view(torch.int16)


def stand_in_mult(wl: Workload) -> float:
    return 0.5 if wl.expert == "dequant_half" else 1.0


def stand_in_oracle(wl: Workload, d_x: np.ndarray, d_s) -> np.ndarray:
    if d_s is None:
        return d_x
    return O.expert_dequant(d_x, d_s, stand_in_mult(wl))


def check_combine(out_gpu_bits: np.ndarray, out_ref_bits: np.ndarray) -> dict:
    diff = bf16_ulp_diff(out_gpu_bits, out_ref_bits)
    assert diff.max(initial=0) <= 1, f"combine differs by {diff.max()} bf16 ulp"
    return {"max_ulp": int(diff.max(initial=0)), "exact_frac": float((diff == 0).mean())
            if diff.size else 1.0}


def run_full(wl: Workload, seed: int, src_rank: int = 0, fused: bool = False) -> dict:
    """Whole path on the GPU and in the oracle; every check; returns stats."""
    inp = make_inputs(wl, seed)
    T = wl.tokens
    g = gpu_plan_dispatch(wl, inp, src_rank, fused)
    pl, d = oracle_plan_dispatch(wl, inp, src_rank)
    check_plan_dispatch(wl, inp, g, pl, d)
    stats = {}
    mult = stand_in_mult(wl)
    if wl.layout == "rank_major":
        y = stand_in_gpu(wl, g.recv_x, g.recv_s, mult)
        out = torch.empty((T, wl.hidden), dtype=torch.int16, device="cuda")
        M.mep_combine(g.m.h, M.MEP_RANK_MAJOR, y, g.w, out)
        ref = O.combine(stand_in_oracle(wl, d["recv_x"], d["recv_scales"]), inp["weights"],
                        inp["indices"], pl, wl.experts_per_rank, wl.cap)
    else:
        cap_em = wl.cap_em
        fp8 = wl.quant == "fp8"
        em_x = torch.full((cap_em, wl.hidden), SENT8 if fp8 else SENT16 - 0x10000,
                          dtype=torch.uint8 if fp8 else torch.int16, device="cuda")
        em_s = (torch.full((cap_em, wl.hidden // 128), float("nan"), device="cuda")
                if fp8 else None)
        em_counts = torch.full((wl.experts,), SENT32, dtype=torch.int32, device="cuda")
        em_offsets = torch.full((wl.experts + 1,), SENT32, dtype=torch.int32, device="cuda")
        em_src = torch.full((cap_em,), SENT32, dtype=torch.int32, device="cuda")
        M.mep_to_expert_major(g.m.h, g.recv_x, g.recv_s, g.recv_i, g.counts, g.spos, em_x, em_s,
                              em_counts, em_offsets, em_src, cap_em)
        em_route = torch.full((max(T, 1), wl.topk), SENT32, dtype=torch.int32, device="cuda")
        M.mep_get_route(g.m.h, g.route, em_route)
        em = O.to_expert_major(d, pl, wl.ranks, wl.experts_per_rank, wl.cap, T, cap_em,
                               src_rank)
        check_expert_major(wl, em, em_x, em_s, em_counts, em_offsets, em_src, em_route[:T])
        y = stand_in_gpu(wl, em_x, em_s, mult)
        out = torch.empty((T, wl.hidden), dtype=torch.int16, device="cuda")
        M.mep_combine(g.m.h, M.MEP_EXPERT_MAJOR, y, g.w, out)
        y_ref = stand_in_oracle(wl, em["em_x"], em["em_scales"])
        ref = O.combine_em(y_ref, inp["weights"], em["tok_em_row"])
    torch.cuda.synchronize()
    stats.update(check_combine(host(out, np.uint16), ref))
    assert M.mep_get_status(g.m.h) == 0
    stats["U"] = int(pl["recv_counts"].sum())
    return stats


def check_expert_major(wl, em, em_x, em_s, em_counts, em_offsets, em_src, em_route):
    assert np.array_equal(host(em_counts), em["em_counts"])
    offs = host(em_offsets)
    assert np.array_equal(offs, em["em_offsets"])
    cap_em = em_x.shape[0]
    used = np.zeros(cap_em, bool)
    for e in range(wl.experts):
        o, n = offs[e], em["em_counts"][e]
        used[o:min(o + n, cap_em)] = True
    fp8 = wl.quant == "fp8"
    ex = host(em_x, np.uint8 if fp8 else np.uint16)
    assert np.array_equal(ex[used], em["em_x"][used]), "expert-major rows differ"
    assert np.all(ex[~used] == (SENT8 if fp8 else SENT16)), "padding rows written"
    if fp8:
        es = host(em_s)
        assert np.array_equal(es[used].view(np.uint32), em["em_scales"][used].view(np.uint32))
    src = host(em_src)
    assert np.array_equal(src[used], em["em_src_pos"][used])
    assert np.all(src[~used] == SENT32)
    assert np.array_equal(host(em_route), em["tok_em_row"])
