"""GPU parity of the conversion of expert-major expert outputs back to the
combine input (mep_convert_combine_input, "MORI-EP User Guide" section 4
convert_combine_input()) and of the combine of the converted rows
(mep_combine with MEP_RANK_SUM), against the CPU oracle on the same inputs.

Reading (oracle R21): a converted row (rank r, slot s) is the fp32 fmaf chain,
in top-k order, of the dispatched weights times the expert-major rows of the
token's experts on rank r (each expert once), rounded once to bf16; the
combine of converted rows adds a token's distinct rank rows in the order of
their first top-k position.

Bar: converted rows bit-exact, every row of the [R, cap, H] output compared
(unwritten rows must keep their sentinel); combine within 1 bf16 ulp (the
kernels mirror the oracle's order, so 0 is expected and asserted where the
case allows).  Also: the status word of a captured iteration across replays
and resets.
"""

import dataclasses

import numpy as np
import pytest
import torch

import combine_mep_plan_amd as M
from oracle import oracle as O
from synthetic import WORKLOADS, Workload, make_inputs

from _gpu_harness import (SENT8, SENT16, SENT32, check_combine, check_expert_major,
                          check_plan_dispatch, dev, gpu_plan_dispatch, host, oracle_plan_dispatch,
                          stand_in_oracle)

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _em_buffers(wl, cap_em):
    fp8 = wl.quant == "fp8"
    H = wl.hidden
    return dict(
        em_x=torch.full((max(cap_em, 1), H), SENT8 if fp8 else SENT16 - 0x10000,
                        dtype=torch.uint8 if fp8 else torch.int16, device="cuda"),
        em_s=(torch.full((max(cap_em, 1), H // 128), float("nan"), device="cuda")
              if fp8 else None),
        em_counts=torch.full((wl.experts,), SENT32, dtype=torch.int32, device="cuda"),
        em_offsets=torch.full((wl.experts + 1,), SENT32, dtype=torch.int32, device="cuda"),
        em_src=torch.full((max(cap_em, 1),), SENT32, dtype=torch.int32, device="cuda"))


def _expert_outputs(wl, em, cap_em, seed, stand_in):
    """bf16 expert outputs in the expert-major layout: the stand-in expert of
    the workload, or random rows everywhere (padding rows too, so that reading
    a row the route does not name would show)."""
    if stand_in:
        return stand_in_oracle(wl, em["em_x"], em["em_scales"])
    rng = np.random.default_rng(7000 + seed)
    v = rng.standard_normal((max(cap_em, 1), wl.hidden)).astype(np.float32)
    return torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def run_convert(wl, inp, seed=0, src_rank=0, cap_em=None, stand_in=False, expect_status=0):
    """Fused plan+dispatch, expert-major conversion, the conversion back and
    the combine of converted rows on the GPU; the same in the oracle; every
    comparison.  Returns the combine statistics."""
    T, H, R, epr, cap = inp["indices"].shape[0], wl.hidden, wl.ranks, wl.experts_per_rank, wl.cap
    cap_em = wl.cap_em if cap_em is None else cap_em
    g = gpu_plan_dispatch(wl, inp, src_rank, fused=True)
    pl, d = oracle_plan_dispatch(wl, inp, src_rank)
    check_plan_dispatch(wl, inp, g, pl, d)
    b = _em_buffers(wl, cap_em)
    M.mep_to_expert_major(g.m.h, g.recv_x, g.recv_s, g.recv_i, g.counts, g.spos, b["em_x"],
                          b["em_s"], b["em_counts"], b["em_offsets"], b["em_src"], cap_em)
    em_route = torch.full((max(T, 1), wl.topk), SENT32, dtype=torch.int32, device="cuda")
    M.mep_get_route(g.m.h, g.route if T else None, em_route)
    em = O.to_expert_major(d, pl, R, epr, cap, T, cap_em, src_rank)
    if cap_em > 0:
        check_expert_major(wl, em, b["em_x"][:cap_em], b["em_s"][:cap_em] if b["em_s"] is not None
                           else None, b["em_counts"], b["em_offsets"], b["em_src"][:cap_em],
                           em_route[:T])
    y_ref = _expert_outputs(wl, em, cap_em, seed, stand_in)
    y = dev(y_ref)
    conv = torch.full((R, cap, H), SENT16 - 0x10000, dtype=torch.int16, device="cuda")
    M.mep_convert_combine_input(g.m.h, y, g.recv_w, conv)
    out = torch.full((max(T, 1), H), SENT16 - 0x10000, dtype=torch.int16, device="cuda")
    M.mep_combine(g.m.h, M.MEP_RANK_SUM, conv, None, out)
    torch.cuda.synchronize()
    ref_conv = O.convert_combine_input(y_ref[:cap_em] if cap_em else y_ref[:0], em, d, pl, R,
                                       epr, cap, fill=SENT16)
    got = host(conv, np.uint16)
    bad = np.argwhere(np.any(got != ref_conv, axis=-1))
    assert bad.size == 0, f"converted rows differ at (rank, slot) {bad[:5].tolist()}"
    ref_out = O.combine_rank_sum(ref_conv, inp["indices"], pl, epr, cap)
    stats = check_combine(host(out, np.uint16)[:T], ref_out)
    assert M.mep_get_status(g.m.h) == (pl["status"] | em["status"]) == expect_status
    stats["U"] = int(pl["recv_counts"].sum())
    return stats


def _wl(name, **kw):
    return dataclasses.replace(WORKLOADS[name], **kw)


def test_convert_full_size_stdmoe():
    # the standard-MoE workload at full size: 4096 tokens, 32 ranks x 8
    # experts, FP8 dispatch, the dequantising expert stand-in
    wl = WORKLOADS["stdmoe"]
    inp = make_inputs(wl, 0)
    st = run_convert(wl, inp, seed=0, stand_in=True)
    _say(f"stdmoe full size: U={st['U']} max_ulp={st['max_ulp']} exact={st['exact_frac']:.4f}")
    assert st["max_ulp"] == 0


@pytest.mark.parametrize("T,R,epr,k,src,quant", [
    (300, 8, 4, 6, 2, "none"),      # ragged, several experts per rank row
    (1, 8, 4, 6, 0, "none"),
    (65, 4, 8, 8, 1, "fp8"),
    (257, 16, 16, 8, 3, "none"),
    (1000, 2, 32, 8, 1, "fp8"),     # two ranks: rows merge up to 8 experts
    (700, 32, 8, 8, 0, "fp8"),
])
def test_convert_ragged(T, R, epr, k, src, quant):
    wl = Workload("cv", T, 512, R, epr, k, max(T, 64), quant, "uniform", "identity",
                  "expert_major")
    inp = make_inputs(wl, T + R)
    st = run_convert(wl, inp, seed=T, src_rank=src)
    _say(f"T={T} R={R} epr={epr} k={k}: U={st['U']} max_ulp={st['max_ulp']}")
    assert st["max_ulp"] == 0


@pytest.mark.parametrize("k,R,epr", [(12, 4, 8), (32, 8, 8), (9, 2, 16)])
def test_convert_wide_top_k(k, R, epr):
    wl = Workload("cvw", 200, 256, R, epr, k, 256, "none", "uniform", "identity", "expert_major")
    inp = make_inputs(wl, k)
    st = run_convert(wl, inp, seed=k)
    assert st["max_ulp"] == 0


def test_convert_empty_batch():
    wl = Workload("cv0", 0, 256, 4, 4, 4, 64, "none", "uniform", "identity", "expert_major")
    inp = {"x": np.zeros((0, 256), np.uint16), "indices": np.zeros((0, 4), np.int32),
           "weights": np.zeros((0, 4), np.float32)}
    run_convert(wl, inp)


def test_convert_bad_and_repeated_ids():
    # a token with an id out of range is not dispatched (its converted rows do
    # not exist and it combines to +0); a token naming one expert twice has
    # one expert-major row, counted once
    wl = Workload("cvb", 130, 256, 8, 4, 6, 130, "none", "uniform", "identity", "expert_major")
    inp = make_inputs(wl, 9)
    idx = inp["indices"].copy()
    idx[5, 2] = 32 + 7          # out of range
    idx[40, 4] = -1
    idx[7, 3] = idx[7, 1]       # repeated expert
    idx[90, 5] = idx[90, 0]
    inp = dict(inp, indices=idx)
    run_convert(wl, inp, seed=9, expect_status=M.MEP_DEV_BAD_INDEX | M.MEP_DEV_DUP_EXPERT)


def test_convert_after_expert_major_overflow():
    # rows dropped past cap_em add nothing to their converted rows
    wl = Workload("cvo", 256, 256, 4, 4, 6, 256, "none", "uniform", "identity", "expert_major")
    inp = make_inputs(wl, 11)
    run_convert(wl, inp, seed=11, cap_em=1000, expect_status=M.MEP_DEV_EM_OVERFLOW)


def test_convert_state_rules():
    wl = Workload("cvs", 64, 256, 4, 4, 4, 64, "none", "uniform", "identity", "expert_major")
    inp = make_inputs(wl, 3)
    g = gpu_plan_dispatch(wl, inp, fused=True)
    y = torch.zeros((wl.cap_em, wl.hidden), dtype=torch.int16, device="cuda")
    conv = torch.zeros((wl.ranks, wl.cap, wl.hidden), dtype=torch.int16, device="cuda")
    # no expert-major layout after this plan yet
    with pytest.raises(M.MepError):
        M.mep_convert_combine_input(g.m.h, y, g.recv_w, conv)
    # after the standard-MoE dispatch there is no rank-major plan
    b = _em_buffers(wl, wl.cap_em)
    M.mep_dispatch_standard_moe(g.m.h, g.idx, wl.tokens, g.x, None, b["em_x"], b["em_s"],
                                b["em_counts"], b["em_offsets"], b["em_src"], wl.cap_em)
    with pytest.raises(M.MepError):
        M.mep_convert_combine_input(g.m.h, y, g.recv_w, conv)
    with pytest.raises(M.MepError):
        M.mep_combine(g.m.h, M.MEP_RANK_SUM, conv, None,
                      torch.zeros((wl.tokens, wl.hidden), dtype=torch.int16, device="cuda"))
    torch.cuda.synchronize()


def test_hip_graph_convert_replay():
    # plan+dispatch, the expert-major conversion, the conversion back and the
    # combine of converted rows captured once, replayed with new routing, rows
    # and expert outputs written in place between replays
    wl = Workload("cvg", 500, 512, 8, 4, 6, 512, "fp8", "uniform", "dequant", "expert_major")
    T, H, R, epr, cap, cap_em = wl.tokens, wl.hidden, wl.ranks, wl.experts_per_rank, wl.cap, \
        wl.cap_em
    inp = make_inputs(wl, 40)
    g = gpu_plan_dispatch(wl, inp, fused=True)
    b = _em_buffers(wl, cap_em)
    y = torch.zeros((cap_em, H), dtype=torch.int16, device="cuda")
    conv = torch.zeros((R, cap, H), dtype=torch.int16, device="cuda")
    out = torch.zeros((T, H), dtype=torch.int16, device="cuda")
    M.mep_to_expert_major(g.m.h, g.recv_x, g.recv_s, g.recv_i, g.counts, g.spos, b["em_x"],
                          b["em_s"], b["em_counts"], b["em_offsets"], b["em_src"], cap_em)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        M.mep_plan_dispatch(g.m.h, g.idx, T, g.counts, g.spos, g.x, g.w, None, g.recv_x, g.recv_s,
                            g.recv_w, g.recv_i)
        M.mep_to_expert_major(g.m.h, g.recv_x, g.recv_s, g.recv_i, g.counts, g.spos, b["em_x"],
                              b["em_s"], b["em_counts"], b["em_offsets"], b["em_src"], cap_em)
        M.mep_convert_combine_input(g.m.h, y, g.recv_w, conv)
        M.mep_combine(g.m.h, M.MEP_RANK_SUM, conv, None, out)
    for rep in range(3):
        new = make_inputs(wl, 600 + rep)
        g.x.copy_(dev(new["x"]))
        g.idx.copy_(dev(new["indices"]))
        g.w.copy_(dev(new["weights"]))
        pl, d = oracle_plan_dispatch(wl, new)
        em = O.to_expert_major(d, pl, R, epr, cap, T, cap_em, 0)
        y_ref = _expert_outputs(wl, em, cap_em, rep, stand_in=False)
        y.copy_(dev(y_ref))
        conv.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _say(f"convert replay {rep}")
        ref_conv = O.convert_combine_input(y_ref, em, d, pl, R, epr, cap, fill=0)
        assert np.array_equal(host(conv, np.uint16), ref_conv), rep
        check_combine(host(out, np.uint16),
                      O.combine_rank_sum(ref_conv, new["indices"], pl, epr, cap))
    assert M.mep_get_status(g.m.h) == 0


def test_hip_graph_status_across_replays_and_resets():
    # A captured iteration reports the bits of its latest replay: each replay
    # starts from a clear word, mep_reset between replays changes nothing, and
    # a plan outside capture returns to the per-reset-epoch words.
    wl = Workload("gst", 64, 256, 4, 4, 4, 64, "none", "uniform", "identity", "rank_major")
    T, H = wl.tokens, wl.hidden
    inp = make_inputs(wl, 12)
    good = inp["indices"].copy()
    bad = good.copy()
    bad[3, 1] = 99                      # out of range
    dup = good.copy()
    dup[9, 2] = dup[9, 0]               # a repeated expert
    g = gpu_plan_dispatch(wl, inp, fused=True)
    M.mep_reset(g.m.h)
    out = torch.zeros((T, H), dtype=torch.int16, device="cuda")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        M.mep_plan_dispatch(g.m.h, g.idx, T, g.counts, g.spos, g.x, g.w, None, g.recv_x, None,
                            g.recv_w, g.recv_i)
        M.mep_combine(g.m.h, M.MEP_RANK_MAJOR, g.recv_x, g.w, out)

    def replay(ids, reset_after):
        g.idx.copy_(dev(ids))
        torch.cuda.synchronize()
        graph.replay()
        st = M.mep_get_status(g.m.h)
        if reset_after:
            M.mep_reset(g.m.h)
        return st

    D, B = M.MEP_DEV_DUP_EXPERT, M.MEP_DEV_BAD_INDEX
    assert replay(good, True) == 0
    assert replay(bad, True) == B
    assert M.mep_get_status(g.m.h) == B       # a reset changes nothing for the graph's word
    assert replay(good, False) == 0           # the next replay starts clean
    assert replay(dup, False) == D
    assert replay(bad, True) == B             # not sticky across replays
    assert replay(good, True) == 0
    # the replayed combine still matches the oracle for the last routing
    pl, d = oracle_plan_dispatch(wl, inp)
    check_combine(host(out, np.uint16),
                  O.combine(d["recv_x"], inp["weights"], good, pl, wl.experts_per_rank, wl.cap))
    # outside capture again: the epoch words, sticky until mep_reset
    M.mep_plan(g.m.h, dev(bad), T, g.counts, g.spos)
    assert M.mep_get_status(g.m.h) == B
    M.mep_plan(g.m.h, dev(good), T, g.counts, g.spos)
    assert M.mep_get_status(g.m.h) == B
    M.mep_reset(g.m.h)
    assert M.mep_get_status(g.m.h) == 0
    M.mep_plan(g.m.h, dev(good), T, g.counts, g.spos)
    assert M.mep_get_status(g.m.h) == 0


def test_hip_graph_expert_major_overflow_per_replay():
    # plan+dispatch and the expert-major conversion captured with a small
    # cap_em: routing every token to experts 0 and 1 fits (rows 0..191),
    # routing spread over all 8 experts needs segments starting at row 256 and
    # overflows; each replay reports its own overflow bit
    wl = Workload("gov", 64, 256, 2, 4, 2, 64, "none", "uniform", "identity", "expert_major")
    T, H, cap_em = wl.tokens, wl.hidden, 200
    inp = make_inputs(wl, 13)
    compact = np.tile(np.array([[0, 1]], np.int32), (T, 1))
    spread = np.stack([np.array([t % 8, (t + 3) % 8]) for t in range(T)]).astype(np.int32)
    inp = dict(inp, indices=compact)
    g = gpu_plan_dispatch(wl, inp, fused=True)
    b = _em_buffers(wl, cap_em)
    M.mep_reset(g.m.h)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        M.mep_plan_dispatch(g.m.h, g.idx, T, g.counts, g.spos, g.x, g.w, None, g.recv_x, None,
                            g.recv_w, g.recv_i)
        M.mep_to_expert_major(g.m.h, g.recv_x, None, g.recv_i, g.counts, g.spos, b["em_x"],
                              None, b["em_counts"], b["em_offsets"], b["em_src"], cap_em)
    for ids, want in ((compact, 0), (spread, M.MEP_DEV_EM_OVERFLOW), (compact, 0),
                      (spread, M.MEP_DEV_EM_OVERFLOW), (spread, M.MEP_DEV_EM_OVERFLOW),
                      (compact, 0)):
        g.idx.copy_(dev(ids))
        torch.cuda.synchronize()
        graph.replay()
        assert M.mep_get_status(g.m.h) == want
        M.mep_reset(g.m.h)
    # the last replay's layout matches the oracle
    pl, d = oracle_plan_dispatch(wl, dict(inp, indices=compact))
    em = O.to_expert_major(d, pl, wl.ranks, wl.experts_per_rank, wl.cap, T, cap_em, 0)
    assert np.array_equal(host(b["em_counts"]), em["em_counts"])
    assert np.array_equal(host(b["em_offsets"]), em["em_offsets"])
