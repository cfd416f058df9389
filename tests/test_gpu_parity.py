"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.

Bar: bit-exact for counts, src_token_pos, receive rows, route, E4M3 codes,
scales, weights, ids and the expert-major layout; combine within 1 bf16 ulp
(the kernels mirror the oracle's fused multiply-add order, so 0 is expected
and the exact fraction is printed).

Sources: "MORI-EP User Guide" section 3 (dispatch, combine, reset,
get_dispatch_src_token_pos), section 4 (standard-MoE layout), section 7
(identity expert); "Choosing an EP API and backend" (OCP E4M3 on gfx950).
"""

import dataclasses

import numpy as np
import pytest
import torch

import combine_mep_plan_amd as M
from oracle import oracle as O
from synthetic import WORKLOADS, Workload, make_inputs

from _gpu_harness import (SENT8, SENT32, GpuResult, alloc_recv, bf16_ulp_diff, check_combine,
                          check_expert_major, check_plan_dispatch, dev, gpu_plan_dispatch, host,
                          oracle_plan_dispatch, run_full, stand_in_oracle)

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


# ---------------------------------------------------------------------------
# device conversions
# ---------------------------------------------------------------------------

def test_probe_e4m3_matches_oracle():
    tab = O.e4m3_decode_table()[:0x7F]
    vals = [tab[c] for c in range(0x7F)] + [0.5 * (tab[c - 1] + tab[c]) for c in range(1, 0x7F)]
    b = np.array(vals, np.float32).view(np.uint32)
    near = np.concatenate([b, b + 1, b + 2, np.maximum(b, 1) - 1]).view(np.float32)
    top = int(np.float32(448.0).view(np.uint32)) + 2  # quotients reach 448 * (1 + 2^-23)
    sweep = np.arange(0, top + 1, 61, dtype=np.uint32).view(np.float32)
    extra = np.float32([448.0, np.nextafter(np.float32(448), np.float32(1e9)), 0.0, 2.0 ** -10,
                        2.0 ** -11, 1e-30, 1e-45])
    v = np.concatenate([near, sweep, extra])
    v = np.concatenate([v, -v]).astype(np.float32)
    v = np.ascontiguousarray(v[np.abs(v) <= np.float32(448.0) * np.float32(1 + 2 ** -23)])
    out = torch.empty(v.size, dtype=torch.uint8, device="cuda")
    M.mep_probe_e4m3(dev(v), out, v.size)
    got = host(out)
    ref = O.e4m3_encode(v)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(v[i]), hex(got[i]), hex(ref[i])) for i in bad[:10]]


def test_probe_bf16_matches_oracle():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2**32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[np.isfinite(v)]
    ties = ((rng.integers(0, 2**16, size=200_000).astype(np.uint32) << 16) | 0x8000) \
        .view(np.float32)
    ties = ties[np.isfinite(ties)]
    den = rng.integers(1, 2**23, size=200_000).astype(np.uint32).view(np.float32)
    v = np.ascontiguousarray(np.concatenate([v, ties, den, -den]).astype(np.float32))
    out = torch.empty(v.size, dtype=torch.int16, device="cuda")
    M.mep_probe_bf16(dev(v), out, v.size)
    got = host(out, np.uint16)
    ref = O.bf16_rne(v)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(v[i]), hex(got[i]), hex(ref[i])) for i in bad[:10]]


# ---------------------------------------------------------------------------
# whole path, reduced and full sizes
# ---------------------------------------------------------------------------

def _variant(name, **kw):
    return dataclasses.replace(WORKLOADS[name], **kw)


SMALL = [
    ("tiny", WORKLOADS["tiny"], (0, 1, 2)),
    ("tiny_T5", _variant("tiny", tokens=5), (3,)),
    ("decode_T77", _variant("decode", tokens=77), (0,)),
    ("decode", WORKLOADS["decode"], (1,)),
    ("prefill_T300", _variant("prefill", tokens=300, cap=512), (0, 1)),
    ("skew_T300", _variant("skew", tokens=300, cap=300), (0,)),
    ("stdmoe_T300", _variant("stdmoe", tokens=300, cap=320), (0,)),
    # ragged rows: 1152 = 9 x 128 columns leaves a partial lane sweep per row
    ("odd_bf16", Workload("odd_bf16", 131, 1152, 5, 3, 3, 140, "none", "uniform", "identity",
                          "rank_major"), (0,)),
    ("odd_fp8", Workload("odd_fp8", 131, 1152, 5, 3, 3, 140, "fp8", "uniform", "dequant_half",
                         "rank_major"), (0,)),
    ("odd_em", Workload("odd_em", 97, 1152, 3, 5, 4, 100, "fp8", "uniform", "dequant",
                        "expert_major"), (0,)),
    ("em_bf16", Workload("em_bf16", 150, 256, 4, 4, 3, 150, "none", "uniform", "identity",
                         "expert_major"), (0,)),
    # top-k above 8 takes the wide combine variant
    ("top12", Workload("top12", 70, 512, 6, 4, 12, 70, "none", "uniform", "identity",
                       "rank_major"), (0,)),
    ("one_rank", Workload("one_rank", 64, 256, 1, 16, 4, 64, "none", "uniform", "identity",
                          "rank_major"), (0,)),
    ("wide64", Workload("wide64", 100, 256, 64, 2, 8, 100, "fp8", "uniform", "dequant_half",
                        "rank_major"), (0,)),
    # top-k up to the maximum of 32, FP8 and expert-major with the wide variants
    ("top20_fp8", Workload("top20_fp8", 300, 512, 16, 4, 20, 300, "fp8", "uniform",
                           "dequant_half", "rank_major"), (0,)),
    ("top32_em", Workload("top32_em", 200, 256, 8, 8, 32, 200, "fp8", "uniform", "dequant",
                          "expert_major"), (0,)),
    # the largest configuration: 64 ranks x 64 experts, top-32
    ("max_cfg", Workload("max_cfg", 300, 256, 64, 64, 32, 300, "fp8", "uniform", "dequant",
                         "expert_major"), (0,)),
    # the narrowest rows: one 16-byte unit of bf16, one FP8 scale block
    ("h8_bf16", Workload("h8_bf16", 200, 8, 4, 4, 4, 200, "none", "uniform", "identity",
                         "rank_major"), (0,)),
    ("h128_fp8", Workload("h128_fp8", 200, 128, 4, 4, 4, 200, "fp8", "uniform", "dequant_half",
                          "expert_major"), (0,)),
]


MODES = [False, True]  # mep_plan + mep_dispatch, or the fused mep_plan_dispatch


@pytest.mark.parametrize("fused", MODES, ids=["separate", "fused"])
@pytest.mark.parametrize("label,wl,seeds", SMALL, ids=[s[0] for s in SMALL])
def test_parity_small(label, wl, seeds, fused):
    for seed in seeds:
        _say(f"[parity-small] {label} fused={fused} seed={seed} T={wl.tokens} H={wl.hidden} "
             f"R={wl.ranks}")
        st = run_full(wl, seed, src_rank=seed % wl.ranks, fused=fused)
        _say(f"    U={st['U']} max_ulp={st['max_ulp']} exact={st['exact_frac']:.6f}")


@pytest.mark.parametrize("fused", MODES, ids=["separate", "fused"])
@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "skew", "stdmoe"])
def test_parity_full_size(name, fused):
    wl = WORKLOADS[name]
    _say(f"[parity-full] {name} fused={fused} T={wl.tokens} H={wl.hidden} R={wl.ranks} "
         f"k={wl.topk}")
    st = run_full(wl, 0, fused=fused)
    _say(f"    U={st['U']} max_ulp={st['max_ulp']} exact={st['exact_frac']:.6f}")


# ---------------------------------------------------------------------------
# edge cases and lifecycle
# ---------------------------------------------------------------------------

def test_empty_batch():
    wl = _variant("tiny", tokens=0)
    inp = {"x": np.zeros((0, wl.hidden), np.uint16), "indices": np.zeros((0, wl.topk), np.int32),
           "weights": np.zeros((0, wl.topk), np.float32)}
    m = M.Mep(wl.hidden, wl.experts_per_rank, wl.topk, wl.cap, wl.ranks)
    counts = torch.full((wl.ranks,), 7, dtype=torch.int32, device="cuda")
    spos = torch.full((wl.ranks, wl.cap), SENT32, dtype=torch.int32, device="cuda")
    M.mep_plan(m.h, None, 0, counts, spos)
    out = torch.empty((1, wl.hidden), dtype=torch.int16, device="cuda")
    rx = torch.zeros((wl.ranks, wl.cap, wl.hidden), dtype=torch.int16, device="cuda")
    rw = torch.zeros((wl.ranks, wl.cap, wl.topk), dtype=torch.float32, device="cuda")
    ri = torch.zeros((wl.ranks, wl.cap, wl.topk), dtype=torch.int32, device="cuda")
    M.mep_dispatch(m.h, None, None, None, None, rx, None, rw, ri)
    M.mep_combine(m.h, M.MEP_RANK_MAJOR, None, None, out)
    torch.cuda.synchronize()
    assert np.all(host(counts) == 0)
    assert np.all(host(spos) == SENT32)
    assert M.mep_get_status(m.h) == 0
    del inp


def test_full_capacity_and_single_rank_hotspot():
    # T == cap and every token on rank 0: rank 0 receives cap rows
    wl = Workload("hot", 256, 512, 4, 4, 4, 256, "fp8", "uniform", "dequant_half", "rank_major")
    inp = make_inputs(wl, 0)
    rng = np.random.default_rng(9)
    inp["indices"] = np.stack([rng.permutation(4)[:4] for _ in range(256)]).astype(np.int32)
    g = gpu_plan_dispatch(wl, inp)
    pl, d = oracle_plan_dispatch(wl, inp)
    check_plan_dispatch(wl, inp, g, pl, d)
    assert host(g.counts)[0] == 256


@pytest.mark.parametrize("T", [16, 700])
@pytest.mark.parametrize("fused", MODES, ids=["separate", "fused"])
def test_bad_and_duplicate_expert_ids(fused, T):
    wl = _variant("tiny", tokens=T, cap=1024)
    inp = make_inputs(wl, 5)
    idx = inp["indices"].copy()
    idx[3] = [1, 99]      # out of range -> token 3 not dispatched
    idx[7] = [-4, 2]      # negative -> token 7 not dispatched
    idx[9] = [5, 5]       # repeated expert -> still routed, status bit
    inp["indices"] = idx
    g = gpu_plan_dispatch(wl, inp, fused=fused)
    pl, d = oracle_plan_dispatch(wl, inp)
    assert pl["status"] == M.MEP_DEV_BAD_INDEX | M.MEP_DEV_DUP_EXPERT
    check_plan_dispatch(wl, inp, g, pl, d)
    out = torch.empty((wl.tokens, wl.hidden), dtype=torch.int16, device="cuda")
    M.mep_combine(g.m.h, M.MEP_RANK_MAJOR, g.recv_x, g.w, out)
    ref = O.combine(d["recv_x"], inp["weights"], idx, pl, wl.experts_per_rank, wl.cap)
    check_combine(host(out, np.uint16), ref)
    assert np.all(host(out, np.uint16)[[3, 7]] == 0)
    assert M.mep_get_status(g.m.h) == M.MEP_DEV_BAD_INDEX | M.MEP_DEV_DUP_EXPERT
    M.mep_reset(g.m.h)
    assert M.mep_get_status(g.m.h) == 0


def test_reset_invalidates_plan():
    wl = WORKLOADS["tiny"]
    inp = make_inputs(wl, 1)
    g = gpu_plan_dispatch(wl, inp)
    counts = host(g.counts).copy()
    M.mep_reset(g.m.h)
    torch.cuda.synchronize()
    assert np.array_equal(host(g.counts), counts)  # caller buffers untouched
    with pytest.raises(M.MepError) as ei:
        M.mep_dispatch(g.m.h, g.x, g.w, None, g.idx, g.recv_x, None, g.recv_w, g.recv_i)
    assert ei.value.code == M.MEP_ERR_STATE
    with pytest.raises(M.MepError):
        M.mep_combine(g.m.h, M.MEP_RANK_MAJOR, g.recv_x, g.w, g.recv_x)


def test_routing_replay_and_determinism():
    # one plan serves several dispatch/combine rounds with new token rows; repeated
    # runs give identical bits
    wl = _variant("prefill", tokens=200, cap=256)
    inp = make_inputs(wl, 2)
    g = gpu_plan_dispatch(wl, inp)
    pl = O.plan(inp["indices"], wl.ranks, wl.experts_per_rank, wl.cap)
    rng = np.random.default_rng(4)
    for round_ in range(3):
        x2 = torch.from_numpy(rng.standard_normal((wl.tokens, wl.hidden), dtype=np.float32)) \
            .to(torch.bfloat16).view(torch.int16)
        x2_np = x2.numpy().view(np.uint16)
        M.mep_dispatch(g.m.h, x2.cuda(), g.w, None, g.idx, g.recv_x, g.recv_s, g.recv_w, g.recv_i)
        d = O.dispatch(x2_np, inp["weights"], inp["indices"], pl, wl.ranks, wl.experts_per_rank,
                       wl.cap, True)
        inp2 = dict(inp, x=x2_np)
        check_plan_dispatch(wl, inp2, g, pl, d)
    first = host(g.recv_x).copy()
    M.mep_dispatch(g.m.h, x2.cuda(), g.w, None, g.idx, g.recv_x, g.recv_s, g.recv_w, g.recv_i)
    assert np.array_equal(first, host(g.recv_x))


def test_combine_random_expert_rows():
    # non-identity expert rows (random per receive row) pin the gather indices
    for wl in (_variant("decode", tokens=100, cap=128), _variant("skew", tokens=150, cap=160)):
        inp = make_inputs(wl, 8)
        g = gpu_plan_dispatch(wl, inp)
        pl = O.plan(inp["indices"], wl.ranks, wl.experts_per_rank, wl.cap)
        rng = np.random.default_rng(10)
        y = torch.from_numpy(rng.standard_normal((wl.ranks, wl.cap, wl.hidden), dtype=np.float32))
        y = y.to(torch.bfloat16).view(torch.int16)
        w = rng.uniform(-1, 1, size=inp["weights"].shape).astype(np.float32)
        out = torch.empty((wl.tokens, wl.hidden), dtype=torch.int16, device="cuda")
        M.mep_combine(g.m.h, M.MEP_RANK_MAJOR, y.cuda(), dev(w), out)
        ref = O.combine(y.numpy().view(np.uint16), w, inp["indices"], pl, wl.experts_per_rank,
                        wl.cap)
        st = check_combine(host(out, np.uint16), ref)
        _say(f"    random rows {wl.name}: max_ulp={st['max_ulp']} exact={st['exact_frac']:.6f}")


def test_expert_major_overflow_sets_status():
    wl = _variant("stdmoe", tokens=64, cap=64)
    inp = make_inputs(wl, 0)
    g = gpu_plan_dispatch(wl, inp)
    cap_em = 700  # 64*8 rows need far more than 700 once each expert is padded to 128
    em_x = torch.zeros((cap_em, wl.hidden), dtype=torch.uint8, device="cuda")
    em_s = torch.zeros((cap_em, wl.hidden // 128), dtype=torch.float32, device="cuda")
    em_c = torch.zeros(wl.experts, dtype=torch.int32, device="cuda")
    em_o = torch.zeros(wl.experts + 1, dtype=torch.int32, device="cuda")
    em_p = torch.full((cap_em,), SENT32, dtype=torch.int32, device="cuda")
    M.mep_to_expert_major(g.m.h, g.recv_x, g.recv_s, g.recv_i, g.counts, g.spos, em_x, em_s, em_c,
                          em_o, em_p, cap_em)
    assert M.mep_get_status(g.m.h) == M.MEP_DEV_EM_OVERFLOW
    pl, d = oracle_plan_dispatch(wl, inp)
    em = O.to_expert_major(d, pl, wl.ranks, wl.experts_per_rank, wl.cap, wl.tokens, cap_em)
    assert em["status"] == O.ST_EM_OVERFLOW
    assert np.array_equal(host(em_c), em["em_counts"])
    assert np.array_equal(host(em_p), np.where(em["em_src_pos"] >= 0, em["em_src_pos"], SENT32))


@pytest.mark.parametrize("fused", MODES, ids=["separate", "fused"])
@pytest.mark.parametrize("T", [1, 63, 64, 65, 255, 256, 257, 1023, 1024, 1025, 2049, 3000])
def test_plan_block_boundaries(T, fused):
    # mep_plan: one workgroup up to 1024 tokens, else count + slot launches split
    # into count blocks of 4 chunks (256 tokens; 16 chunks above 4096 tokens);
    # fused: one launch up to 256 tokens, else count + dispatch launches
    wl = _variant("skew", tokens=T, cap=3072, hidden=256)
    inp = make_inputs(wl, T)
    g = gpu_plan_dispatch(wl, inp, src_rank=3, fused=fused)
    pl, d = oracle_plan_dispatch(wl, inp, src_rank=3)
    check_plan_dispatch(wl, inp, g, pl, d)


def test_status_is_sticky_until_reset():
    wl = _variant("tiny", tokens=8)
    inp = make_inputs(wl, 0)
    bad = dict(inp, indices=inp["indices"].copy())
    bad["indices"][2] = [0, 50]
    g = gpu_plan_dispatch(wl, bad)
    assert M.mep_get_status(g.m.h) == M.MEP_DEV_BAD_INDEX
    # a second plan with clean ids in the same epoch keeps the bit
    M.mep_plan(g.m.h, g.idx.copy_(dev(inp["indices"])), wl.tokens, g.counts, g.spos)
    assert M.mep_get_status(g.m.h) == M.MEP_DEV_BAD_INDEX
    M.mep_reset(g.m.h)
    assert M.mep_get_status(g.m.h) == 0
    M.mep_reset(g.m.h)  # reset without a plan in between
    assert M.mep_get_status(g.m.h) == 0
    M.mep_plan(g.m.h, dev(bad["indices"]), wl.tokens, g.counts, g.spos)
    assert M.mep_get_status(g.m.h) == M.MEP_DEV_BAD_INDEX
    M.mep_reset(g.m.h)
    M.mep_plan(g.m.h, g.idx, wl.tokens, g.counts, g.spos)
    assert M.mep_get_status(g.m.h) == 0


@pytest.mark.parametrize("T", [4096, 4160])
def test_fused_plan_dispatch_64_ranks(T):
    # 64 ranks (the widest rank mask) over 64 and 65 count chunks
    wl = Workload("wide", T, 256, 64, 2, 8, T, "fp8", "uniform", "dequant_half", "rank_major")
    inp = make_inputs(wl, 1)
    g = gpu_plan_dispatch(wl, inp, src_rank=5, fused=True)
    pl, d = oracle_plan_dispatch(wl, inp, src_rank=5)
    check_plan_dispatch(wl, inp, g, pl, d)
    assert M.mep_get_status(g.m.h) == 0


@pytest.mark.parametrize("T,R", [(4097, 8), (5200, 8), (9000, 8), (8193, 33), (20000, 8)])
def test_fused_plan_dispatch_long_batches(T, R):
    # past 4096 tokens the count blocks hold 16 chunks instead of 4 (4097: the
    # first such batch); past 16384 tokens a token's chunk has more than the
    # 16 earlier block totals a dispatch wave loads with its mask, and sums
    # the rest after (20000 tokens: up to 19 earlier blocks)
    wl = Workload("long", T, 256, R, 4, 8, T, "fp8", "uniform", "dequant_half", "rank_major")
    inp = make_inputs(wl, 2)
    for fused in (True, False):
        g = gpu_plan_dispatch(wl, inp, src_rank=1, fused=fused)
        pl, d = oracle_plan_dispatch(wl, inp, src_rank=1)
        check_plan_dispatch(wl, inp, g, pl, d)
        assert M.mep_get_status(g.m.h) == 0


@pytest.mark.parametrize("R", [1, 3, 8, 12, 16])
def test_fused_plan_dispatch_repeated(R):
    # one handle, successive fused calls with fresh routing each time, over
    # batch sizes that take the two-launch path (above 256 tokens) and the
    # one-launch path (100 tokens) in turn: every call must match the oracle
    # whatever the call before it left in the workspace
    cap = 4096
    wl0 = Workload("lb", cap, 256, R, 8, 8, cap, "fp8", "uniform", "dequant_half", "rank_major")
    src = min(2, R - 1)
    m = M.Mep(wl0.hidden, wl0.experts_per_rank, wl0.topk, cap, R, rank=src, fp8=True)
    for i, T in enumerate([cap, 257, 1000, 100, cap - 1, 64 * 5 + 3, cap]):
        wl = dataclasses.replace(wl0, tokens=T)
        inp = make_inputs(wl, 300 + i)
        x, w, idx = dev(inp["x"]), dev(inp["weights"]), dev(inp["indices"])
        counts = torch.full((R,), SENT32, dtype=torch.int32, device="cuda")
        spos = torch.full((R, cap), SENT32, dtype=torch.int32, device="cuda")
        recv = alloc_recv(wl)
        M.mep_plan_dispatch(m.h, idx, T, counts, spos, x, w, None, *recv)
        route = torch.full((T, wl.topk), SENT32, dtype=torch.int32, device="cuda")
        M.mep_get_route(m.h, route)
        torch.cuda.synchronize()
        g = GpuResult(m, x, w, idx, counts, spos, *recv, route)
        pl, d = oracle_plan_dispatch(wl, inp, src_rank=src)
        _say(f"R={R} call {i} T={T}")
        check_plan_dispatch(wl, inp, g, pl, d)
        assert M.mep_get_status(m.h) == 0
        M.mep_reset(m.h)


@pytest.mark.parametrize("T", [128, 700])
def test_hip_graph_capture_replay(T):
    # plan+dispatch and combine captured once in a HIP graph, replayed with new
    # token rows and routing written in place between replays (with eager work
    # and synchronisation in between); every replay must match the oracle
    wl = _variant("prefill", tokens=T, cap=1024, hidden=1024)
    R, epr, k, cap, H = wl.ranks, wl.experts_per_rank, wl.topk, wl.cap, wl.hidden
    inp = make_inputs(wl, 100)
    g = gpu_plan_dispatch(wl, inp, fused=True)  # eager warm-up, allocates everything
    y = torch.zeros((R, cap, H), dtype=torch.int16, device="cuda")
    out = torch.zeros((T, H), dtype=torch.int16, device="cuda")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        M.mep_plan_dispatch(g.m.h, g.idx, T, g.counts, g.spos, g.x, g.w, None, g.recv_x, g.recv_s,
                            g.recv_w, g.recv_i)
        M.mep_combine(g.m.h, M.MEP_RANK_MAJOR, y, g.w, out)
    for rep in range(4):
        new = make_inputs(wl, 200 + rep)
        g.x.copy_(dev(new["x"]))
        g.idx.copy_(dev(new["indices"]))
        g.w.copy_(dev(new["weights"]))
        pl, d = oracle_plan_dispatch(wl, new)
        yo = O.expert_dequant(d["recv_x"], d["recv_scales"], 0.5)
        y.copy_(dev(yo))  # the expert stand-in for this replay, written before it
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        counts = host(g.counts)
        assert np.array_equal(counts, pl["recv_counts"]), rep
        rx, rs = host(g.recv_x), host(g.recv_s)
        for r in range(R):
            n = int(counts[r])
            assert np.array_equal(host(g.spos)[r, :n], pl["src_token_pos"][r, :n]), rep
            assert np.array_equal(rx[r, :n], d["recv_x"][r, :n]), rep
            assert np.array_equal(rs[r, :n].view(np.uint32),
                                  d["recv_scales"][r, :n].view(np.uint32)), rep
        ref = O.combine(yo, new["weights"], new["indices"], pl, epr, cap)
        check_combine(host(out, np.uint16), ref)
    assert M.mep_get_status(g.m.h) == 0


def test_hip_graph_expert_major_replay():
    # plan+dispatch, the expert-major conversion and the expert-major combine
    # captured once in a HIP graph, replayed with new routing and token rows
    # (eager refills in between): each replay must match the oracle
    wl = _variant("stdmoe", tokens=700, cap=1024, hidden=1024)
    T, H, cap_em = wl.tokens, wl.hidden, wl.cap_em
    inp = make_inputs(wl, 400)
    g = gpu_plan_dispatch(wl, inp, fused=True)
    em_x = torch.empty((cap_em, H), dtype=torch.uint8, device="cuda")
    em_s = torch.empty((cap_em, H // 128), dtype=torch.float32, device="cuda")
    em_counts = torch.empty((wl.experts,), dtype=torch.int32, device="cuda")
    em_offsets = torch.empty((wl.experts + 1,), dtype=torch.int32, device="cuda")
    em_src = torch.empty((cap_em,), dtype=torch.int32, device="cuda")
    y = torch.zeros((cap_em, H), dtype=torch.int16, device="cuda")
    out = torch.zeros((T, H), dtype=torch.int16, device="cuda")
    M.mep_to_expert_major(g.m.h, g.recv_x, g.recv_s, g.recv_i, g.counts, g.spos, em_x, em_s,
                          em_counts, em_offsets, em_src, cap_em)  # eager warm-up
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        M.mep_plan_dispatch(g.m.h, g.idx, T, g.counts, g.spos, g.x, g.w, None, g.recv_x, g.recv_s,
                            g.recv_w, g.recv_i)
        M.mep_to_expert_major(g.m.h, g.recv_x, g.recv_s, g.recv_i, g.counts, g.spos, em_x, em_s,
                              em_counts, em_offsets, em_src, cap_em)
        M.mep_combine(g.m.h, M.MEP_EXPERT_MAJOR, y, g.w, out)
    for rep in range(4):
        new = make_inputs(wl, 500 + rep)
        g.x.copy_(dev(new["x"]))
        g.idx.copy_(dev(new["indices"]))
        g.w.copy_(dev(new["weights"]))
        em_x.fill_(SENT8)
        em_src.fill_(SENT32)
        pl, d = oracle_plan_dispatch(wl, new)
        em = O.to_expert_major(d, pl, wl.ranks, wl.experts_per_rank, wl.cap, T, cap_em, 0)
        y_ref = stand_in_oracle(wl, em["em_x"], em["em_scales"])
        y.copy_(dev(y_ref))  # the expert stand-in for this replay, written before it
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _say(f"expert-major replay {rep}")
        em_route = torch.full((T, wl.topk), SENT32, dtype=torch.int32, device="cuda")
        M.mep_get_route(g.m.h, torch.empty((T, wl.topk), dtype=torch.int32, device="cuda"),
                        em_route)
        torch.cuda.synchronize()
        check_expert_major(wl, em, em_x, em_s, em_counts, em_offsets, em_src, em_route)
        check_combine(host(out, np.uint16), O.combine_em(y_ref, new["weights"], em["tok_em_row"]))
    assert M.mep_get_status(g.m.h) == 0


def test_two_handles_on_two_streams():
    # two handles, each bound to its own (default-priority) stream, with their
    # calls interleaved on the host: no state is shared between handles, and
    # each stream's work matches the oracle
    wls = [_variant("prefill", tokens=500, cap=512), _variant("skew", tokens=300, cap=300)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    runs = []
    for i, wl in enumerate(wls):
        inp = make_inputs(wl, 20 + i)
        with torch.cuda.stream(streams[i]):
            g = gpu_plan_dispatch(wl, inp, src_rank=i, fused=bool(i))
        runs.append((wl, inp, g))
    outs = []
    for i, (wl, inp, g) in enumerate(runs):
        with torch.cuda.stream(streams[i]):
            y = g.recv_x if wl.quant == "none" else None
            if y is None:
                q = g.recv_x.view(torch.float8_e4m3fn).float()
                y = ((q * g.recv_s.repeat_interleave(128, dim=-1)) * 0.5).to(torch.bfloat16) \
                    .view(torch.int16)
            out = torch.empty((wl.tokens, wl.hidden), dtype=torch.int16, device="cuda")
            M.mep_combine(g.m.h, M.MEP_RANK_MAJOR, y, g.w, out)
            outs.append((y, out))
    torch.cuda.synchronize()
    for i, (wl, inp, g) in enumerate(runs):
        pl, d = oracle_plan_dispatch(wl, inp, src_rank=i)
        check_plan_dispatch(wl, inp, g, pl, d)
        y, out = outs[i]
        # expert outputs on the oracle side come from the oracle's own dispatch
        ref = O.combine(stand_in_oracle(wl, d["recv_x"], d["recv_scales"]), inp["weights"],
                        inp["indices"], pl, wl.experts_per_rank, wl.cap)
        check_combine(host(out, np.uint16), ref)
        assert M.mep_get_status(g.m.h, streams[i]) == 0


@pytest.mark.parametrize("H,T,R,epr,k,quant,layout", [
    (16384, 200, 8, 4, 4, "fp8", "rank_major"),
    (16384, 200, 8, 4, 4, "fp8", "expert_major"),
    (16384, 77, 4, 4, 8, "none", "rank_major"),
    (1 << 20, 9, 2, 2, 2, "fp8", "rank_major"),
    (1 << 20, 9, 2, 2, 2, "none", "rank_major"),
])
def test_wide_hidden(H, T, R, epr, k, quant, layout):
    # rows wider than the 7168-column workloads, up to the widest the config
    # accepts (2^20 columns: 1024 combine slices per token, 8192 scale words
    # per FP8 row); whole path, both call modes, last rank as the source
    expert = "identity" if quant == "none" else "dequant_half"
    wl = Workload("wide", T, H, R, epr, k, T, quant, "uniform", expert, layout)
    for fused in (False, True):
        _say(f"H={H} T={T} R={R} {quant} {layout} fused={fused}")
        st = run_full(wl, 11, src_rank=R - 1, fused=fused)
        assert st["max_ulp"] <= 1


def test_buffers_past_4_gib():
    # 45000 bf16 tokens of 7168 columns: the receive buffers (5.2 GB) and the
    # expert-major rows (5.6 GB) reach byte offsets past 2^32, so every row
    # address needs 64-bit arithmetic.  Checked in full against the oracle:
    # plan outputs, every received row, weight and id, the combine of every
    # token (identity expert); then the expert-major layout and rows from the
    # standard-MoE dispatch and its combine, every token.
    wl = dataclasses.replace(WORKLOADS["decode"], tokens=45000, cap=45000)
    T, R, cap, H, k, epr, E = wl.tokens, wl.ranks, wl.cap, wl.hidden, wl.topk, \
        wl.experts_per_rank, wl.experts
    assert R * cap * H * 2 > 2**32
    inp = make_inputs(wl, 11)
    idx_h, w_h, x_h = inp["indices"], inp["weights"], inp["x"]
    pl = O.plan(idx_h, R, epr, cap)
    m = M.Mep(H, epr, k, cap, R)
    x, w, idx = dev(x_h), dev(w_h), dev(idx_h)
    counts = torch.empty(R, dtype=torch.int32, device="cuda")
    spos = torch.empty((R, cap), dtype=torch.int32, device="cuda")
    recv_x = torch.empty((R, cap, H), dtype=torch.int16, device="cuda")
    recv_w = torch.empty((R, cap, k), dtype=torch.float32, device="cuda")
    recv_i = torch.empty((R, cap, k), dtype=torch.int32, device="cuda")
    route = torch.empty((T, k), dtype=torch.int32, device="cuda")
    out = torch.empty((T, H), dtype=torch.int16, device="cuda")
    _say(f"[big] T={T} H={H} R={R} fused plan+dispatch, combine")
    M.mep_plan_dispatch(m.h, idx, T, counts, spos, x, w, None, recv_x, None, recv_w, recv_i)
    M.mep_get_route(m.h, route)
    M.mep_combine(m.h, M.MEP_RANK_MAJOR, recv_x, w, out)
    torch.cuda.synchronize()
    assert M.mep_get_status(m.h) == 0
    n = pl["recv_counts"]
    assert np.array_equal(host(counts), n)
    sp = host(spos)
    for r in range(R):
        assert np.array_equal(sp[r, :n[r]], pl["src_token_pos"][r, :n[r]])
    rt = host(route)
    assert np.array_equal(rt, np.where(pl["slot"] >= 0, (idx_h // epr) * cap + pl["slot"], -1))
    d = O.dispatch(x_h, w_h, idx_h, pl, R, epr, cap, False)
    for r in range(R):  # rank by rank, to keep host copies to one rank's rows
        nr = int(n[r])
        assert np.array_equal(host(recv_x[r, :nr], np.uint16), d["recv_x"][r, :nr]), r
        assert np.array_equal(host(recv_w[r, :nr]).view(np.uint32),
                              d["recv_weights"][r, :nr].view(np.uint32)), r
        assert np.array_equal(host(recv_i[r, :nr]), d["recv_indices"][r, :nr]), r
    ref = O.combine(d["recv_x"], w_h, idx_h, pl, epr, cap)
    _say(f"[big] rank-major combine: {check_combine(host(out, np.uint16), ref)}")
    del recv_x, recv_w, recv_i
    torch.cuda.empty_cache()

    # the same tokens straight into the expert-major layout, and its combine
    M.mep_reset(m.h)
    cap_em = wl.cap_em
    assert cap_em * H * 2 > 2**32
    em_x = torch.empty((cap_em, H), dtype=torch.int16, device="cuda")
    emc = torch.empty(E, dtype=torch.int32, device="cuda")
    emo = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    emp = torch.empty(cap_em, dtype=torch.int32, device="cuda")
    em_route = torch.empty((T, k), dtype=torch.int32, device="cuda")
    out2 = torch.empty((T, H), dtype=torch.int16, device="cuda")
    _say(f"[big] standard-MoE dispatch, cap_em={cap_em}, expert-major combine")
    M.mep_dispatch_standard_moe(m.h, idx, T, x, None, em_x, None, emc, emo, emp, cap_em)
    M.mep_get_route(m.h, None, em_route)
    M.mep_combine(m.h, M.MEP_EXPERT_MAJOR, em_x, w, out2)
    torch.cuda.synchronize()
    assert M.mep_get_status(m.h) == 0
    cnt = np.bincount(idx_h.ravel(), minlength=E)
    assert np.array_equal(host(emc), cnt)
    offs = np.concatenate([[0], np.cumsum((cnt + 127) // 128 * 128)])
    assert np.array_equal(host(emo), offs)
    em = O.to_expert_major(d, pl, R, epr, cap, T, cap_em, 0)
    del d
    assert np.array_equal(host(em_route), em["tok_em_row"])
    pos = host(emp)
    for e in range(E):
        o, ne = int(offs[e]), int(cnt[e])
        assert np.array_equal(pos[o:o + ne], em["em_src_pos"][o:o + ne]), e
        assert np.array_equal(host(em_x[o:o + ne], np.uint16), em["em_x"][o:o + ne]), e
    ref2 = O.combine_em(em["em_x"], w_h, em["tok_em_row"])
    _say(f"[big] expert-major combine: {check_combine(host(out2, np.uint16), ref2)}")


@pytest.mark.parametrize("R,epr,k,layout", [(8, 32, 16, "rank_major"), (8, 32, 32, "rank_major"),
                                           (5, 8, 12, "rank_major"), (16, 16, 16, "rank_major"),
                                           (8, 32, 32, "expert_major")])
def test_wide_top_k_combine(R, epr, k, layout):
    # top-k above 8: up to 8 ranks, each distinct rank row is held once and the
    # positions pick it in j order; more ranks or the expert-major layout go
    # through groups of 8 positions.  Whole path against the oracle.
    wl = Workload("wide_k", 700, 1024, R, epr, k, 700, "fp8", "uniform", "dequant_half", layout)
    stats = run_full(wl, 21, src_rank=R - 1, fused=True)
    _say(f"[wide] R={R} k={k} {layout}: {stats}")


@pytest.mark.parametrize("R,epr,k", [(8, 32, 16), (7, 4, 28), (16, 16, 16)])
def test_wide_top_k_in_flight_rounding(R, epr, k):
    # the E4M3 rounding in flight at top-k above 8 equals cast + E4M3 combine
    wl = Workload("wide_r", 300, 512, R, epr, k, 300, "none", "uniform", "identity",
                  "rank_major")
    inp = make_inputs(wl, 22)
    g = gpu_plan_dispatch(wl, inp, fused=True)
    pl, d = oracle_plan_dispatch(wl, inp)
    y8 = torch.zeros(g.recv_x.shape, dtype=torch.uint8, device="cuda")
    M.mep_cast_fp8_direct(g.m.h, M.MEP_RANK_MAJOR, g.recv_x, y8)
    two = torch.empty((wl.tokens, wl.hidden), dtype=torch.int16, device="cuda")
    M.mep_combine_fp8(g.m.h, M.MEP_RANK_MAJOR, y8, g.w, two)
    one = torch.empty_like(two)
    M.mep_combine_fp8_direct(g.m.h, M.MEP_RANK_MAJOR, g.recv_x, g.w, one)
    torch.cuda.synchronize()
    assert torch.equal(one, two)
    n = pl["recv_counts"]
    used = np.arange(wl.cap)[None, :] < n[:, None]
    ref8 = np.zeros(d["recv_x"].shape, dtype=np.uint8)
    ref8[used] = O.cast_fp8_direct(d["recv_x"][used])
    ref = O.combine(O.e4m3_to_bf16(ref8), inp["weights"], inp["indices"], pl, epr, wl.cap)
    check_combine(host(one, np.uint16), ref)
    assert M.mep_get_status(g.m.h) == 0
