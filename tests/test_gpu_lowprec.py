"""GPU parity of the low-precision variants: MXFP4 dispatch payloads, carried
FP4 payloads, and the FP8 direct-cast combine payload.

Sources: "Choosing an EP API and backend" (FP4 conversion kernels on gfx950;
the HIP backend's dispatch can move FP8/FP4 rows that arrive quantized;
OCP E4M3 on gfx950), and "MORI-EP User Guide" section 10 Tuning, whose intra-node tuning
matrix pairs an FP4 dispatch with a bf16 combine and quant type
fp8_direct_cast.  The block formats are the readings the
oracle documents (OCP MX FP4: E2M1 codes, E8M0 scale per 32 columns; E4M3
direct cast without a scale, saturating at 448).

Bar: bit-exact for every byte and scale; combine within 1 bf16 ulp.
"""

import dataclasses

import numpy as np
import pytest
import torch

import combine_mep_plan_amd as M
from oracle import oracle as O
from synthetic import WORKLOADS, make_fp8_payload, make_inputs

from _gpu_harness import SENT8, SENT32, check_combine, dev, host

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _bf16_bits(v):
    return torch.from_numpy(np.asarray(v, dtype=np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


def _edge_rows(x):
    """Plant MX edge blocks in the first rows of x (bf16 bits [T,H], H >= 256)."""
    x = x.copy()
    x[0, 0:32] = 0                                        # zero block
    x[1, 32:64] = 0x8000                                  # negative zeros
    x[2, 64:96] = np.arange(1, 33, dtype=np.uint16)       # bf16 subnormals only
    x[2, 96:128] = np.arange(1, 33, dtype=np.uint16) | 0x8000
    x[3, 0:32] = 0x7F7F - np.arange(32, dtype=np.uint16)  # near the bf16 maximum
    ties = np.array([6, .25, .75, 1.25, 1.75, 2.5, 3.5, 5, -.25, -.75, -1.25, -1.75, -2.5,
                     -3.5, -5, 0.5, 1, 1.5, 2, 3, 4, -6, 0, -0.0, .3, .7, 1.3, 1.7, 2.4, 3.6,
                     4.9, 5.1]) * 8.0
    x[4, 128:160] = _bf16_bits(ties)                      # every E2M1 rounding tie
    return x


def _mep(wl, quant, sd=None):
    return M.Mep(wl.hidden, wl.experts_per_rank, wl.topk, wl.cap, wl.ranks, quant=quant,
                 scale_dim=sd)


def _run_rank_major(wl, m, x, w, idx, sc, fused, sd_words):
    R, cap, k = wl.ranks, wl.cap, wl.topk
    row_bytes = wl.hidden // 2
    counts = torch.full((R,), SENT32, dtype=torch.int32, device="cuda")
    spos = torch.full((R, cap), SENT32, dtype=torch.int32, device="cuda")
    rx = torch.full((R, cap, row_bytes), SENT8, dtype=torch.uint8, device="cuda")
    rs = (torch.full((R, cap, sd_words), float("nan"), device="cuda") if sd_words else None)
    rw = torch.full((R, cap, k), float("nan"), device="cuda")
    ri = torch.full((R, cap, k), SENT32, dtype=torch.int32, device="cuda")
    T = idx.shape[0]
    if fused:
        M.mep_plan_dispatch(m.h, idx, T, counts, spos, x, w, sc, rx, rs, rw, ri)
    else:
        M.mep_plan(m.h, idx, T, counts, spos)
        M.mep_dispatch(m.h, x, w, sc, idx, rx, rs, rw, ri)
    return counts, spos, rx, rs, rw, ri


def _check_rank_major(wl, inp, pl, d, got, sd_words):
    counts, spos, rx, rs, rw, ri = got
    torch.cuda.synchronize()
    assert np.array_equal(host(counts), pl["recv_counts"])
    written = np.arange(wl.cap)[None, :] < pl["recv_counts"][:, None]
    assert np.array_equal(host(spos)[written], pl["src_token_pos"][written])
    assert np.array_equal(host(rx), d["recv_x"]), "received FP4 rows differ"
    if sd_words:
        hs = host(rs)
        assert np.array_equal(hs[written].view(np.uint32), d["recv_scales"][written].view(np.uint32))
        assert np.all(np.isnan(hs[~written]))
    assert np.array_equal(host(rw)[written].view(np.uint32),
                          d["recv_weights"][written].view(np.uint32))
    assert np.array_equal(host(ri)[written], d["recv_indices"][written])


# ---------------------------------------------------------------------------
# MXFP4 and carried FP4 through the rank-major dispatch and the conversion
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("fused", [False, True], ids=["separate", "fused"])
@pytest.mark.parametrize("T", [5, 300, 4096])
def test_mxfp4_dispatch(T, fused):
    wl = WORKLOADS["prefill"].with_tokens(T)
    _say(f"[mxfp4] T={T} fused={fused}")
    inp = make_inputs(wl, 41)
    inp["x"] = _edge_rows(inp["x"])
    m = _mep(wl, M.MEP_QUANT_MXFP4)
    got = _run_rank_major(wl, m, dev(inp["x"]), dev(inp["weights"]), dev(inp["indices"]), None,
                          fused, wl.hidden // 128)
    pl = O.plan(inp["indices"], wl.ranks, wl.experts_per_rank, wl.cap)
    d = O.dispatch(inp["x"], inp["weights"], inp["indices"], pl, wl.ranks, wl.experts_per_rank,
                   wl.cap, 4, fill=SENT8)
    _check_rank_major(wl, inp, pl, d, got, wl.hidden // 128)
    assert M.mep_get_status(m.h) == 0
    # the MXFP4 rows convert to expert-major with their scale words
    counts, spos, rx, rs, rw, ri = got
    ce = wl.cap_em
    emx = torch.full((ce, wl.hidden // 2), SENT8, dtype=torch.uint8, device="cuda")
    ems = torch.full((ce, wl.hidden // 128), float("nan"), device="cuda")
    emc = torch.empty(wl.experts, dtype=torch.int32, device="cuda")
    emo = torch.empty(wl.experts + 1, dtype=torch.int32, device="cuda")
    emp = torch.full((ce,), SENT32, dtype=torch.int32, device="cuda")
    M.mep_to_expert_major(m.h, rx, rs, ri, counts, spos, emx, ems, emc, emo, emp, ce)
    em = O.to_expert_major(d, pl, wl.ranks, wl.experts_per_rank, wl.cap, T, ce, fill=SENT8)
    torch.cuda.synchronize()
    assert np.array_equal(host(emc), em["em_counts"])
    assert np.array_equal(host(emo), em["em_offsets"])
    assert np.array_equal(host(emx), em["em_x"])
    used = host(emp) != SENT32
    assert np.array_equal(host(emp)[used], em["em_src_pos"][used])
    assert np.array_equal(host(ems)[used].view(np.uint32), em["em_scales"][used].view(np.uint32))


@pytest.mark.parametrize("fused", [False, True], ids=["separate", "fused"])
@pytest.mark.parametrize("T,sd", [(70, 0), (700, 3), (4096, 56)])
def test_fp4_carry_dispatch(T, sd, fused):
    wl = WORKLOADS["prefill"].with_tokens(T)
    _say(f"[fp4 carry] T={T} sd={sd} fused={fused}")
    inp = make_inputs(wl, 43)
    p = make_fp8_payload(T, wl.hidden // 2, sd, 43)  # arbitrary bytes serve as packed E2M1
    m = _mep(wl, M.MEP_QUANT_FP4_CARRY, sd)
    got = _run_rank_major(wl, m, dev(p["q"]), dev(inp["weights"]), dev(inp["indices"]),
                          dev(p["scales"]) if sd else None, fused, sd)
    pl = O.plan(inp["indices"], wl.ranks, wl.experts_per_rank, wl.cap)
    d = O.dispatch(p["q"], inp["weights"], inp["indices"], pl, wl.ranks, wl.experts_per_rank,
                   wl.cap, 3, fill=SENT8, scales=p["scales"])
    _check_rank_major(wl, inp, pl, d, got, sd)


@pytest.mark.parametrize("mode,T", [("mxfp4", 1000), ("mxfp4", 4096), ("fp4carry", 700)])
def test_standard_moe_fp4(mode, T):
    wl = WORKLOADS["stdmoe"].with_tokens(T)
    _say(f"[std fp4] {mode} T={T}")
    inp = make_inputs(wl, 47)
    E, H, ce = wl.experts, wl.hidden, wl.cap_em
    if mode == "mxfp4":
        quant, sd, x, sc, q = M.MEP_QUANT_MXFP4, H // 128, _edge_rows(inp["x"]), None, 4
    else:
        p = make_fp8_payload(T, H // 2, 5, 47)
        quant, sd, x, sc, q = M.MEP_QUANT_FP4_CARRY, 5, p["q"], p["scales"], 3
    m = _mep(wl, quant, sd)
    emx = torch.full((ce, H // 2), SENT8, dtype=torch.uint8, device="cuda")
    ems = torch.full((ce, sd), float("nan"), device="cuda")
    emc = torch.empty(E, dtype=torch.int32, device="cuda")
    emo = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    emp = torch.full((ce,), SENT32, dtype=torch.int32, device="cuda")
    M.mep_dispatch_standard_moe(m.h, dev(inp["indices"]), T, dev(x),
                                dev(sc) if sc is not None else None, emx, ems, emc, emo, emp, ce)
    em = O.dispatch_standard_moe(x, inp["weights"], inp["indices"], wl.ranks,
                                 wl.experts_per_rank, wl.cap, q, ce, fill=SENT8, scales=sc)
    torch.cuda.synchronize()
    assert np.array_equal(host(emc), em["em_counts"])
    assert np.array_equal(host(emo), em["em_offsets"])
    assert np.array_equal(host(emx), em["em_x"])
    used = host(emp) != SENT32
    assert np.array_equal(host(emp)[used], em["em_src_pos"][used])
    assert used.sum() == em["em_counts"].sum()
    assert np.array_equal(host(ems)[used].view(np.uint32), em["em_scales"][used].view(np.uint32))
    assert M.mep_get_status(m.h) == 0


# ---------------------------------------------------------------------------
# FP8 direct-cast combine payload
# ---------------------------------------------------------------------------

def _expert_outputs(shape, seed):
    """bf16 expert outputs with values past +-448, exact E4M3 ties, signed zeros."""
    rng = np.random.default_rng(seed)
    v = rng.standard_normal(shape).astype(np.float32) * 60.0
    flat = v.reshape(-1)
    flat[:8] = [1000.0, -1000.0, 448.0, -464.0, 0.0, -0.0, 17.0, -0.009765625]  # ties, zeros
    return _bf16_bits(v)


def _check_in_flight(m, layout, y_dev, w_dev, out_two_step):
    """mep_combine_fp8_direct (the rounding in registers) equals the cast +
    E4M3 combine bit for bit."""
    out = torch.empty_like(out_two_step)
    M.mep_combine_fp8_direct(m.h, layout, y_dev, w_dev, out)
    torch.cuda.synchronize()
    assert torch.equal(out, out_two_step), "in-flight rounding differs from cast + combine"


_TABLES = {}


def _oracle_cast(y_bits):
    """The oracle's E4M3 direct cast of bf16 values, looked up in the oracle's
    own encodes of all 65536 bf16 patterns (the cast depends on the input
    pattern alone, so this is the oracle's result for every element; its
    search-based encoder over 10^8 values would take minutes)."""
    if "cast" not in _TABLES:
        _TABLES["cast"] = O.cast_fp8_direct(np.arange(65536, dtype=np.uint16))
    return _TABLES["cast"][y_bits]


def _oracle_e4m3_to_bf16(codes):
    """The oracle's exact E4M3 -> bf16 of every code, looked up likewise."""
    if "dec" not in _TABLES:
        _TABLES["dec"] = O.e4m3_to_bf16(np.arange(256, dtype=np.uint8))
    return _TABLES["dec"][codes]


def _check_cast_combine(y, y8_gpu, out_gpu, used, tok_rows, combine_ref, T, sample):
    """y: bf16 bits [rows, H]; used: routed rows; tok_rows[t]: rows token t reads.
    Checks the cast of the routed rows (all of them, or those of `sample`
    tokens), the untouched rows, and the combined outputs of those tokens."""
    rng = np.random.default_rng(T)
    toks = np.arange(T) if sample is None else np.unique(
        np.concatenate([[0, T - 1], rng.choice(T, sample, replace=False)]))
    need = np.zeros(used.shape, bool)
    for t in toks:
        need[[r for r in tok_rows[t] if r >= 0]] = True
    if sample is None:
        need |= used
    ref8 = np.full(y.shape, SENT8, dtype=np.uint8)
    ref8[need] = _oracle_cast(y[need])
    g8 = host(y8_gpu).reshape(y.shape)
    assert np.array_equal(g8[need], ref8[need]), "direct cast differs"
    assert np.all(g8[~used] == SENT8), "direct cast touched rows that are not routed"
    ref = combine_ref(_oracle_e4m3_to_bf16(ref8))
    return check_combine(host(out_gpu, np.uint16)[toks], ref[toks])


@pytest.mark.parametrize("T,sample", [(1, None), (200, None), (4096, None)])
def test_fp8_direct_cast_and_combine_rank_major(T, sample):
    wl = WORKLOADS["prefill"].with_tokens(T)
    _say(f"[fp8 direct] rank-major T={T}")
    inp = make_inputs(wl, 53)
    R, cap, H, epr = wl.ranks, wl.cap, wl.hidden, wl.experts_per_rank
    m = _mep(wl, M.MEP_QUANT_NONE, 0)
    counts = torch.empty(R, dtype=torch.int32, device="cuda")
    spos = torch.empty((R, cap), dtype=torch.int32, device="cuda")
    idx, w = dev(inp["indices"]), dev(inp["weights"])
    M.mep_plan(m.h, idx, T, counts, spos)
    y = _expert_outputs((R * cap, H), 53)
    y_dev = dev(y)
    y8 = torch.full((R, cap, H), SENT8, dtype=torch.uint8, device="cuda")
    M.mep_cast_fp8_direct(m.h, M.MEP_RANK_MAJOR, y_dev, y8)
    out = torch.empty((T, H), dtype=torch.int16, device="cuda")
    M.mep_combine_fp8(m.h, M.MEP_RANK_MAJOR, y8, w, out)
    torch.cuda.synchronize()
    _check_in_flight(m, M.MEP_RANK_MAJOR, y_dev, w, out)
    pl = O.plan(inp["indices"], R, epr, cap)
    used = (np.arange(cap)[None, :] < pl["recv_counts"][:, None]).reshape(-1)
    tok_rows = (inp["indices"] // epr) * cap + pl["slot"]
    ref_fn = lambda y8r: O.combine(y8r.reshape(R, cap, H), inp["weights"], inp["indices"],  # noqa: E731
                                   pl, epr, cap)
    stats = _check_cast_combine(y, y8, out, used, tok_rows, ref_fn, T, sample)
    _say(f"[fp8 direct] T={T}: {stats}")


@pytest.mark.parametrize("R,epr,k", [(1, 8, 8), (2, 8, 8), (4, 4, 8), (3, 4, 7), (8, 2, 5)])
def test_fp8_combine_shared_rank_rows(R, epr, k):
    # top-k positions sharing rank rows: one rank (eight positions on one row),
    # four ranks at top-8 (up to four rows repeated), an odd top-7, top-5:
    # every repeated row is read back from where the E4M3 combine parks it
    wl = dataclasses.replace(WORKLOADS["prefill"], tokens=300, cap=300, hidden=512, ranks=R,
                             experts_per_rank=epr, topk=k)
    _say(f"[fp8 direct] shared rank rows R={R} epr={epr} k={k}")
    inp = make_inputs(wl, 61)
    T, cap, H = wl.tokens, wl.cap, wl.hidden
    m = _mep(wl, M.MEP_QUANT_NONE, 0)
    counts = torch.empty(R, dtype=torch.int32, device="cuda")
    spos = torch.empty((R, cap), dtype=torch.int32, device="cuda")
    idx, w = dev(inp["indices"]), dev(inp["weights"])
    M.mep_plan(m.h, idx, T, counts, spos)
    y = _expert_outputs((R * cap, H), 61)
    y_dev = dev(y)
    y8 = torch.full((R, cap, H), SENT8, dtype=torch.uint8, device="cuda")
    M.mep_cast_fp8_direct(m.h, M.MEP_RANK_MAJOR, y_dev, y8)
    out = torch.empty((T, H), dtype=torch.int16, device="cuda")
    M.mep_combine_fp8(m.h, M.MEP_RANK_MAJOR, y8, w, out)
    torch.cuda.synchronize()
    _check_in_flight(m, M.MEP_RANK_MAJOR, y_dev, w, out)
    pl = O.plan(inp["indices"], R, epr, cap)
    used = (np.arange(cap)[None, :] < pl["recv_counts"][:, None]).reshape(-1)
    tok_rows = (inp["indices"] // epr) * cap + pl["slot"]
    ref_fn = lambda y8r: O.combine(y8r.reshape(R, cap, H), inp["weights"], inp["indices"],  # noqa: E731
                                   pl, epr, cap)
    stats = _check_cast_combine(y, y8, out, used, tok_rows, ref_fn, T, None)
    _say(f"[fp8 direct] R={R} k={k}: {stats}")
    assert M.mep_get_status(m.h) == 0


@pytest.mark.parametrize("T,sample", [(300, None), (4096, None)])
def test_fp8_direct_cast_and_combine_expert_major(T, sample):
    wl = WORKLOADS["stdmoe"].with_tokens(T)
    wl = dataclasses.replace(wl, quant="none")
    _say(f"[fp8 direct] expert-major T={T}")
    inp = make_inputs(wl, 59)
    H, E, ce = wl.hidden, wl.experts, wl.cap_em
    m = _mep(wl, M.MEP_QUANT_NONE, 0)
    emx = torch.empty((ce, H), dtype=torch.int16, device="cuda")
    emc = torch.empty(E, dtype=torch.int32, device="cuda")
    emo = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    emp = torch.empty(ce, dtype=torch.int32, device="cuda")
    M.mep_dispatch_standard_moe(m.h, dev(inp["indices"]), T, dev(inp["x"]), None, emx, None,
                                emc, emo, emp, ce)
    y = _expert_outputs((ce, H), 59)
    y_dev, w_dev = dev(y), dev(inp["weights"])
    y8 = torch.full((ce, H), SENT8, dtype=torch.uint8, device="cuda")
    M.mep_cast_fp8_direct(m.h, M.MEP_EXPERT_MAJOR, y_dev, y8)
    out = torch.empty((T, H), dtype=torch.int16, device="cuda")
    M.mep_combine_fp8(m.h, M.MEP_EXPERT_MAJOR, y8, w_dev, out)
    torch.cuda.synchronize()
    _check_in_flight(m, M.MEP_EXPERT_MAJOR, y_dev, w_dev, out)
    # the layout, from the routing alone (no payload needed)
    em = O.dispatch_standard_moe(np.zeros((T, 16), np.uint16), inp["weights"], inp["indices"],
                                 wl.ranks, wl.experts_per_rank, wl.cap, 0, ce)
    used = np.zeros(ce, bool)
    for e in range(E):
        o = em["em_offsets"][e]
        used[o:o + em["em_counts"][e]] = True
    ref_fn = lambda y8r: O.combine_em(y8r, inp["weights"], em["tok_em_row"])  # noqa: E731
    stats = _check_cast_combine(y, y8, out, used, em["tok_em_row"], ref_fn, T, sample)
    _say(f"[fp8 direct] EM T={T}: {stats}")


@pytest.mark.parametrize("R,epr,k", [(6, 4, 12), (4, 8, 32)])
def test_fp8_direct_and_mxfp4_wide_topk(R, epr, k):
    # top-k above 8: the cast walks a token's rows in groups of 8 and the combine
    # takes its wide variant; ranks shared by several experts repeat rows
    wl = dataclasses.replace(WORKLOADS["prefill"].with_tokens(150, cap=150), ranks=R,
                             experts_per_rank=epr, topk=k, hidden=512)
    _say(f"[wide] R={R} epr={epr} k={k}")
    inp = make_inputs(wl, 61)
    cap, H = wl.cap, wl.hidden
    # MXFP4 dispatch
    m4 = _mep(wl, M.MEP_QUANT_MXFP4)
    got = _run_rank_major(wl, m4, dev(inp["x"]), dev(inp["weights"]), dev(inp["indices"]),
                          None, True, H // 128)
    pl = O.plan(inp["indices"], R, epr, cap)
    d = O.dispatch(inp["x"], inp["weights"], inp["indices"], pl, R, epr, cap, 4, fill=SENT8)
    _check_rank_major(wl, inp, pl, d, got, H // 128)
    # direct cast and E4M3 combine
    m = _mep(wl, M.MEP_QUANT_NONE, 0)
    idx, w = dev(inp["indices"]), dev(inp["weights"])
    M.mep_plan(m.h, idx, wl.tokens, torch.empty(R, dtype=torch.int32, device="cuda"),
               torch.empty((R, cap), dtype=torch.int32, device="cuda"))
    y = _expert_outputs((R * cap, H), 61)
    y_dev = dev(y)
    y8 = torch.full((R, cap, H), SENT8, dtype=torch.uint8, device="cuda")
    M.mep_cast_fp8_direct(m.h, M.MEP_RANK_MAJOR, y_dev, y8)
    out = torch.empty((wl.tokens, H), dtype=torch.int16, device="cuda")
    M.mep_combine_fp8(m.h, M.MEP_RANK_MAJOR, y8, w, out)
    torch.cuda.synchronize()
    _check_in_flight(m, M.MEP_RANK_MAJOR, y_dev, w, out)
    used = (np.arange(cap)[None, :] < pl["recv_counts"][:, None]).reshape(-1)
    tok_rows = (inp["indices"] // epr) * cap + pl["slot"]
    ref_fn = lambda y8r: O.combine(y8r.reshape(R, cap, H), inp["weights"], inp["indices"],  # noqa: E731
                                   pl, epr, cap)
    _check_cast_combine(y, y8, out, used, tok_rows, ref_fn, wl.tokens, None)


def test_fp8_direct_state_and_shape_rules():
    wl = WORKLOADS["tiny"]
    m = _mep(wl, M.MEP_QUANT_NONE, 0)
    y = torch.zeros((wl.ranks, wl.cap, wl.hidden), dtype=torch.int16, device="cuda")
    y8 = torch.zeros((wl.ranks, wl.cap, wl.hidden), dtype=torch.uint8, device="cuda")
    for fn in (lambda: M.mep_cast_fp8_direct(m.h, M.MEP_RANK_MAJOR, y, y8),
               lambda: M.mep_combine_fp8(m.h, M.MEP_EXPERT_MAJOR, y8, None, y),
               lambda: M.mep_combine_fp8_direct(m.h, M.MEP_RANK_MAJOR, y, None, y)):
        with pytest.raises(M.MepError) as e:
            fn()
        assert e.value.code == M.MEP_ERR_STATE
    odd = M.Mep(24, 2, 2, 16, 4)  # H = 24: not a whole number of 16-byte E4M3 units
    idx = torch.zeros((1, 2), dtype=torch.int32, device="cuda")
    idx[0, 1] = 1
    M.mep_plan(odd.h, idx, 1, torch.empty(4, dtype=torch.int32, device="cuda"),
               torch.empty((4, 16), dtype=torch.int32, device="cuda"))
    y24 = torch.zeros((4, 16, 24), dtype=torch.int16, device="cuda")
    with pytest.raises(M.MepError) as e:
        M.mep_cast_fp8_direct(odd.h, M.MEP_RANK_MAJOR, y24, y24)
    assert e.value.code == M.MEP_ERR_SHAPE
