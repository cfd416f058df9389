"""GPU parity over seeded random configurations.

Each case draws a configuration -- ranks, experts per rank, top-k, tokens,
capacity slack, hidden size, payload mode, layout, fused or separate plan,
source rank, planted bad or repeated expert ids, combine payload (bf16, the
E4M3 rounding in flight, or cast + E4M3 combine) -- runs the whole path through
the C ABI and checks it against the oracle: plan outputs, received rows and
scales, the expert-major layout (by conversion or by the standard-MoE call),
and the combine.  The draws are small so the oracle stays fast; they reach
combinations the hand-picked cases do not.

Sources as for the other parity tests ("MORI-EP User Guide" sections 3 and 4;
"Choosing an EP API and backend").
"""

import dataclasses

import numpy as np
import pytest
import torch

import combine_mep_plan_amd as M
from oracle import oracle as O
from synthetic import Workload, make_fp8_payload, make_inputs

from _gpu_harness import SENT8, SENT16, SENT32, check_combine, dev, host

pytestmark = pytest.mark.gpu

MODES = {  # name: (library mode, oracle mode, rows arrive quantised, bytes per value)
    "bf16": (M.MEP_QUANT_NONE, 0, False),
    "fp8": (M.MEP_QUANT_FP8_E4M3_BLOCK128, 1, False),
    "fp8carry": (M.MEP_QUANT_FP8_CARRY, 2, True),
    "fp4carry": (M.MEP_QUANT_FP4_CARRY, 3, True),
    "mxfp4": (M.MEP_QUANT_MXFP4, 4, False),
}


def draw(seed):
    rng = np.random.default_rng(1000 + seed)
    while True:
        R = int(rng.choice([1, 2, 3, 4, 7, 8, 16, 33, 64]))
        epr = int(rng.choice([1, 2, 3, 5, 8, 13, 32, 64]))
        if R * epr <= 4096:
            break
    E = R * epr
    k = int(min(E, rng.choice([1, 2, 3, 4, 6, 8, 9, 16, 32])))
    T = int(rng.choice([0, 1, 2, 63, 64, 65, 129, 255, 256, 257, 400, 600]))
    cap = T + int(rng.choice([0, 1, 17, 100]))
    cap = max(cap, 1)
    mode = str(rng.choice(list(MODES)))
    quantising = mode in ("fp8", "mxfp4")
    H = int(rng.choice([128, 256, 384, 1152])) if mode in ("fp8", "mxfp4") else \
        int(rng.choice([32, 64, 160, 1024])) if mode == "fp4carry" else \
        int(rng.choice([16, 48, 256, 1040])) if mode == "fp8carry" else \
        int(rng.choice([8, 24, 264, 1024]))
    layout = str(rng.choice(["rank_major", "expert_major", "standard"]))
    fused = bool(rng.integers(0, 2))
    src_rank = int(rng.integers(0, R))
    sd = H // 128 if quantising else (int(rng.choice([0, 1, 5])) if "carry" in mode else 0)
    plant = bool(rng.integers(0, 3) == 0)
    # combine payload: bf16 rows, the E4M3 rounding in flight, or cast + E4M3 combine
    combine = str(rng.choice(["bf16", "inflight", "cast"])) if H % 16 == 0 else "bf16"
    return dict(R=R, epr=epr, k=k, T=T, cap=cap, mode=mode, H=H, layout=layout, fused=fused,
                src_rank=src_rank, sd=sd, plant=plant, combine=combine)


CASES = [draw(i) for i in range(200)]


def _label(c):
    return (f"{c['mode']}-{c['layout']}-R{c['R']}x{c['epr']}-k{c['k']}-T{c['T']}-H{c['H']}"
            f"{'-fused' if c['fused'] else ''}{'-plant' if c['plant'] else ''}-{c['combine']}")


def _inputs(c, seed):
    wl = Workload("rand", max(c["T"], 1), c["H"], c["R"], c["epr"], c["k"], c["cap"], "none",
                  "uniform", "identity", "rank_major")
    inp = make_inputs(wl, seed)
    T = c["T"]
    idx = inp["indices"][:T].copy()
    if c["plant"] and T > 2:
        idx[T // 2, 0] = c["R"] * c["epr"]        # out of range
        if c["k"] > 1:
            idx[T - 1, c["k"] - 1] = idx[T - 1, 0]  # repeated expert
    x, scales = inp["x"][:T], None
    if MODES[c["mode"]][2]:
        row_bytes = c["H"] // 2 if c["mode"] == "fp4carry" else c["H"]
        p = make_fp8_payload(max(T, 1), row_bytes, c["sd"], seed)
        x, scales = p["q"][:T], p["scales"][:T]
    return x, idx, inp["weights"][:T], scales


@pytest.mark.parametrize("c", CASES, ids=[_label(c) for c in CASES])
def test_random_config(c):
    print(f"[rand] {_label(c)}", flush=True)
    R, epr, k, T, cap, H = c["R"], c["epr"], c["k"], c["T"], c["cap"], c["H"]
    E = R * epr
    lib_mode, o_mode, _ = MODES[c["mode"]]
    sd = c["sd"]
    x, idx, w, scales = _inputs(c, 7)
    m = M.Mep(H, epr, k, cap, R, rank=c["src_rank"], quant=lib_mode, scale_dim=sd)
    byte_rows = c["mode"] != "bf16"
    rcols = H // 2 if c["mode"] in ("fp4carry", "mxfp4") else H
    rdt = torch.uint8 if byte_rows else torch.int16
    fill = SENT8 if byte_rows else SENT16 - 0x10000
    d_x = dev(x) if T else None
    d_idx = dev(idx) if T else None
    d_w = dev(w) if T else None
    d_s = dev(scales) if (T and scales is not None and sd) else None
    pl = O.plan(idx.reshape(T, k), R, epr, cap, c["src_rank"])
    cap_em = T * k + 127 * E

    if c["layout"] == "standard":
        emx = torch.full((max(cap_em, 1), rcols), fill, dtype=rdt, device="cuda")
        ems = torch.full((max(cap_em, 1), sd), float("nan"), device="cuda") if sd else None
        emc = torch.full((E,), SENT32, dtype=torch.int32, device="cuda")
        emo = torch.full((E + 1,), SENT32, dtype=torch.int32, device="cuda")
        emp = torch.full((max(cap_em, 1),), SENT32, dtype=torch.int32, device="cuda")
        M.mep_dispatch_standard_moe(m.h, d_idx, T, d_x, d_s, emx, ems, emc, emo, emp, cap_em)
        em = O.dispatch_standard_moe(x, w, idx.reshape(T, k), R, epr, cap, o_mode, cap_em,
                                     c["src_rank"], fill=fill & 0xFF, scales=scales)
        em_route = _check_em(c, em, emx, ems, emc, emo, emp, m, T, k, cap_em, byte_rows, sd)
        _combine_em(c, m, em, em_route, emx, w, T, H, cap_em, byte_rows)
        return

    counts = torch.full((R,), SENT32, dtype=torch.int32, device="cuda")
    spos = torch.full((R, cap), SENT32, dtype=torch.int32, device="cuda")
    rx = torch.full((R, cap, rcols), fill, dtype=rdt, device="cuda")
    rs = torch.full((R, cap, sd), float("nan"), device="cuda") if sd else None
    rw = torch.full((R, cap, k), float("nan"), device="cuda")
    ri = torch.full((R, cap, k), SENT32, dtype=torch.int32, device="cuda")
    if c["fused"]:
        M.mep_plan_dispatch(m.h, d_idx, T, counts, spos, d_x, d_w, d_s, rx, rs, rw, ri)
    else:
        M.mep_plan(m.h, d_idx, T, counts, spos)
        M.mep_dispatch(m.h, d_x, d_w, d_s, d_idx, rx, rs, rw, ri)
    d = O.dispatch(x, w, idx.reshape(T, k), pl, R, epr, cap, o_mode, fill=fill & 0xFF,
                   scales=scales)
    torch.cuda.synchronize()
    assert np.array_equal(host(counts), pl["recv_counts"])
    written = np.arange(cap)[None, :] < pl["recv_counts"][:, None]
    assert np.array_equal(host(spos)[written], pl["src_token_pos"][written])
    assert np.all(host(spos)[~written] == SENT32)
    gx = host(rx, np.uint8 if byte_rows else np.uint16)
    assert np.array_equal(gx, d["recv_x"]), "received rows differ"
    if sd:
        assert np.array_equal(host(rs)[written].view(np.uint32),
                              d["recv_scales"][written].view(np.uint32))
    assert np.array_equal(host(rw)[written].view(np.uint32), d["recv_weights"][written].view(np.uint32))
    assert np.array_equal(host(ri)[written], d["recv_indices"][written])
    assert M.mep_get_status(m.h) == pl["status"]
    route = torch.full((max(T, 1), k), SENT32, dtype=torch.int32, device="cuda")
    M.mep_get_route(m.h, route)
    ref_route = np.where(pl["slot"] >= 0, (idx.reshape(T, k) // epr) * cap + pl["slot"], -1)
    assert np.array_equal(host(route)[:T], ref_route)

    if c["layout"] == "expert_major":
        emx = torch.full((max(cap_em, 1), rcols), fill, dtype=rdt, device="cuda")
        ems = torch.full((max(cap_em, 1), sd), float("nan"), device="cuda") if sd else None
        emc = torch.full((E,), SENT32, dtype=torch.int32, device="cuda")
        emo = torch.full((E + 1,), SENT32, dtype=torch.int32, device="cuda")
        emp = torch.full((max(cap_em, 1),), SENT32, dtype=torch.int32, device="cuda")
        M.mep_to_expert_major(m.h, rx, rs, ri, counts, spos, emx, ems, emc, emo, emp, cap_em)
        em = O.to_expert_major(d, pl, R, epr, cap, T, cap_em, c["src_rank"], fill=fill & 0xFF)
        em["status"] |= pl["status"]
        em_route = _check_em(c, em, emx, ems, emc, emo, emp, m, T, k, cap_em, byte_rows, sd)
        _combine_em(c, m, em, em_route, emx, w, T, H, cap_em, byte_rows)
        return

    # rank-major combine on bf16 expert outputs derived from the received rows
    y_np = _outputs(d["recv_x"], byte_rows, H)
    out = _run_combine(c, m, M.MEP_RANK_MAJOR, y_np, d_w, T, H)
    ref = O.combine(_as_combined(c, y_np, written), w, idx.reshape(T, k), pl, epr, cap)
    torch.cuda.synchronize()
    if T:
        check_combine(host(out, np.uint16)[:T], ref)


def _run_combine(c, m, layout, y_np, d_w, T, H):
    """The configuration's combine call on bf16 expert outputs y_np."""
    y = dev(y_np)
    out = torch.empty((max(T, 1), H), dtype=torch.int16, device="cuda")
    if c["combine"] == "inflight":
        M.mep_combine_fp8_direct(m.h, layout, y, d_w, out)
    elif c["combine"] == "cast":
        y8 = torch.zeros(y.shape, dtype=torch.uint8, device="cuda")
        M.mep_cast_fp8_direct(m.h, layout, y, y8)
        M.mep_combine_fp8(m.h, layout, y8, d_w, out)
    else:
        M.mep_combine(m.h, layout, y, d_w, out)
    return out


def _as_combined(c, y_np, used):
    """The values the combine multiplies: y_np itself, or, with the E4M3
    payload, its direct cast decoded back (rows in `used` only)."""
    if c["combine"] == "bf16":
        return y_np
    y = np.zeros_like(y_np)
    y[used] = O.e4m3_to_bf16(O.cast_fp8_direct(y_np[used]))
    return y


def _outputs(rows, byte_rows, H):
    """bf16 expert outputs (harness): the rows themselves for bf16 payloads,
    otherwise a seeded function of the row bytes (finite bf16 values)."""
    if not byte_rows:
        return rows
    flat = rows.reshape(-1, rows.shape[-1]).astype(np.uint16)
    rep = np.repeat(flat, 2, axis=1) if flat.shape[1] * 2 == H else flat
    y = ((rep.astype(np.uint32) * 37 + 11) & 0x3FFF).astype(np.uint16) | 0x3C00  # [1, 4) range
    return y.reshape(rows.shape[:-1] + (H,))


def _check_em(c, em, emx, ems, emc, emo, emp, m, T, k, cap_em, byte_rows, sd):
    torch.cuda.synchronize()
    assert np.array_equal(host(emc), em["em_counts"])
    offs = host(emo)
    assert np.array_equal(offs, em["em_offsets"])
    used = np.zeros(max(cap_em, 1), bool)
    for e in range(c["R"] * c["epr"]):
        used[offs[e]:min(offs[e] + em["em_counts"][e], cap_em)] = True
    used = used[:cap_em]
    gx = host(emx, np.uint8 if byte_rows else np.uint16)[:cap_em]
    assert np.array_equal(gx[used], em["em_x"][used])
    sent = SENT8 if byte_rows else SENT16
    assert np.all(gx[~used] == sent), "padding rows written"
    if sd:
        assert np.array_equal(host(ems)[:cap_em][used].view(np.uint32),
                              em["em_scales"][used].view(np.uint32))
    gp = host(emp)[:cap_em]
    assert np.array_equal(gp[used], em["em_src_pos"][used])
    assert np.all(gp[~used] == SENT32)
    r = torch.full((max(T, 1), k), SENT32, dtype=torch.int32, device="cuda")
    M.mep_get_route(m.h, None, r)
    route = host(r)[:T]
    assert np.array_equal(route, em["tok_em_row"])
    assert M.mep_get_status(m.h) == em["status"]
    return route


def _combine_em(c, m, em, em_route, emx, w, T, H, cap_em, byte_rows):
    y_np = _outputs(em["em_x"], byte_rows, H)
    out = _run_combine(c, m, M.MEP_EXPERT_MAJOR, y_np, dev(w) if T else None, T, H)
    used = np.zeros(y_np.shape[0], bool)
    rows = em["tok_em_row"]
    used[rows[rows >= 0]] = True
    ref = O.combine_em(_as_combined(c, y_np, used), w, em["tok_em_row"])
    torch.cuda.synchronize()
    if T:
        check_combine(host(out, np.uint16)[:T], ref)
