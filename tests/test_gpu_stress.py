"""GPU stress: many rounds of the whole path compared with verified results.

Like the pages' check of tuned configurations (many rounds of dispatch and
combine output against expected values; "MORI-EP User Guide", section 10
Tuning), 500 rounds of fused plan +
FP8 dispatch + combine + reset run back to back over four input sets with
different routings and token counts.  The first round of each set is checked
against the oracle; every later round must reproduce it bit for bit (the
comparison runs on the device, so the rounds stay back to back).  A race in
the scans or a stale status epoch would show as a mismatch or a status bit.
"""

import dataclasses

import numpy as np
import pytest
import torch

import combine_mep_plan_amd as M
from oracle import oracle as O
from synthetic import WORKLOADS, make_inputs

from _gpu_harness import check_combine, dev, host

pytestmark = pytest.mark.gpu

ROUNDS = 500


def test_500_rounds_bitwise_stable():
    base = dataclasses.replace(WORKLOADS["prefill"], hidden=1024, cap=1024)
    Ts = [1024, 700, 257, 64]  # several fused-path shapes: two launches, one launch
    m = M.Mep(base.hidden, base.experts_per_rank, base.topk, base.cap, base.ranks, fp8=True)
    R, cap, H, k, epr = base.ranks, base.cap, base.hidden, base.topk, base.experts_per_rank
    sets = []
    for i, T in enumerate(Ts):
        wl = base.with_tokens(T, cap=cap)
        inp = make_inputs(wl, 100 + i)
        pl = O.plan(inp["indices"], R, epr, cap)
        d = O.dispatch(inp["x"], inp["weights"], inp["indices"], pl, R, epr, cap, True)
        y_np = O.expert_dequant(d["recv_x"], d["recv_scales"], 0.5)
        ref = O.combine(y_np, inp["weights"], inp["indices"], pl, epr, cap)
        s = {"T": T, "x": dev(inp["x"]), "w": dev(inp["weights"]), "idx": dev(inp["indices"]),
             "y": dev(y_np), "ref": ref, "pl": pl,
             "counts": torch.empty(R, dtype=torch.int32, device="cuda"),
             "spos": torch.empty((R, cap), dtype=torch.int32, device="cuda"),
             "rx": torch.empty((R, cap, H), dtype=torch.uint8, device="cuda"),
             "rs": torch.empty((R, cap, H // 128), dtype=torch.float32, device="cuda"),
             "rw": torch.empty((R, cap, k), dtype=torch.float32, device="cuda"),
             "ri": torch.empty((R, cap, k), dtype=torch.int32, device="cuda"),
             "out": torch.empty((T, H), dtype=torch.int16, device="cuda")}
        sets.append(s)

    def run(s):
        M.mep_plan_dispatch(m.h, s["idx"], s["T"], s["counts"], s["spos"], s["x"], s["w"], None,
                            s["rx"], s["rs"], s["rw"], s["ri"])
        M.mep_combine(m.h, M.MEP_RANK_MAJOR, s["y"], s["w"], s["out"])

    # first round of each set: against the oracle, then frozen as the expected bits
    for s in sets:
        run(s)
        assert M.mep_get_status(m.h) == 0
        torch.cuda.synchronize()
        assert np.array_equal(host(s["counts"]), s["pl"]["recv_counts"])
        check_combine(host(s["out"], np.uint16), s["ref"])
        s["exp_out"] = s["out"].clone()
        s["exp_counts"] = s["counts"].clone()
        n = s["pl"]["recv_counts"]
        s["mask"] = torch.from_numpy(np.arange(cap)[None, :] < n[:, None]).cuda()
        s["exp_rx"] = s["rx"].clone()
        M.mep_reset(m.h)
    bad = torch.zeros((), dtype=torch.int64, device="cuda")
    for i in range(ROUNDS):
        s = sets[i % len(sets)]
        run(s)
        # device-side comparison, accumulated without a host round trip
        bad += (s["out"] != s["exp_out"]).sum()
        bad += (s["counts"] != s["exp_counts"]).sum()
        bad += ((s["rx"] != s["exp_rx"]) & s["mask"][:, :, None]).sum()
        if i % 100 == 99:  # the epoch's sticky status, before the reset clears it
            assert M.mep_get_status(m.h) == 0
            print(f"[stress] {i + 1} rounds, mismatches {int(bad.item())}", flush=True)
        M.mep_reset(m.h)
    torch.cuda.synchronize()
    assert int(bad.item()) == 0
    assert M.mep_get_status(m.h) == 0


SEQS = ("fused_rank_major", "separate_expert_major", "standard_expert_major", "fused_direct")
MIXED_ROUNDS = 480  # 40 passes over every (input set, call sequence) pair


def test_mixed_call_sequences_bitwise_stable():
    """One handle drives four call sequences in turn over three input sets:
    fused plan+dispatch -> rank-major combine; plan -> dispatch -> expert-major
    conversion -> expert-major combine; standard-MoE dispatch -> expert-major
    combine; fused plan+dispatch -> combine with the E4M3 rounding in flight.
    Each (set, sequence) pair is checked against the oracle the first time and
    must then reproduce its bits every time it comes round again, so a stale
    plan, status epoch or scratch area left by a different sequence shows up."""
    base = dataclasses.replace(WORKLOADS["prefill"], hidden=512, cap=1024)
    Ts = [1024, 300, 64]
    R, cap, H, k, epr = base.ranks, base.cap, base.hidden, base.topk, base.experts_per_rank
    cap_em = base.with_tokens(max(Ts), cap=cap).cap_em
    m = M.Mep(H, epr, k, cap, R, fp8=True)
    sets = []
    for i, T in enumerate(Ts):
        wl = base.with_tokens(T, cap=cap)
        inp = make_inputs(wl, 200 + i)
        pl = O.plan(inp["indices"], R, epr, cap)
        d = O.dispatch(inp["x"], inp["weights"], inp["indices"], pl, R, epr, cap, True)
        em = O.to_expert_major(d, pl, R, epr, cap, T, cap_em)
        y_rm = O.expert_dequant(d["recv_x"], d["recv_scales"], 1.0)
        y_em = O.expert_dequant(em["em_x"], em["em_scales"], 1.0)
        used = np.arange(cap)[None, :] < pl["recv_counts"][:, None]  # [R, cap]
        y8 = np.zeros(y_rm.shape, dtype=np.uint8)
        y8[used] = O.cast_fp8_direct(y_rm[used])
        refs = {
            "fused_rank_major": O.combine(y_rm, inp["weights"], inp["indices"], pl, epr, cap),
            "separate_expert_major": O.combine_em(y_em, inp["weights"], em["tok_em_row"]),
            "fused_direct": O.combine(O.e4m3_to_bf16(y8), inp["weights"], inp["indices"], pl,
                                      epr, cap),
        }
        refs["standard_expert_major"] = refs["separate_expert_major"]
        z = lambda shape, dt: torch.zeros(shape, dtype=dt, device="cuda")  # noqa: E731
        s = {"T": T, "x": dev(inp["x"]), "w": dev(inp["weights"]), "idx": dev(inp["indices"]),
             "y_rm": dev(y_rm), "y_em": dev(y_em), "refs": refs,
             "ref_counts": pl["recv_counts"], "ref_em_counts": em["em_counts"],
             "counts": z(R, torch.int32), "spos": z((R, cap), torch.int32),
             "rx": z((R, cap, H), torch.uint8), "rs": z((R, cap, H // 128), torch.float32),
             "rw": z((R, cap, k), torch.float32), "ri": z((R, cap, k), torch.int32),
             "emx": z((cap_em, H), torch.uint8), "ems": z((cap_em, H // 128), torch.float32),
             "emc": z(R * epr, torch.int32), "emo": z(R * epr + 1, torch.int32),
             "emp": z(cap_em, torch.int32),
             "out": {q: z((T, H), torch.int16) for q in SEQS}}
        sets.append(s)

    def run(s, seq):
        T = s["T"]
        rm = (s["rx"], s["rs"], s["rw"], s["ri"])
        if seq in ("fused_rank_major", "fused_direct"):
            M.mep_plan_dispatch(m.h, s["idx"], T, s["counts"], s["spos"], s["x"], s["w"], None,
                                *rm)
        elif seq == "separate_expert_major":
            M.mep_plan(m.h, s["idx"], T, s["counts"], s["spos"])
            M.mep_dispatch(m.h, s["x"], s["w"], None, s["idx"], *rm)
            M.mep_to_expert_major(m.h, s["rx"], s["rs"], s["ri"], s["counts"], s["spos"],
                                  s["emx"], s["ems"], s["emc"], s["emo"], s["emp"], cap_em)
        else:
            M.mep_dispatch_standard_moe(m.h, s["idx"], T, s["x"], None, s["emx"], s["ems"],
                                        s["emc"], s["emo"], s["emp"], cap_em)
        out = s["out"][seq]
        if seq == "fused_rank_major":
            M.mep_combine(m.h, M.MEP_RANK_MAJOR, s["y_rm"], s["w"], out)
        elif seq == "fused_direct":
            M.mep_combine_fp8_direct(m.h, M.MEP_RANK_MAJOR, s["y_rm"], s["w"], out)
        else:
            M.mep_combine(m.h, M.MEP_EXPERT_MAJOR, s["y_em"], s["w"], out)
        return out, (s["counts"] if seq.startswith("fused") else s["emc"])

    expected = {}
    bad = torch.zeros((), dtype=torch.int64, device="cuda")
    for i in range(MIXED_ROUNDS):
        si, seq = i % len(sets), SEQS[(i // len(sets)) % len(SEQS)]
        s = sets[si]
        out, cnt = run(s, seq)
        if (si, seq) not in expected:  # first time: against the oracle, then frozen
            assert M.mep_get_status(m.h) == 0
            check_combine(host(out, np.uint16), s["refs"][seq])
            ref_cnt = s["ref_counts"] if seq.startswith("fused") else s["ref_em_counts"]
            assert np.array_equal(host(cnt), ref_cnt), (si, seq)
            expected[(si, seq)] = (out.clone(), cnt.clone())
        else:
            e_out, e_cnt = expected[(si, seq)]
            bad += (out != e_out).sum() + (cnt != e_cnt).sum()
        if i % 120 == 119:
            assert M.mep_get_status(m.h) == 0
            print(f"[stress] {i + 1} mixed rounds, mismatches {int(bad.item())}", flush=True)
        M.mep_reset(m.h)
    torch.cuda.synchronize()
    assert len(expected) == len(sets) * len(SEQS)
    assert int(bad.item()) == 0
    assert M.mep_get_status(m.h) == 0
