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
