"""The entry point that allocates nothing (mep_plan_dispatch_noalloc) against
the existing fused plan+dispatch (mep_plan_dispatch, handle and workspace),
through the C ABI: two calls in a row, the second with a smaller batch, every
output bit-exact (counts, source positions, receive rows, scales, weights,
ids; unwritten rows keep their sentinel on both sides).  The oracle checks the
existing entry point's side as well."""

import numpy as np
import pytest
import torch

import combine_mep_plan_amd as M
from synthetic import Workload, make_inputs

from _gpu_harness import (GpuResult, alloc_recv, check_plan_dispatch, dev, gpu_plan_dispatch, host,
                          oracle_plan_dispatch)

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _noalloc(wl, inp, src_rank=0):
    T = inp["indices"].shape[0]
    nb = wl.hidden // 128 if wl.quant == "fp8" else 0
    cfg = M.MepConfig(wl.hidden, nb, wl.experts_per_rank, wl.topk, wl.cap, wl.ranks, src_rank,
                      M.MEP_QUANT_FP8_E4M3_BLOCK128 if wl.quant == "fp8" else M.MEP_QUANT_NONE)
    x, w, idx = dev(inp["x"]), dev(inp["weights"]), dev(inp["indices"])
    counts = torch.full((wl.ranks,), -0x5A5A5A5B, dtype=torch.int32, device="cuda")
    spos = torch.full((wl.ranks, wl.cap), -0x5A5A5A5B, dtype=torch.int32, device="cuda")
    recv = alloc_recv(wl)
    M.mep_plan_dispatch_noalloc(cfg, idx, T, counts, spos, x, w, None, *recv)
    torch.cuda.synchronize()
    return counts, spos, recv


def _same(a, b, what):
    if a is None:
        assert b is None
        return
    ha, hb = host(a), host(b)
    assert np.array_equal(ha.view(np.uint8), hb.view(np.uint8)), what


@pytest.mark.parametrize("quant,T1,T2,src", [("fp8", 4096, 700, 0), ("none", 3000, 130, 2),
                                             ("fp8", 1000, 1, 1)])
def test_noalloc_matches_plan_dispatch_twice(quant, T1, T2, src):
    for i, T in enumerate((T1, T2)):
        wl = Workload("na", T, 1024, 8, 32, 8, 4096, quant, "uniform", "dequant_half",
                      "rank_major")
        inp = make_inputs(wl, 50 + i)
        _say(f"no-alloc call {i}: T={T} {quant} src_rank={src}")
        counts, spos, recv = _noalloc(wl, inp, src)
        g = gpu_plan_dispatch(wl, inp, src_rank=src, fused=True)
        _same(counts, g.counts, "recv_counts")
        _same(spos, g.spos, "src_token_pos")
        for name, a, b in zip(("recv_x", "recv_scales", "recv_weights", "recv_indices"), recv,
                              (g.recv_x, g.recv_s, g.recv_w, g.recv_i)):
            _same(a, b, name)
        pl, d = oracle_plan_dispatch(wl, inp, src)
        check_plan_dispatch(wl, inp, g, pl, d)

