"""Host-side checks of the benchmark script (no GPU): the one-GPU rule, and the
algorithmic byte counts it prices the kernels with, recomputed here from the
buffer shapes they move."""

import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line for a run that did not happen


def test_byte_counts_match_the_buffers_they_move():
    T, H, k, U, R, E = 4096, 7168, 8, 21706, 8, 256
    f32, i32 = 4, 4
    # FP8 dispatch: bf16 rows + weights + ids in; per received row the E4M3 row,
    # its H/128 fp32 scales, k weights and k ids out
    fp8_row = np.zeros(H, np.uint8).nbytes + np.zeros(H // 128, np.float32).nbytes
    assert bench.dispatch_bytes(T, H, k, U, "fp8") == \
        T * H * 2 + T * k * (f32 + i32) + U * (fp8_row + k * (f32 + i32))
    # MXFP4: packed E2M1 (two a byte) + one E8M0 byte per 32 columns
    assert bench.row_bytes(H, "mxfp4") == H // 2 + H // 32
    assert bench.row_bytes(H, "none") == H * 2
    # combine: the U distinct bf16 rows + weights and ids read, T bf16 rows written
    assert bench.combine_bytes(T, H, k, U) == U * H * 2 + T * k * 8 + T * H * 2
    # expert-major combine: k rows per token
    assert bench.combine_em_bytes(T, H, k) == T * k * H * 2 + T * k * 8 + T * H * 2
    # plan: ids in, per-rank source positions and counts out
    assert bench.plan_bytes(T, k, R, U) == T * k * i32 + U * i32 + R * i32
    # standard-MoE dispatch writes each expert row, its scales and source once
    assert bench.standard_moe_bytes(T, H, k, E, T * k, "fp8") == \
        T * H * 2 + T * k * i32 + T * k * (fp8_row + i32) + E * 8
    # conversion back to rank rows: every expert-major row read with its
    # dispatched weight, the route of every (token, position) read, each rank
    # row written; their combine reads the rank rows and one route entry per
    # position, writes the tokens
    Uem = T * k
    assert bench.convert_combine_input_bytes(T, H, k, U, Uem) == \
        Uem * (H * 2 + f32) + T * k * 2 * i32 + U * H * 2
    assert bench.combine_rank_sum_bytes(T, H, k, U) == U * H * 2 + T * k * i32 + T * H * 2


def test_probe_mixes_split_each_operation_bytes_into_reads_and_writes():
    # the streaming-probe ceiling of an operation is taken at that operation's
    # own bytes: its read and write parts add up to the bytes it is priced with
    from synthetic import WORKLOADS
    U, Uem = 21706, 32768
    for name in ("skew", "stdmoe", "prefill_mxfp4", "prefill_fp8direct"):
        wl = WORKLOADS[name]
        T, H, k = wl.tokens, wl.hidden, wl.topk
        em, fp8c = wl.layout == "expert_major", wl.combine == "fp8_direct"
        want = {"dispatch": bench.dispatch_bytes(T, H, k, U, wl.quant)}
        if em:
            want.update(combine=bench.combine_em_bytes(T, H, k),
                        to_expert_major=bench.to_expert_major_bytes(T, H, k, U, wl.quant),
                        dispatch_standard_moe=bench.standard_moe_bytes(T, H, k, wl.experts, Uem,
                                                                       wl.quant),
                        convert_combine_input=bench.convert_combine_input_bytes(T, H, k, U, Uem),
                        combine_rank_sum=bench.combine_rank_sum_bytes(T, H, k, U))
        elif fp8c:
            want.update(cast_fp8_direct=bench.cast_fp8_bytes(H, U),
                        combine=bench.combine_fp8_bytes(T, H, k, U),
                        combine_in_flight=bench.combine_bytes(T, H, k, U))
        else:
            want.update(combine=bench.combine_bytes(T, H, k, U))
        mixes = bench.op_mixes(wl, U, Uem, wl.quant, em, fp8c)
        assert set(mixes) == set(want), name
        for op, (rd, wr) in mixes.items():
            assert rd > 0 and wr > 0 and rd + wr == want[op], (name, op)
