"""ctypes wrapper around the plain-C CPU oracle (mep_oracle.c).

TEST INFRASTRUCTURE: only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  It shares no code with the GPU
library and never loads it.

Every function takes and returns numpy arrays in the layouts the C file
documents; the arithmetic lives in the C file.
"""

from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mep_oracle.c")
_LIB = os.path.join(_HERE, "libmep_oracle.so")

ST_BAD_INDEX = 1
ST_DUP_EXPERT = 2
ST_EM_OVERFLOW = 4

GCC_FLAGS = ["-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
             "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no FMA contraction, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", *GCC_FLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = C.CDLL(_LIB)
        p = C.c_void_p
        i32, i64, f32 = C.c_int32, C.c_int64, C.c_float
        L.oracle_bf16_to_f32.argtypes, L.oracle_bf16_to_f32.restype = [C.c_uint16], f32
        L.oracle_bf16_rne.argtypes, L.oracle_bf16_rne.restype = [f32], C.c_uint16
        L.oracle_e4m3_decode.argtypes, L.oracle_e4m3_decode.restype = [C.c_uint8], C.c_double
        L.oracle_e4m3_encode.argtypes, L.oracle_e4m3_encode.restype = [f32], C.c_uint8
        L.oracle_e4m3_encode_array.argtypes = [p, i64, p]
        L.oracle_bf16_rne_array.argtypes = [p, i64, p]
        L.oracle_plan.argtypes = [p, i32, i32, i32, i32, i32, i32, p, p, p]
        L.oracle_plan.restype = i32
        L.oracle_quant_row.argtypes = [p, i32, p, p]
        L.oracle_e2m1_decode.argtypes, L.oracle_e2m1_decode.restype = [C.c_uint8], C.c_double
        L.oracle_e2m1_encode.argtypes, L.oracle_e2m1_encode.restype = [C.c_double], C.c_uint8
        L.oracle_mx4_quant_row.argtypes = [p, i32, p, p]
        L.oracle_mx4_decode_row.argtypes = [p, p, i32, p]
        L.oracle_cast_fp8_direct.argtypes = [p, i64, p]
        L.oracle_dispatch.argtypes = [p, p, i32, p, p, p, i32, i32, i32, i32, i32, i32, i32,
                                      p, p, p, p, p, p]
        L.oracle_combine.argtypes = [p, p, p, p, i32, i32, i32, i32, i32, p]
        L.oracle_to_expert_major.argtypes = [p, p, p, p, p, i32, i32, i32, i32, i32, i32,
                                             i32, i32, i32, i64, p, p, p, p, p, p]
        L.oracle_to_expert_major.restype = i32
        L.oracle_combine_em.argtypes = [p, p, p, i32, i32, i32, p]
        L.oracle_expert_dequant.argtypes = [p, p, i64, i32, f32, p]
        L.oracle_convert_combine_input.argtypes = [p, i64, p, p, p, p, p, p, p, i32, i32, i32,
                                                   i32, i32, p, p]
        L.oracle_combine_rank_sum.argtypes = [p, p, p, i32, i32, i32, i32, i32, p, p]
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(C.c_void_p)


# --- codecs -------------------------------------------------------------------

def bf16_rne(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint16)
    lib().oracle_bf16_rne_array(_p(v), v.size, _p(out))
    return out


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint8)
    lib().oracle_e4m3_encode_array(_p(v), v.size, _p(out))
    return out


def e4m3_decode_table() -> np.ndarray:
    return np.array([lib().oracle_e4m3_decode(c) for c in range(256)], dtype=np.float64)


def quant_row(x_row: np.ndarray):
    x_row = np.ascontiguousarray(x_row, dtype=np.uint16)
    H = x_row.shape[0]
    q = np.empty(H, dtype=np.uint8)
    s = np.empty(H // 128, dtype=np.float32)
    lib().oracle_quant_row(_p(x_row), H, _p(q), _p(s))
    return q, s


def e2m1_decode_table() -> np.ndarray:
    return np.array([lib().oracle_e2m1_decode(c) for c in range(16)], dtype=np.float64)


def e2m1_encode(v: float) -> int:
    return int(lib().oracle_e2m1_encode(float(v)))


def mx4_quant_row(x_row: np.ndarray):
    """Reading R11 for one bf16 row: (packed codes [H/2] uint8, scale bytes [H/32])."""
    x_row = np.ascontiguousarray(x_row, dtype=np.uint16)
    H = x_row.shape[0]
    q = np.empty(H // 2, dtype=np.uint8)
    e8 = np.empty(H // 32, dtype=np.uint8)
    lib().oracle_mx4_quant_row(_p(x_row), H, _p(q), _p(e8))
    return q, e8


def mx4_decode_row(q: np.ndarray, e8: np.ndarray) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.uint8)
    e8 = np.ascontiguousarray(e8, dtype=np.uint8)
    H = 2 * q.shape[0]
    out = np.empty(H, dtype=np.float64)
    lib().oracle_mx4_decode_row(_p(q), _p(e8), H, _p(out))
    return out


def cast_fp8_direct(y_bits: np.ndarray) -> np.ndarray:
    """Reading R12: E4M3 codes of bf16 values, no scale."""
    y = np.ascontiguousarray(y_bits, dtype=np.uint16)
    out = np.empty(y.shape, dtype=np.uint8)
    lib().oracle_cast_fp8_direct(_p(y), y.size, _p(out))
    return out


def e4m3_to_bf16(codes: np.ndarray) -> np.ndarray:
    """bf16 bits of E4M3 values (every E4M3 value is a bf16 value, so this is
    exact); lets the combine run on direct-cast rows."""
    tab = e4m3_decode_table().astype(np.float32)
    f = np.ascontiguousarray(tab[np.asarray(codes, dtype=np.uint8)])
    out = np.empty(f.shape, dtype=np.uint16)
    lib().oracle_bf16_rne_array(_p(f), f.size, _p(out))
    return out


# --- the path -----------------------------------------------------------------

def plan(indices: np.ndarray, R: int, epr: int, cap: int, src_rank: int = 0) -> dict:
    idx = np.ascontiguousarray(indices, dtype=np.int32)
    T, k = idx.shape
    counts = np.zeros(R, dtype=np.int32)
    spos = np.full((R, cap), -1, dtype=np.int32)
    slot = np.empty((T, k), dtype=np.int32)
    st = lib().oracle_plan(_p(idx), T, k, R, epr, cap, src_rank, _p(counts), _p(spos), _p(slot))
    return {"recv_counts": counts, "src_token_pos": spos, "slot": slot, "status": int(st)}


def dispatch(x: np.ndarray, weights: np.ndarray, indices: np.ndarray, pl: dict, R: int,
             epr: int, cap: int, quant, fill: int = 0, scales: np.ndarray | None = None) -> dict:
    """quant: 0/False bf16 copy, 1/True FP8 block quantisation, 2 FP8 carry (x
    holds E4M3 bytes [T,H], scales [T,sd] 32-bit words), 3 FP4 carry (x holds
    packed E2M1 bytes [T,H/2], scales [T,sd]), 4 MXFP4 quantisation (reading
    R11).  Returns recv_x ([R,cap,H] uint16 bf16 bits, [R,cap,H] uint8 E4M3
    codes, or [R,cap,H/2] uint8 packed E2M1), recv_scales ([R,cap,nb] float32
    words, or None), recv_weights, recv_indices.  Unwritten rows keep ``fill``
    (bytes) so callers can see which rows were written."""
    quant = int(quant)
    x = np.ascontiguousarray(x, dtype=np.uint8 if quant in (2, 3) else np.uint16)
    w = np.ascontiguousarray(weights, dtype=np.float32)
    idx = np.ascontiguousarray(indices, dtype=np.int32)
    T, H = x.shape
    if quant == 3:
        H *= 2  # two E2M1 codes per byte
    k = idx.shape[1]
    if quant in (2, 3):
        xs = np.ascontiguousarray(scales if scales is not None else np.zeros((T, 0)),
                                  dtype=np.float32)
        nb = xs.shape[1]
    else:
        xs = np.zeros(1, dtype=np.float32)
        nb = H // 128 if quant in (1, 4) else 0
    if quant:
        rx = np.full((R, cap, H // 2 if quant >= 3 else H), fill, dtype=np.uint8)
        rs = np.zeros((R, cap, max(nb, 1)), dtype=np.float32)
    else:
        rx = np.full((R, cap, H), fill * 0x0101, dtype=np.uint16)
        rs = np.zeros(1, dtype=np.float32)
    rw = np.zeros((R, cap, k), dtype=np.float32)
    ri = np.full((R, cap, k), -1, dtype=np.int32)
    qt = np.empty(H, dtype=np.uint8)
    st = np.empty(max(nb, H // 128, 1), dtype=np.float32)
    lib().oracle_dispatch(_p(x), _p(xs), nb, _p(w), _p(idx), _p(pl["slot"]), T, H, k, R, epr,
                          cap, quant, _p(rx), _p(rs), _p(rw), _p(ri), _p(qt), _p(st))
    return {"recv_x": rx, "recv_scales": rs if nb else None, "recv_weights": rw,
            "recv_indices": ri}


def dispatch_standard_moe(x: np.ndarray, weights: np.ndarray, indices: np.ndarray, R: int,
                          epr: int, cap: int, quant, cap_em: int, src_rank: int = 0,
                          fill: int = 0, scales: np.ndarray | None = None) -> dict:
    """Standard-MoE dispatch, reading R10: plan, dispatch and the expert-major
    conversion one after the other."""
    pl = plan(indices, R, epr, cap, src_rank)
    disp = dispatch(x, weights, indices, pl, R, epr, cap, quant, fill=fill, scales=scales)
    em = to_expert_major(disp, pl, R, epr, cap, indices.shape[0], cap_em, src_rank, fill=fill)
    em["status"] |= pl["status"]
    return em


def combine(y: np.ndarray, weights: np.ndarray, indices: np.ndarray, pl: dict, epr: int,
            cap: int) -> np.ndarray:
    y = np.ascontiguousarray(y, dtype=np.uint16)
    w = np.ascontiguousarray(weights, dtype=np.float32)
    idx = np.ascontiguousarray(indices, dtype=np.int32)
    T, k = idx.shape
    H = y.shape[-1]
    out = np.empty((T, H), dtype=np.uint16)
    lib().oracle_combine(_p(y), _p(w), _p(idx), _p(pl["slot"]), T, H, k, epr, cap, _p(out))
    return out


def to_expert_major(disp: dict, pl: dict, R: int, epr: int, cap: int, T: int, cap_em: int,
                    src_rank: int = 0, fill: int = 0) -> dict:
    rx = np.ascontiguousarray(disp["recv_x"])
    elem = rx.dtype.itemsize
    H = rx.shape[-1]
    rs = disp["recv_scales"]
    nb = 0 if rs is None else rs.shape[-1]
    ri = np.ascontiguousarray(disp["recv_indices"], dtype=np.int32)
    k = ri.shape[-1]
    E = R * epr
    em_x = np.full((cap_em, H), fill * (0x0101 if elem == 2 else 1), dtype=rx.dtype)
    em_s = np.zeros((cap_em, max(nb, 1)), dtype=np.float32)
    em_counts = np.zeros(E, dtype=np.int32)
    em_offsets = np.zeros(E + 1, dtype=np.int32)
    em_src = np.full(cap_em, -1, dtype=np.int32)
    tok = np.empty((T, k), dtype=np.int32)
    rs_arr = np.ascontiguousarray(rs if rs is not None else np.zeros(1, np.float32))
    st = lib().oracle_to_expert_major(_p(rx), _p(rs_arr), _p(ri), _p(pl["recv_counts"]),
                                      _p(pl["src_token_pos"]), R, epr, cap, H, nb, k, elem,
                                      src_rank, T, cap_em, _p(em_x), _p(em_s), _p(em_counts),
                                      _p(em_offsets), _p(em_src), _p(tok))
    return {"em_x": em_x, "em_scales": em_s if nb else None, "em_counts": em_counts,
            "em_offsets": em_offsets, "em_src_pos": em_src, "tok_em_row": tok,
            "status": int(st)}


def combine_em(y_em: np.ndarray, weights: np.ndarray, tok_em_row: np.ndarray) -> np.ndarray:
    y_em = np.ascontiguousarray(y_em, dtype=np.uint16)
    w = np.ascontiguousarray(weights, dtype=np.float32)
    tok = np.ascontiguousarray(tok_em_row, dtype=np.int32)
    T, k = tok.shape
    H = y_em.shape[-1]
    out = np.empty((T, H), dtype=np.uint16)
    lib().oracle_combine_em(_p(y_em), _p(w), _p(tok), T, H, k, _p(out))
    return out


def convert_combine_input(y_em: np.ndarray, em: dict, disp: dict, pl: dict, R: int, epr: int,
                          cap: int, fill: int = 0) -> np.ndarray:
    """Reading R21: expert-major expert outputs y_em ([cap_em,H] bf16 bits, in
    the layout `em` describes) back to one bf16 row per received row,
    [R,cap,H]; each row is its rank's experts' outputs weighted by the
    dispatched weights (disp["recv_weights"]).  Rows past the counts keep
    ``fill``."""
    y_em = np.ascontiguousarray(y_em, dtype=np.uint16)
    cap_em, H = y_em.shape
    rw = np.ascontiguousarray(disp["recv_weights"], dtype=np.float32)
    ri = np.ascontiguousarray(disp["recv_indices"], dtype=np.int32)
    k = ri.shape[-1]
    out = np.full((R, cap, H), fill, dtype=np.uint16)
    tmp = np.empty(k, dtype=np.int64)
    lib().oracle_convert_combine_input(
        _p(y_em), cap_em, _p(np.ascontiguousarray(em["em_counts"], dtype=np.int32)),
        _p(np.ascontiguousarray(em["em_offsets"], dtype=np.int32)),
        _p(np.ascontiguousarray(em["em_src_pos"], dtype=np.int32)), _p(rw), _p(ri),
        _p(np.ascontiguousarray(pl["recv_counts"], dtype=np.int32)),
        _p(np.ascontiguousarray(pl["src_token_pos"], dtype=np.int32)), R, epr, cap, H, k,
        _p(out), _p(tmp))
    return out


def combine_rank_sum(y_rm: np.ndarray, indices: np.ndarray, pl: dict, epr: int,
                     cap: int) -> np.ndarray:
    """Reading R21: combine of converted rows -- each token's distinct rank
    rows added in fp32 in the order of their first top-k position, no
    weights, then bf16."""
    y_rm = np.ascontiguousarray(y_rm, dtype=np.uint16)
    idx = np.ascontiguousarray(indices, dtype=np.int32)
    T, k = idx.shape
    H = y_rm.shape[-1]
    out = np.empty((T, H), dtype=np.uint16)
    tmp = np.empty(k, dtype=np.int64)
    lib().oracle_combine_rank_sum(_p(y_rm), _p(idx), _p(np.ascontiguousarray(pl["slot"])), T, H,
                                  k, epr, cap, _p(out), _p(tmp))
    return out


def expert_dequant(q: np.ndarray, scales: np.ndarray, mult: float) -> np.ndarray:
    """Expert stand-in for FP8 payloads: bf16((decode(q) * scale) * mult)."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    H = q.shape[-1]
    rows = q.size // H
    s = np.ascontiguousarray(scales, dtype=np.float32)
    y = np.empty(q.shape, dtype=np.uint16)
    lib().oracle_expert_dequant(_p(q), _p(s), rows, H, mult, _p(y))
    return y
