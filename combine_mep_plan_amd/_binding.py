"""ctypes marshalling for libmep.so: one Python function per C entry point,
same names, same argument order.  Tensors are passed as their device
pointers; ``stream=None`` means torch's current stream on the tensors'
device.  Non-zero return codes raise MepError (except mep_get_status, which
returns the device status word)."""

from __future__ import annotations

import ctypes as C
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmep.so")

MEP_OK = 0
MEP_ERR_NULL = -1
MEP_ERR_CONFIG = -2
MEP_ERR_SHAPE = -3
MEP_ERR_ALIGN = -4
MEP_ERR_STATE = -5
MEP_ERR_HIP = -6
MEP_ERR_DEVICE = -7
MEP_ERR_NOMEM = -8

MEP_DEV_BAD_INDEX = 1
MEP_DEV_DUP_EXPERT = 2
MEP_DEV_EM_OVERFLOW = 4

MEP_QUANT_NONE = 0
MEP_QUANT_FP8_E4M3_BLOCK128 = 1
MEP_QUANT_FP8_CARRY = 2
MEP_QUANT_FP4_CARRY = 3
MEP_QUANT_MXFP4 = 4
MEP_RANK_MAJOR = 0
MEP_EXPERT_MAJOR = 1
MEP_RANK_SUM = 2


class MepConfig(C.Structure):
    _fields_ = [
        ("hidden_dim", C.c_int32),
        ("scale_dim", C.c_int32),
        ("num_experts_per_rank", C.c_int32),
        ("num_experts_per_token", C.c_int32),
        ("max_num_inp_token_per_rank", C.c_int32),
        ("world_size", C.c_int32),
        ("rank", C.c_int32),
        ("quant", C.c_int32),
    ]


class MepError(RuntimeError):
    def __init__(self, fn: str, code: int):
        self.code = code
        super().__init__(f"{fn}: {mep_error_string(code)} ({code})")


_lib = None


def lib() -> C.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m combine_mep_plan_amd.build` (there is no fallback)")
        L = C.CDLL(LIB_PATH)
        p, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
        cfgp = C.POINTER(MepConfig)
        sig = {
            "mep_error_string": ([C.c_int], C.c_char_p),
            "mep_workspace_bytes": ([cfgp], sz),
            "mep_create": ([cfgp, p, sz, C.POINTER(p)], C.c_int),
            "mep_destroy": ([p], C.c_int),
            "mep_plan": ([p, p, i32, p, p, p], C.c_int),
            "mep_dispatch": ([p, p, p, p, p, p, p, p, p, p], C.c_int),
            "mep_plan_dispatch": ([p, p, i32, p, p, p, p, p, p, p, p, p, p], C.c_int),
            "mep_plan_dispatch_noalloc": ([cfgp, p, i32, p, p, p, p, p, p, p, p, p, p],
                                          C.c_int),
            "mep_dispatch_standard_moe": ([p, p, i32, p, p, p, p, p, p, p, i64, p], C.c_int),
            "mep_to_expert_major": ([p, p, p, p, p, p, p, p, p, p, p, i64, p], C.c_int),
            "mep_combine": ([p, i32, p, p, p, p], C.c_int),
            "mep_combine_fp8": ([p, i32, p, p, p, p], C.c_int),
            "mep_combine_fp8_direct": ([p, i32, p, p, p, p], C.c_int),
            "mep_cast_fp8_direct": ([p, i32, p, p, p], C.c_int),
            "mep_convert_combine_input": ([p, p, p, p, p], C.c_int),
            "mep_reset": ([p, p], C.c_int),
            "mep_get_status": ([p, p, C.POINTER(i32)], C.c_int),
            "mep_get_route": ([p, p, p, p], C.c_int),
            "mep_probe_e4m3": ([p, p, i64, p], C.c_int),
            "mep_probe_bf16": ([p, p, i64, p], C.c_int),
            "mep_probe_mxfp4": ([p, p, p, i64, p], C.c_int),
            "mep_probe_fp8_block": ([p, p, p, i64, p], C.c_int),
            "mep_probe_stream": ([p, p, i64, i64, i64, p], C.c_int),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes, f.restype = args, res
        _lib = L
    return _lib


def _ptr(t):
    """Device pointer of a tensor (must be contiguous and on a GPU), an int
    (taken as a device address), or None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("tensors passed to libmep must be on the GPU (a host pointer "
                         "would make the kernels fault)")
    if not t.is_contiguous():
        raise ValueError("tensors passed to libmep must be contiguous")
    return t.data_ptr()


def _stream(stream, *tensors):
    """The HIP stream to launch on: the one given, else torch's current stream
    on the device of the first GPU tensor (the current device if none).  The
    raw-handle query takes ~0.1 us against ~2.5 us for building a Stream
    object, a fifth of a decode call's host time."""
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    dev = next((d for d in (t.get_device() for t in tensors if hasattr(t, "get_device"))
                if d >= 0), None)
    if dev is None:
        dev = torch.cuda.current_device()
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None:
        return raw(dev)
    return torch.cuda.current_stream(dev).cuda_stream


def _check(fn: str, rc: int) -> None:
    if rc != MEP_OK:
        raise MepError(fn, rc)


# ---------------------------------------------------------------------------
# buffer sizes.  The C ABI trusts the caller's buffer sizes (a short buffer
# would be written past its end on the GPU); for handles made here, the
# binding checks every tensor against the sizes the call will touch, using the
# handle's config and the token count of its last plan.
# ---------------------------------------------------------------------------

# handle -> {"cfg": MepConfig, "T": planned tokens, "cap_em": rows, "rm"/"em": whether
# the rank-major plan / the expert-major layout is valid (the library's call
# order, mirrored so that a call the library will refuse is not size-checked)
_handles: dict = {}


def _row_bytes_in(c) -> int:
    """Bytes of one token row the dispatch reads."""
    return {MEP_QUANT_FP8_CARRY: c.hidden_dim, MEP_QUANT_FP4_CARRY: c.hidden_dim // 2}.get(
        c.quant, 2 * c.hidden_dim)


def _row_bytes_out(c) -> int:
    """Bytes of one received (or expert-major) row."""
    if c.quant == MEP_QUANT_NONE:
        return 2 * c.hidden_dim
    if c.quant in (MEP_QUANT_MXFP4, MEP_QUANT_FP4_CARRY):
        return c.hidden_dim // 2
    return c.hidden_dim


_INT32 = {"indices", "recv_counts", "src_token_pos", "recv_indices", "em_counts",
          "em_offsets", "em_src_pos", "recv_row", "em_row"}
_FLOAT32 = {"weights", "recv_weights"}  # scale buffers hold opaque 32-bit words in some modes


def _need(fn: str, name: str, t, nbytes: int) -> None:
    if t is None or isinstance(t, int):
        return
    import torch
    want = torch.int32 if name in _INT32 else torch.float32 if name in _FLOAT32 else None
    if want is not None and t.dtype != want:
        raise ValueError(f"{fn}: {name} must be {want}, not {t.dtype}")
    if nbytes <= 0:
        return
    have = t.nbytes
    if have < nbytes:
        raise ValueError(f"{fn}: {name} holds {have} bytes, the call touches {nbytes}")


def _state(h):
    return _handles.get(h)


def _check_plan_buffers(fn, st, indices, T, recv_counts, src_token_pos):
    c = st["cfg"]
    _need(fn, "indices", indices, 4 * T * c.num_experts_per_token)
    _need(fn, "recv_counts", recv_counts, 4 * c.world_size)
    _need(fn, "src_token_pos", src_token_pos, 4 * c.world_size * c.max_num_inp_token_per_rank)


def _check_dispatch_buffers(fn, st, T, x, weights, scales, indices, recv_x, recv_scales,
                            recv_weights, recv_indices):
    c = st["cfg"]
    k, rows = c.num_experts_per_token, c.world_size * c.max_num_inp_token_per_rank
    sd = c.scale_dim if c.quant != MEP_QUANT_NONE else 0
    _need(fn, "x", x, T * _row_bytes_in(c))
    _need(fn, "weights", weights, 4 * T * k)
    _need(fn, "indices", indices, 4 * T * k)
    if c.quant in (MEP_QUANT_FP8_CARRY, MEP_QUANT_FP4_CARRY):
        _need(fn, "scales", scales, 4 * T * sd)
    _need(fn, "recv_x", recv_x, rows * _row_bytes_out(c))
    _need(fn, "recv_scales", recv_scales, 4 * rows * sd)
    _need(fn, "recv_weights", recv_weights, 4 * rows * k)
    _need(fn, "recv_indices", recv_indices, 4 * rows * k)


def _check_em_buffers(fn, st, cap_em, em_x, em_scales, em_counts, em_offsets, em_src_pos):
    c = st["cfg"]
    E = c.world_size * c.num_experts_per_rank
    sd = c.scale_dim if c.quant != MEP_QUANT_NONE else 0
    _need(fn, "em_x", em_x, cap_em * _row_bytes_out(c))
    _need(fn, "em_scales", em_scales, 4 * cap_em * sd)
    _need(fn, "em_counts", em_counts, 4 * E)
    _need(fn, "em_offsets", em_offsets, 4 * (E + 1))
    _need(fn, "em_src_pos", em_src_pos, 4 * cap_em)


def _layout_ready(st, layout) -> bool:
    if st is None or layout not in (MEP_RANK_MAJOR, MEP_EXPERT_MAJOR, MEP_RANK_SUM):
        return False
    return st.get("em" if layout == MEP_EXPERT_MAJOR else "rm", False)


def _combine_rows(st, layout) -> int:
    """Rows of the layout's expert-output buffer (0 when no token is planned:
    the call then reads nothing)."""
    c = st["cfg"]
    if not st.get("T"):
        return 0
    if layout in (MEP_RANK_MAJOR, MEP_RANK_SUM):
        return c.world_size * c.max_num_inp_token_per_rank
    return st.get("cap_em") or 0


def _check_combine_buffers(fn, st, layout, y, y_value_bytes, weights, out):
    c = st["cfg"]
    T = st.get("T") or 0
    _need(fn, "y", y, _combine_rows(st, layout) * c.hidden_dim * y_value_bytes)
    if layout != MEP_RANK_SUM:  # converted rows carry their weights
        _need(fn, "weights", weights, 4 * T * c.num_experts_per_token)
    _need(fn, "out", out, 2 * T * c.hidden_dim)


def mep_error_string(code: int) -> str:
    return lib().mep_error_string(code).decode()


def mep_workspace_bytes(cfg: MepConfig) -> int:
    return lib().mep_workspace_bytes(C.byref(cfg))


def mep_create(cfg: MepConfig, workspace, workspace_bytes: int) -> int:
    h = C.c_void_p()
    _check("mep_create", lib().mep_create(C.byref(cfg), _ptr(workspace), workspace_bytes,
                                          C.byref(h)))
    c = MepConfig()
    C.pointer(c)[0] = cfg  # a copy: later edits of cfg do not change the checks
    _handles[h.value] = {"cfg": c, "T": None, "cap_em": None, "rm": False, "em": False}
    return h.value


def mep_destroy(h: int) -> None:
    _check("mep_destroy", lib().mep_destroy(h))
    _handles.pop(h, None)


def mep_plan(h, indices, T, recv_counts, src_token_pos, stream=None) -> None:
    st = _state(h)
    if st is not None and 0 <= T <= st["cfg"].max_num_inp_token_per_rank:
        _check_plan_buffers("mep_plan", st, indices, T, recv_counts, src_token_pos)
    s = _stream(stream, recv_counts)
    _check("mep_plan", lib().mep_plan(h, _ptr(indices), T, _ptr(recv_counts),
                                      _ptr(src_token_pos), s))
    if st is not None:
        st.update(T=T, rm=True, em=False)


def mep_dispatch(h, x, weights, scales, indices, recv_x, recv_scales, recv_weights,
                 recv_indices, stream=None) -> None:
    st = _state(h)
    if _layout_ready(st, MEP_RANK_MAJOR):
        _check_dispatch_buffers("mep_dispatch", st, st["T"], x, weights, scales, indices, recv_x,
                                recv_scales, recv_weights, recv_indices)
    s = _stream(stream, recv_x)
    _check("mep_dispatch", lib().mep_dispatch(h, _ptr(x), _ptr(weights), _ptr(scales),
                                              _ptr(indices), _ptr(recv_x), _ptr(recv_scales),
                                              _ptr(recv_weights), _ptr(recv_indices), s))


def mep_plan_dispatch(h, indices, T, recv_counts, src_token_pos, x, weights, scales, recv_x,
                      recv_scales, recv_weights, recv_indices, stream=None) -> None:
    st = _state(h)
    if st is not None and 0 <= T <= st["cfg"].max_num_inp_token_per_rank:
        _check_plan_buffers("mep_plan_dispatch", st, indices, T, recv_counts, src_token_pos)
        _check_dispatch_buffers("mep_plan_dispatch", st, T, x, weights, scales, indices, recv_x,
                                recv_scales, recv_weights, recv_indices)
    s = _stream(stream, recv_x)
    _check("mep_plan_dispatch", lib().mep_plan_dispatch(
        h, _ptr(indices), T, _ptr(recv_counts), _ptr(src_token_pos), _ptr(x), _ptr(weights),
        _ptr(scales), _ptr(recv_x), _ptr(recv_scales), _ptr(recv_weights), _ptr(recv_indices),
        s))
    if st is not None:
        st.update(T=T, rm=True, em=False)


def mep_plan_dispatch_noalloc(cfg, indices, T, recv_counts, src_token_pos, x, weights, scales,
                              recv_x, recv_scales, recv_weights, recv_indices,
                              stream=None) -> None:
    """mep_plan_dispatch without a handle or workspace (the library's own
    scratch); buffers are checked against cfg as for mep_plan_dispatch."""
    fn = "mep_plan_dispatch_noalloc"
    if 0 <= T <= cfg.max_num_inp_token_per_rank:
        st = {"cfg": cfg}
        _check_plan_buffers(fn, st, indices, T, recv_counts, src_token_pos)
        _check_dispatch_buffers(fn, st, T, x, weights, scales, indices, recv_x, recv_scales,
                                recv_weights, recv_indices)
    s = _stream(stream, recv_x)
    _check(fn, lib().mep_plan_dispatch_noalloc(
        C.byref(cfg), _ptr(indices), T, _ptr(recv_counts), _ptr(src_token_pos), _ptr(x),
        _ptr(weights), _ptr(scales), _ptr(recv_x), _ptr(recv_scales), _ptr(recv_weights),
        _ptr(recv_indices), s))


def mep_dispatch_standard_moe(h, indices, T, x, scales, em_x, em_scales, em_counts, em_offsets,
                              em_src_pos, cap_em, stream=None) -> None:
    st = _state(h)
    fn = "mep_dispatch_standard_moe"
    if st is not None and 0 <= T <= st["cfg"].max_num_inp_token_per_rank and cap_em >= 0:
        c = st["cfg"]
        _need(fn, "indices", indices, 4 * T * c.num_experts_per_token)
        _need(fn, "x", x, T * _row_bytes_in(c))
        if c.quant in (MEP_QUANT_FP8_CARRY, MEP_QUANT_FP4_CARRY):
            _need(fn, "scales", scales, 4 * T * c.scale_dim)
        _check_em_buffers(fn, st, cap_em, em_x, em_scales, em_counts, em_offsets, em_src_pos)
    s = _stream(stream, em_x)
    _check(fn, lib().mep_dispatch_standard_moe(
        h, _ptr(indices), T, _ptr(x), _ptr(scales), _ptr(em_x), _ptr(em_scales),
        _ptr(em_counts), _ptr(em_offsets), _ptr(em_src_pos), cap_em, s))
    if st is not None:
        st.update(T=T, cap_em=cap_em, rm=False, em=True)


def mep_to_expert_major(h, recv_x, recv_scales, recv_indices, recv_counts, src_token_pos, em_x,
                        em_scales, em_counts, em_offsets, em_src_pos, cap_em,
                        stream=None) -> None:
    st = _state(h)
    fn = "mep_to_expert_major"
    if _layout_ready(st, MEP_RANK_MAJOR) and cap_em >= 0:
        c = st["cfg"]
        rows = c.world_size * c.max_num_inp_token_per_rank
        sd = c.scale_dim if c.quant != MEP_QUANT_NONE else 0
        _need(fn, "recv_x", recv_x, rows * _row_bytes_out(c))
        _need(fn, "recv_scales", recv_scales, 4 * rows * sd)
        _need(fn, "recv_indices", recv_indices, 4 * rows * c.num_experts_per_token)
        _need(fn, "recv_counts", recv_counts, 4 * c.world_size)
        _need(fn, "src_token_pos", src_token_pos, 4 * rows)
        _check_em_buffers(fn, st, cap_em, em_x, em_scales, em_counts, em_offsets, em_src_pos)
    s = _stream(stream, em_x)
    _check(fn, lib().mep_to_expert_major(
        h, _ptr(recv_x), _ptr(recv_scales), _ptr(recv_indices), _ptr(recv_counts),
        _ptr(src_token_pos), _ptr(em_x), _ptr(em_scales), _ptr(em_counts), _ptr(em_offsets),
        _ptr(em_src_pos), cap_em, s))
    if st is not None:
        st.update(cap_em=cap_em, em=True)


def mep_combine(h, layout, y, weights, out, stream=None) -> None:
    st = _state(h)
    if _layout_ready(st, layout):
        _check_combine_buffers("mep_combine", st, layout, y, 2, weights, out)
    s = _stream(stream, out)
    _check("mep_combine", lib().mep_combine(h, layout, _ptr(y), _ptr(weights), _ptr(out), s))


def mep_combine_fp8(h, layout, y8, weights, out, stream=None) -> None:
    st = _state(h)
    if _layout_ready(st, layout):
        _check_combine_buffers("mep_combine_fp8", st, layout, y8, 1, weights, out)
    s = _stream(stream, out)
    _check("mep_combine_fp8", lib().mep_combine_fp8(h, layout, _ptr(y8), _ptr(weights), _ptr(out),
                                                    s))


def mep_combine_fp8_direct(h, layout, y, weights, out, stream=None) -> None:
    st = _state(h)
    if _layout_ready(st, layout):
        _check_combine_buffers("mep_combine_fp8_direct", st, layout, y, 2, weights, out)
    s = _stream(stream, out)
    _check("mep_combine_fp8_direct", lib().mep_combine_fp8_direct(
        h, layout, _ptr(y), _ptr(weights), _ptr(out), s))


def mep_cast_fp8_direct(h, layout, y, y8, stream=None) -> None:
    st = _state(h)
    if _layout_ready(st, layout):
        rows, H = _combine_rows(st, layout), st["cfg"].hidden_dim
        _need("mep_cast_fp8_direct", "y", y, rows * H * 2)
        _need("mep_cast_fp8_direct", "y8", y8, rows * H)
    s = _stream(stream, y8)
    _check("mep_cast_fp8_direct", lib().mep_cast_fp8_direct(h, layout, _ptr(y), _ptr(y8), s))


def mep_convert_combine_input(h, em_y, recv_weights, y, stream=None) -> None:
    st = _state(h)
    fn = "mep_convert_combine_input"
    if st is not None and st["rm"] and st["em"] and st["T"]:
        c = st["cfg"]
        rows = c.world_size * c.max_num_inp_token_per_rank
        _need(fn, "em_y", em_y, (st.get("cap_em") or 0) * c.hidden_dim * 2)
        _need(fn, "recv_weights", recv_weights, 4 * rows * c.num_experts_per_token)
        _need(fn, "y", y, rows * c.hidden_dim * 2)
    s = _stream(stream, y)
    _check(fn, lib().mep_convert_combine_input(h, _ptr(em_y), _ptr(recv_weights), _ptr(y), s))


def mep_reset(h, stream=None) -> None:
    _check("mep_reset", lib().mep_reset(h, _stream(stream)))
    st = _state(h)
    if st is not None:
        st.update(rm=False, em=False)


def mep_get_status(h, stream=None) -> int:
    v = C.c_int32(0)
    rc = lib().mep_get_status(h, _stream(stream), C.byref(v))
    if rc not in (MEP_OK, MEP_ERR_DEVICE):
        raise MepError("mep_get_status", rc)
    return v.value


def mep_get_route(h, recv_row, em_row=None, stream=None) -> None:
    st = _state(h)
    if st is not None and st["T"] is not None:
        n = 4 * st["T"] * st["cfg"].num_experts_per_token
        if st["rm"]:
            _need("mep_get_route", "recv_row", recv_row, n)
        if st["em"]:
            _need("mep_get_route", "em_row", em_row, n)
    s = _stream(stream, recv_row)
    _check("mep_get_route", lib().mep_get_route(h, _ptr(recv_row), _ptr(em_row), s))


def mep_probe_e4m3(inp, out, n, stream=None) -> None:
    _check("mep_probe_e4m3", lib().mep_probe_e4m3(_ptr(inp), _ptr(out), n, _stream(stream, out)))


def mep_probe_bf16(inp, out, n, stream=None) -> None:
    _check("mep_probe_bf16", lib().mep_probe_bf16(_ptr(inp), _ptr(out), n, _stream(stream, out)))


def mep_probe_fp8_block(inp, q, scales, nblocks, stream=None) -> None:
    _check("mep_probe_fp8_block", lib().mep_probe_fp8_block(_ptr(inp), _ptr(q), _ptr(scales),
                                                            nblocks, _stream(stream, q)))


def mep_probe_mxfp4(inp, q, e8, nblocks, stream=None) -> None:
    _check("mep_probe_mxfp4", lib().mep_probe_mxfp4(_ptr(inp), _ptr(q), _ptr(e8), nblocks,
                                                    _stream(stream, q)))


def mep_probe_stream(src, dst, waves, rd_units, wr_units, stream=None) -> None:
    fn = "mep_probe_stream"
    _need(fn, "src", src, rd_units * 1024)
    _need(fn, "dst", dst, max(wr_units * 1024, 16))
    _check(fn, lib().mep_probe_stream(_ptr(src), _ptr(dst), waves, rd_units, wr_units,
                                      _stream(stream, dst)))


class Mep:
    """A handle together with the device workspace it is bound to (allocated
    here with torch, the only allocation on the Python side).  ``fp8=True``
    selects block quantisation; ``quant``/``scale_dim`` set the payload mode
    explicitly (MEP_QUANT_FP8_CARRY takes the caller's scale columns)."""

    def __init__(self, hidden_dim, num_experts_per_rank, num_experts_per_token,
                 max_num_inp_token_per_rank, world_size, rank=0, fp8=False, device="cuda",
                 quant=None, scale_dim=None):
        import torch
        if quant is None:
            quant = MEP_QUANT_FP8_E4M3_BLOCK128 if fp8 else MEP_QUANT_NONE
        if scale_dim is None:
            scale_dim = hidden_dim // 128 if quant != MEP_QUANT_NONE else 0
        self.cfg = MepConfig(hidden_dim, scale_dim, num_experts_per_rank, num_experts_per_token,
                             max_num_inp_token_per_rank, world_size, rank, quant)
        nbytes = mep_workspace_bytes(self.cfg)
        if nbytes == 0:
            raise MepError("mep_workspace_bytes", MEP_ERR_CONFIG)
        self.workspace = torch.zeros(nbytes, dtype=torch.uint8, device=device)
        self.h = mep_create(self.cfg, self.workspace, nbytes)

    def close(self):
        if self.h:
            mep_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
