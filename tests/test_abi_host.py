"""Host-side checks of the C ABI (no GPU needed, no kernel launched): the
library loads, exports every entry point include/mep.h declares, and rejects
bad configs, shapes, alignment and call order before touching the device.
The device pointers used here are fake aligned addresses; every call below
returns before any HIP call would dereference them."""

import ctypes as C
import os
import re

import pytest

import combine_mep_plan_amd as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x7F0000000000  # 256-byte aligned, never dereferenced on the host


def declared_functions():
    src = open(os.path.join(ROOT, "include", "mep.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mep_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 13
    L = C.CDLL(M.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n


def cfg(**kw):
    base = dict(hidden_dim=7168, scale_dim=0, num_experts_per_rank=32, num_experts_per_token=8,
                max_num_inp_token_per_rank=4096, world_size=8, rank=0, quant=M.MEP_QUANT_NONE)
    base.update(kw)
    return M.MepConfig(**base)


@pytest.mark.parametrize("bad", [
    dict(hidden_dim=0), dict(hidden_dim=7170), dict(world_size=0), dict(world_size=65),
    dict(num_experts_per_rank=0), dict(num_experts_per_rank=65),
    dict(num_experts_per_token=0), dict(num_experts_per_token=33),
    dict(num_experts_per_token=5, world_size=2, num_experts_per_rank=2),
    dict(max_num_inp_token_per_rank=0), dict(rank=8), dict(rank=-1),
    dict(scale_dim=56),                                    # scales without quant
    dict(quant=M.MEP_QUANT_FP8_E4M3_BLOCK128, scale_dim=0),  # quant without scales
    dict(quant=M.MEP_QUANT_FP8_E4M3_BLOCK128, hidden_dim=7176, scale_dim=56),
    dict(quant=7),
    dict(quant=M.MEP_QUANT_FP8_CARRY, hidden_dim=7176, scale_dim=56),  # E4M3 rows: H % 16
    dict(quant=M.MEP_QUANT_FP8_CARRY, scale_dim=-1),
    dict(quant=M.MEP_QUANT_FP8_CARRY, scale_dim=(1 << 16) + 1),
    dict(world_size=64, max_num_inp_token_per_rank=1 << 25),  # rows overflow int32
])
def test_bad_configs_rejected(bad):
    c = cfg(**bad)
    assert M.mep_workspace_bytes(c) == 0
    h = C.c_void_p()
    assert M.lib().mep_create(C.byref(c), FAKE, 1 << 40, C.byref(h)) == M.MEP_ERR_CONFIG
    assert h.value is None


def test_workspace_size_and_create_checks():
    c = cfg(quant=M.MEP_QUANT_FP8_E4M3_BLOCK128, scale_dim=56)
    n = M.mep_workspace_bytes(c)
    assert n > 4096 * 8 * 4  # at least the receive-row map
    L = M.lib()
    h = C.c_void_p()
    assert L.mep_create(C.byref(c), None, n, C.byref(h)) == M.MEP_ERR_NULL
    assert L.mep_create(C.byref(c), FAKE + 8, n, C.byref(h)) == M.MEP_ERR_ALIGN
    assert L.mep_create(C.byref(c), FAKE, n - 1, C.byref(h)) == M.MEP_ERR_SHAPE
    assert L.mep_create(C.byref(c), FAKE, n, None) == M.MEP_ERR_NULL
    assert L.mep_create(None, FAKE, n, C.byref(h)) == M.MEP_ERR_NULL
    assert L.mep_create(C.byref(c), FAKE, n, C.byref(h)) == M.MEP_OK
    assert L.mep_destroy(h) == M.MEP_OK


@pytest.mark.parametrize("R,epr", [(1, 1), (4, 2), (8, 32), (16, 16), (32, 8), (64, 64), (7, 13)])
def test_create_accepts_the_expert_rank_maps(R, epr):
    # mep_create checks its divide-free expert -> rank map for every expert id
    c = cfg(world_size=R, num_experts_per_rank=epr, num_experts_per_token=min(8, R * epr),
            max_num_inp_token_per_rank=64)
    h = C.c_void_p()
    assert M.lib().mep_create(C.byref(c), FAKE, M.mep_workspace_bytes(c), C.byref(h)) == M.MEP_OK
    M.lib().mep_destroy(h)


def test_call_order_and_argument_checks_before_any_launch():
    L = M.lib()
    c = cfg()
    n = M.mep_workspace_bytes(c)
    h = C.c_void_p()
    assert L.mep_create(C.byref(c), FAKE, n, C.byref(h)) == M.MEP_OK
    h = h.value
    f = FAKE
    # no plan yet: dispatch, expert-major conversion, combine and route inspection refuse
    assert L.mep_dispatch(h, f, f, None, f, f, None, f, f, None) == M.MEP_ERR_STATE
    assert L.mep_to_expert_major(h, f, None, f, f, f, f, None, f, f, f, 1000, None) \
        == M.MEP_ERR_STATE
    assert L.mep_combine(h, M.MEP_RANK_MAJOR, f, f, f, None) == M.MEP_ERR_STATE
    assert L.mep_combine(h, 5, f, f, f, None) == M.MEP_ERR_SHAPE
    assert L.mep_get_route(h, f, None, None) == M.MEP_ERR_STATE
    # converted rows: the conversion needs a plan and an expert-major layout,
    # their combine a plan; only the bf16 combine takes them
    assert L.mep_convert_combine_input(h, f, f, f, None) == M.MEP_ERR_STATE
    assert L.mep_combine(h, M.MEP_RANK_SUM, f, None, f, None) == M.MEP_ERR_STATE
    assert L.mep_combine_fp8(h, M.MEP_RANK_SUM, f, f, f, None) == M.MEP_ERR_SHAPE
    assert L.mep_combine_fp8_direct(h, M.MEP_RANK_SUM, f, f, f, None) == M.MEP_ERR_SHAPE
    assert L.mep_cast_fp8_direct(h, M.MEP_RANK_SUM, f, f, None) == M.MEP_ERR_SHAPE
    # plan argument checks
    assert L.mep_plan(h, f, 4097, f, f, None) == M.MEP_ERR_SHAPE
    assert L.mep_plan(h, f, -1, f, f, None) == M.MEP_ERR_SHAPE
    assert L.mep_plan(h, None, 16, f, f, None) == M.MEP_ERR_NULL
    assert L.mep_plan(h, f, 16, None, f, None) == M.MEP_ERR_NULL
    assert L.mep_plan(h, f + 4, 16, f, f, None) == M.MEP_ERR_ALIGN
    assert L.mep_plan(h, f, 16, f, f + 4, None) == M.MEP_ERR_ALIGN
    # probes and status
    assert L.mep_probe_e4m3(f, f, -1, None) == M.MEP_ERR_SHAPE
    assert L.mep_probe_bf16(None, f, 8, None) == M.MEP_ERR_NULL
    assert L.mep_probe_bf16(f + 2, f, 8, None) == M.MEP_ERR_ALIGN
    assert L.mep_probe_mxfp4(f, f, f, -1, None) == M.MEP_ERR_SHAPE
    assert L.mep_probe_mxfp4(f, None, f, 1, None) == M.MEP_ERR_NULL
    assert L.mep_probe_mxfp4(f + 2, f, f, 1, None) == M.MEP_ERR_ALIGN
    assert L.mep_probe_mxfp4(None, None, None, 0, None) == M.MEP_OK
    assert L.mep_probe_fp8_block(f, f, f, -1, None) == M.MEP_ERR_SHAPE
    assert L.mep_probe_fp8_block(f, f, None, 1, None) == M.MEP_ERR_NULL
    assert L.mep_probe_fp8_block(f, f + 8, f, 1, None) == M.MEP_ERR_ALIGN
    assert L.mep_probe_fp8_block(f, f, f + 2, 1, None) == M.MEP_ERR_ALIGN
    assert L.mep_probe_fp8_block(None, None, None, 0, None) == M.MEP_OK
    assert L.mep_get_status(None, None, None) == M.MEP_ERR_NULL
    ps = L.mep_probe_stream  # (src, dst, waves, rd_units, wr_units, stream)
    assert ps(f, f, 100, 1601, 0, None) == M.MEP_ERR_SHAPE      # 17 read units in a wave
    assert ps(f, f, (1 << 24) + 1, 0, 1, None) == M.MEP_ERR_SHAPE
    assert ps(f, f, -1, 0, 0, None) == M.MEP_ERR_SHAPE
    assert ps(f, f, 0, 1, 0, None) == M.MEP_ERR_SHAPE
    assert ps(f, f, 0, 0, 0, None) == M.MEP_OK                  # nothing to do, no launch
    assert ps(None, f, 10, 5, 5, None) == M.MEP_ERR_NULL
    assert ps(f, None, 10, 5, 0, None) == M.MEP_ERR_NULL
    assert ps(f + 4, f, 10, 5, 5, None) == M.MEP_ERR_ALIGN
    assert L.mep_destroy(h) == M.MEP_OK
    assert L.mep_destroy(None) == M.MEP_ERR_NULL


@pytest.mark.parametrize("sd", [0, 3, 56, 1 << 16])
def test_carry_configs_accepted(sd):
    c = cfg(quant=M.MEP_QUANT_FP8_CARRY, scale_dim=sd)
    h = C.c_void_p()
    assert M.lib().mep_create(C.byref(c), FAKE, M.mep_workspace_bytes(c), C.byref(h)) == M.MEP_OK
    M.lib().mep_destroy(h)


def test_standard_moe_and_carry_argument_checks():
    L = M.lib()
    f = FAKE
    c = cfg(quant=M.MEP_QUANT_FP8_CARRY, scale_dim=56)
    h = C.c_void_p()
    assert L.mep_create(C.byref(c), f, M.mep_workspace_bytes(c), C.byref(h)) == M.MEP_OK
    h = h.value
    sm = L.mep_dispatch_standard_moe
    # (h, indices, T, x, scales, em_x, em_scales, em_counts, em_offsets, em_src_pos, cap_em, s)
    assert sm(h, f, 4097, f, f, f, f, f, f, f, 1000, None) == M.MEP_ERR_SHAPE
    assert sm(h, f, -1, f, f, f, f, f, f, f, 1000, None) == M.MEP_ERR_SHAPE
    assert sm(h, f, 16, f, f, f, f, f, f, f, -1, None) == M.MEP_ERR_SHAPE
    assert sm(h, f, 16, f, f, f, f, f, f, f, 1 << 31, None) == M.MEP_ERR_SHAPE
    assert sm(h, f, 16, f, None, f, f, f, f, f, 1000, None) == M.MEP_ERR_NULL  # carried scales
    assert sm(h, f, 16, f, f, f, None, f, f, f, 1000, None) == M.MEP_ERR_NULL
    assert sm(h, None, 16, f, f, f, f, f, f, f, 1000, None) == M.MEP_ERR_NULL
    assert sm(h, f, 16, None, f, f, f, f, f, f, 1000, None) == M.MEP_ERR_NULL
    assert sm(h, f, 16, f, f, None, f, f, f, f, 1000, None) == M.MEP_ERR_NULL
    assert sm(h, f, 16, f, f, f, f, f, f, None, 1000, None) == M.MEP_ERR_NULL
    assert sm(h, f, 16, f, f + 4, f, f, f, f, f, 1000, None) == M.MEP_ERR_ALIGN
    assert sm(h, f, 16, f, f, f, f, f, f + 8, f, 1000, None) == M.MEP_ERR_ALIGN
    assert sm(None, f, 16, f, f, f, f, f, f, f, 1000, None) == M.MEP_ERR_NULL
    # the rank-major dispatch of carried rows needs the scales too (checked
    # before the call-order rule only once a plan exists, so here: state)
    assert L.mep_dispatch(h, f, f, None, f, f, f, f, f, None) == M.MEP_ERR_STATE
    assert L.mep_plan_dispatch(h, f, 16, f, f, f, f, None, f, f, f, f, None) == M.MEP_ERR_NULL
    assert L.mep_plan_dispatch(h, f, 16, f, f, f, f, f + 4, f, f, f, f, None) == M.MEP_ERR_ALIGN
    assert L.mep_destroy(h) == M.MEP_OK


def test_expert_major_offsets_must_fit_int32():
    # segment offsets are int32 sums of counts padded to 128 rows: a batch whose
    # T*k + 127*E could pass INT32_MAX is refused before any launch
    L = M.lib()
    f = FAKE
    c = cfg(world_size=1, num_experts_per_rank=64, num_experts_per_token=32,
            max_num_inp_token_per_rank=1 << 27, hidden_dim=256)
    n = M.mep_workspace_bytes(c)
    assert n > 0
    h = C.c_void_p()
    assert L.mep_create(C.byref(c), f, n, C.byref(h)) == M.MEP_OK
    h = h.value
    T = (2**31 - 1 - 127 * 64) // 32 + 1      # the smallest batch that does not fit
    sm = L.mep_dispatch_standard_moe
    assert sm(h, f, T, f, None, f, None, f, f, f, 1 << 30, None) == M.MEP_ERR_SHAPE
    assert sm(h, f, 1 << 26, f, None, f, None, f, f, f, 1 << 30, None) == M.MEP_ERR_SHAPE
    assert L.mep_destroy(h) == M.MEP_OK


def test_noalloc_refuses_batches_beyond_its_scratch():
    # the entry point that allocates nothing keeps its plan in a 2 MiB scratch:
    # 16384 tokens at top-32 on 64 ranks need more and are refused before any
    # HIP call (the pointers are fake), as are the usual argument errors
    L = M.lib()
    f = FAKE
    cfg = M.MepConfig(256, 0, 2, 32, 16384, 64, 0, M.MEP_QUANT_NONE)
    na = L.mep_plan_dispatch_noalloc
    assert na(C.byref(cfg), f, 16384, f, f, f, f, None, f, None, f, f, None) == M.MEP_ERR_SHAPE
    assert na(C.byref(cfg), f, 16385, f, f, f, f, None, f, None, f, f, None) == M.MEP_ERR_SHAPE
    assert na(None, f, 16, f, f, f, f, None, f, None, f, f, None) == M.MEP_ERR_NULL
    assert na(C.byref(cfg), None, 16, f, f, f, f, None, f, None, f, f, None) == M.MEP_ERR_NULL
    assert na(C.byref(cfg), f, 16, f, f + 4, f, f, None, f, None, f, f, None) == M.MEP_ERR_ALIGN
    bad = M.MepConfig(256, 0, 2, 32, 16384, 64, 64, M.MEP_QUANT_NONE)  # rank out of range
    assert na(C.byref(bad), f, 16, f, f, f, f, None, f, None, f, f, None) == M.MEP_ERR_CONFIG


def test_error_strings():
    for code in range(-8, 1):
        assert M.mep_error_string(code) not in ("", "unknown")
    assert M.mep_error_string(-99) == "unknown"


def test_binding_refuses_host_tensors():
    # a host tensor's address handed to a kernel would fault the GPU: the
    # binding refuses it before any call reaches the library
    import torch
    t = torch.zeros(64, dtype=torch.int32)
    with pytest.raises(ValueError, match="on the GPU"):
        M.mep_probe_bf16(t, t, 0)
    from combine_mep_plan_amd import _binding as B
    assert B._ptr(None) is None and B._ptr(1 << 20) == 1 << 20


def test_binding_checks_buffer_sizes():
    # the binding knows each handle's config and last planned token count and
    # refuses a buffer shorter than what the call would touch
    import torch
    c = cfg(quant=M.MEP_QUANT_FP8_E4M3_BLOCK128, scale_dim=56)
    h = M.mep_create(c, FAKE, M.mep_workspace_bytes(c))
    R, cap, H, k = c.world_size, c.max_num_inp_token_per_rank, c.hidden_dim, \
        c.num_experts_per_token
    i32 = lambda n: torch.zeros(n, dtype=torch.int32)  # noqa: E731
    f32 = lambda n: torch.zeros(n, dtype=torch.float32)  # noqa: E731
    T = 16
    with pytest.raises(ValueError, match="indices holds"):
        M.mep_plan(h, i32(T * k - 1), T, i32(R), i32(R * cap))
    with pytest.raises(ValueError, match="src_token_pos holds"):
        M.mep_plan(h, i32(T * k), T, i32(R), i32(R * cap - 1))
    ok = dict(x=torch.zeros((T, H), dtype=torch.int16), w=f32(T * k),
              rx=torch.zeros((R, cap, H), dtype=torch.uint8), rs=f32(R * cap * H // 128),
              rw=f32(R * cap * k), ri=i32(R * cap * k))
    for name, short in (("recv_x", torch.zeros(R * cap * H - 1, dtype=torch.uint8)),
                        ("recv_scales", f32(R * cap * H // 128 - 1)),
                        ("x", torch.zeros(T * H - 1, dtype=torch.int16))):
        a = dict(ok)
        a[{"recv_x": "rx", "recv_scales": "rs", "x": "x"}[name]] = short
        with pytest.raises(ValueError, match=f"{name} holds"):
            M.mep_plan_dispatch(h, i32(T * k), T, i32(R), i32(R * cap), a["x"], a["w"], None,
                                a["rx"], a["rs"], a["rw"], a["ri"])
    with pytest.raises(ValueError, match="indices must be torch.int32"):
        M.mep_plan(h, torch.zeros(T * k, dtype=torch.int64), T, i32(R), i32(R * cap))
    with pytest.raises(ValueError, match="weights must be torch.float32"):
        M.mep_plan_dispatch(h, i32(T * k), T, i32(R), i32(R * cap), ok["x"],
                            torch.zeros(T * k, dtype=torch.float64), None, ok["rx"], ok["rs"],
                            ok["rw"], ok["ri"])
    # every size right: the host tensors are then refused as host memory
    with pytest.raises(ValueError, match="on the GPU"):
        M.mep_plan_dispatch(h, i32(T * k), T, i32(R), i32(R * cap), ok["x"], ok["w"], None,
                            ok["rx"], ok["rs"], ok["rw"], ok["ri"], stream=0)
    M.mep_destroy(h)
