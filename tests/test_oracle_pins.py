"""Pins for the CPU oracle: each test checks the oracle against something other
than itself -- torch's independent codecs, a different formulation of the same
result (stable sort, bincount), closed forms from the format definitions,
invariants the pages fix, and a hand-worked example.

Pages: "MORI-EP User Guide" (section 3 Operator API: dispatch(), combine(),
get_dispatch_src_token_pos(); section 4 Standard MoE Compatibility; section 7
Complete Example: identity expert), "Choosing an EP API and backend" (OCP E4M3
on gfx950), ROCm/mori issue #57 (redundant transfer removed).
"""

import os

import dataclasses

import numpy as np
import pytest
import torch

from synthetic import WORKLOADS, make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f32_bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def torch_bf16(v32):
    return torch.from_numpy(np.ascontiguousarray(v32, np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def torch_e4m3(v32):
    return torch.from_numpy(np.ascontiguousarray(v32, np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def bf16_f32(h):
    return (np.asarray(h, np.uint16).astype(np.uint32) << 16).view(np.float32)


def unique_pairs(idx, epr):
    """(t, r) pairs in token order, first occurrence of each rank per token."""
    pairs = []
    for t in range(idx.shape[0]):
        seen = []
        for e in idx[t]:
            r = int(e) // epr
            if r not in seen:
                seen.append(r)
                pairs.append((t, r))
    return pairs


# ----------------------------------------------------------------------------
# codecs
# ----------------------------------------------------------------------------

def test_bf16_rne_matches_torch(oracle):
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2**32, size=400_000, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[np.isfinite(v)]
    # exact ties: low 16 bits == 0x8000, both parities of the kept bit
    ties = ((rng.integers(0, 2**16, size=20_000).astype(np.uint32) << 16) | 0x8000).view(np.float32)
    ties = ties[np.isfinite(ties)]
    denorm = (rng.integers(1, 2**23, size=20_000).astype(np.uint32)).view(np.float32)
    for arr in (v, ties, denorm, -denorm, np.float32([0.0, -0.0, 1.0, 65504.0])):
        assert np.array_equal(oracle.bf16_rne(arr), torch_bf16(arr))


def test_e4m3_decode_table(oracle):
    tab = oracle.e4m3_decode_table()
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    finite = ~np.isnan(ref)
    assert np.array_equal(np.isnan(tab), np.isnan(ref))
    assert np.array_equal(tab[finite], ref[finite])
    # closed forms of the OCP format: 448 largest finite, 2^-6 smallest normal,
    # 2^-9 smallest subnormal, S.1111.111 NaN, magnitudes increasing with the code
    assert tab[0x7E] == 448.0 and tab[0xFE] == -448.0
    assert tab[0x08] == 2.0 ** -6 and tab[0x01] == 2.0 ** -9
    assert np.isnan(tab[0x7F]) and np.isnan(tab[0xFF])
    assert np.all(np.diff(tab[:0x7F]) > 0)


def test_e4m3_encode_matches_torch_sweep(oracle):
    # every 61st fp32 bit pattern from 0 up to 464 (torch and the OCP reading agree
    # there; above it torch gives NaN while the reading saturates)
    top = int(np.float32(464.0).view(np.uint32))
    pats = np.arange(0, top + 1, 61, dtype=np.uint32)
    v = pats.view(np.float32)
    for arr in (v, -v):
        assert np.array_equal(oracle.e4m3_encode(arr), torch_e4m3(arr))


def test_e4m3_encode_at_every_boundary(oracle):
    tab = oracle.e4m3_decode_table()[:0x7F]
    vals = []
    for c in range(0x7F):
        vals.append(tab[c])
        if c:
            mid = 0.5 * (tab[c - 1] + tab[c])
            vals.append(mid)
    base = np.array(vals, dtype=np.float32)
    assert np.array_equal(base.astype(np.float64), np.array(vals))  # all exact in fp32
    b = base.view(np.uint32)
    near = np.concatenate([b, b + 1, b + 2, np.maximum(b, 1) - 1]).view(np.float32)
    near = near[near <= 464.0]
    for arr in (near, -near):
        assert np.array_equal(oracle.e4m3_encode(arr), torch_e4m3(arr))
    # explicit ties: the midpoint goes to the even code
    for c in range(1, 0x7F):
        mid = np.float32(0.5 * (tab[c - 1] + tab[c]))
        even = c - 1 if (c - 1) % 2 == 0 else c
        assert oracle.e4m3_encode(np.array([mid]))[0] == even


def test_e4m3_saturates_and_keeps_sign(oracle):
    v = np.float32([448.0, 448.00003, 463.9, 464.0, 470.0, 1e6, -1e6, -0.0, 0.0, -1e-30])
    got = oracle.e4m3_encode(v)
    assert list(got) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x80, 0x00, 0x80]


# ----------------------------------------------------------------------------
# routing plan
# ----------------------------------------------------------------------------

def _read_golden(name):
    d = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            d[key] = [int(v) for v in vals]
    return d


def test_plan_hand_worked_example(oracle):
    g = _read_golden("plan_tiny.txt")
    R, epr, cap, src = g["R"][0], g["epr"][0], g["cap"][0], g["src_rank"][0]
    idx = np.array(g["indices"], np.int32).reshape(-1, 2)
    pl = oracle.plan(idx, R, epr, cap, src)
    assert list(pl["recv_counts"]) == g["recv_counts"]
    assert list(pl["src_token_pos"][0, :3]) == g["src_token_pos_rank0"]
    assert list(pl["src_token_pos"][1, :3]) == g["src_token_pos_rank1"]
    assert list(pl["slot"].ravel()) == g["slot"]
    assert pl["status"] == 0


def _check_plan_against_sort(idx, R, epr, cap, pl, src_rank=0):
    T, k = idx.shape
    pairs = unique_pairs(idx, epr)
    ts = np.array([p[0] for p in pairs])
    rs = np.array([p[1] for p in pairs])
    # counts: histogram of the unique pairs' ranks
    assert np.array_equal(pl["recv_counts"], np.bincount(rs, minlength=R).astype(np.int32))
    # slots: rank of each pair inside its rank group after a stable sort by rank
    order = np.argsort(rs, kind="stable")
    starts = np.concatenate([[0], np.cumsum(np.bincount(rs, minlength=R))[:-1]])
    pos_in_group = np.empty(len(pairs), np.int64)
    pos_in_group[order] = np.arange(len(pairs)) - starts[rs[order]]
    want = {(int(t), int(r)): int(s) for t, r, s in zip(ts, rs, pos_in_group)}
    for t in range(T):
        for j in range(k):
            assert pl["slot"][t, j] == want[(t, int(idx[t, j]) // epr)]
    # src_token_pos: the sorted pairs' tokens, encoded
    for r in range(R):
        n = pl["recv_counts"][r]
        exp = src_rank * R * cap + ts[order][starts[r]:starts[r] + n]
        assert np.array_equal(pl["src_token_pos"][r, :n], exp)
        assert np.all(pl["src_token_pos"][r, n:] == -1)  # nothing else written


@pytest.mark.parametrize("name", ["tiny", "decode", "skew", "prefill", "stdmoe"])
def test_plan_matches_stable_sort_and_invariants(oracle, name):
    wl = WORKLOADS[name]
    if wl.tokens > 1024:
        wl = wl.with_tokens(1024)
    for seed in (0, 1):
        inp = make_inputs(wl, seed)
        idx = inp["indices"]
        src = 1 if seed else 0
        pl = oracle.plan(idx, wl.ranks, wl.experts_per_rank, wl.cap, src)
        assert pl["status"] == 0
        _check_plan_against_sort(idx, wl.ranks, wl.experts_per_rank, wl.cap, pl, src)
        # invariants: sum of counts = unique pairs; positions strictly increasing per
        # rank; (r, s) -> (t, r) is a bijection onto the unique pairs; counts <= T
        U = len(unique_pairs(idx, wl.experts_per_rank))
        assert pl["recv_counts"].sum() == U
        seen = set()
        for r in range(wl.ranks):
            n = pl["recv_counts"][r]
            assert n <= wl.tokens
            p = pl["src_token_pos"][r, :n] - src * wl.ranks * wl.cap
            assert np.all(np.diff(p) > 0)
            seen.update((int(t), r) for t in p)
        assert len(seen) == U


def test_plan_single_rank_and_top1(oracle):
    rng = np.random.default_rng(3)
    # R = 1: every token lands once on rank 0 at slot t
    idx = np.stack([rng.permutation(8)[:3] for _ in range(50)]).astype(np.int32)
    pl = oracle.plan(idx, 1, 8, 64)
    assert np.array_equal(pl["slot"], np.repeat(np.arange(50)[:, None], 3, 1))
    assert list(pl["recv_counts"]) == [50]
    # k = 1: a stable counting sort of tokens by rank
    idx = rng.integers(0, 12, size=(200, 1)).astype(np.int32)
    pl = oracle.plan(idx, 4, 3, 256)
    r = idx[:, 0] // 3
    for rr in range(4):
        toks = np.nonzero(r == rr)[0]
        assert np.array_equal(pl["slot"][toks, 0], np.arange(len(toks)))


def test_plan_uniform_rank_fanout(oracle):
    # statistical sanity: with k distinct uniform experts of E, a token reaches
    # R * (1 - C(E-epr, k)/C(E, k)) ranks on average (5.295 for 8 x 32, top-8)
    from math import comb
    wl = WORKLOADS["prefill"]
    idx = make_inputs(wl, 0)["indices"]
    pl = oracle.plan(idx, wl.ranks, wl.experts_per_rank, wl.cap)
    E, epr, k, R = wl.experts, wl.experts_per_rank, wl.topk, wl.ranks
    mean = R * (1 - comb(E - epr, k) / comb(E, k))
    assert abs(pl["recv_counts"].sum() / wl.tokens - mean) < 0.05


def test_plan_status_bits(oracle):
    idx = np.array([[0, 1], [2, 9], [3, 3], [-1, 0]], np.int32)  # E = 4
    pl = oracle.plan(idx, 2, 2, 8)
    assert pl["status"] == oracle.ST_BAD_INDEX | oracle.ST_DUP_EXPERT
    assert list(pl["slot"][1]) == [-1, -1] and list(pl["slot"][3]) == [-1, -1]
    assert list(pl["recv_counts"]) == [1, 1]  # t0 -> rank 0; t2 -> rank 1 (once)


# ----------------------------------------------------------------------------
# dispatch
# ----------------------------------------------------------------------------

def _dispatch(oracle, wl, seed, T=None):
    if T is not None:
        wl = wl.with_tokens(T)
    inp = make_inputs(wl, seed)
    pl = oracle.plan(inp["indices"], wl.ranks, wl.experts_per_rank, wl.cap)
    d = oracle.dispatch(inp["x"], inp["weights"], inp["indices"], pl, wl.ranks,
                        wl.experts_per_rank, wl.cap, wl.quant == "fp8", fill=0xA5)
    return wl, inp, pl, d


@pytest.mark.parametrize("name", ["tiny", "decode", "skew"])
def test_dispatch_bf16_rows_are_copies(oracle, name):
    wl, inp, pl, d = _dispatch(oracle, WORKLOADS[name], 0, T=min(WORKLOADS[name].tokens, 512))
    epr = wl.experts_per_rank
    written = np.zeros((wl.ranks, wl.cap), bool)
    for t, r in unique_pairs(inp["indices"], epr):
        s = pl["slot"][t][[int(e) // epr for e in inp["indices"][t]].index(r)]
        assert np.array_equal(d["recv_x"][r, s], inp["x"][t])
        assert np.array_equal(d["recv_weights"][r, s], inp["weights"][t])
        assert np.array_equal(d["recv_indices"][r, s], inp["indices"][t])
        written[r, s] = True
    assert np.all(d["recv_x"][~written] == 0xA5A5)


def test_dispatch_fp8_scales_and_codes(oracle):
    wl, inp, pl, d = _dispatch(oracle, WORKLOADS["prefill"], 1, T=96)
    x32 = bf16_f32(inp["x"]).reshape(wl.tokens, -1, 128)
    amax = np.abs(x32).max(axis=2)
    s_ref = (amax.astype(np.float32) / np.float32(448.0)).astype(np.float32)
    q_ref = torch_e4m3((x32 / s_ref[:, :, None]).astype(np.float32)).reshape(wl.tokens, -1)
    epr = wl.experts_per_rank
    for t, r in unique_pairs(inp["indices"], epr):
        s = pl["slot"][t][[int(e) // epr for e in inp["indices"][t]].index(r)]
        assert np.array_equal(d["recv_scales"][r, s], s_ref[t])
        assert np.array_equal(d["recv_x"][r, s], q_ref[t])


def test_quant_row_edge_blocks(oracle):
    # a zero block (scale 0, signed zeros), a block whose amax element maps to 448,
    # a block of subnormal-scale values, and the FP8 error bound
    rng = np.random.default_rng(5)
    x32 = rng.standard_normal(512).astype(np.float32)
    x32[0:128] = 0.0
    x32[5] = -0.0
    x32[256:384] *= np.float32(1e-38)
    xb = torch_bf16(x32)
    q, s = oracle.quant_row(xb)
    xf = bf16_f32(xb)
    assert s[0] == 0.0 and np.all(q[0:128][xf[0:128].view(np.uint32) == 0] == 0x00)
    assert q[5] == 0x80
    tab = oracle.e4m3_decode_table()
    for b in range(1, 4):
        blk = xf[b * 128:(b + 1) * 128]
        i = np.argmax(np.abs(blk))
        assert q[b * 128 + i] & 0x7F == 0x7E
        deq = tab[q[b * 128:(b + 1) * 128]] * np.float64(s[b])
        v = np.abs(blk.astype(np.float64) / np.float64(s[b]))
        err = np.abs(deq - blk)
        big = v >= 2.0 ** -6
        assert np.all(err[big] <= 2.0 ** -4 * np.abs(blk[big]) * (1 + 1e-6))
        assert np.all(err[~big] <= np.float64(s[b]) * 2.0 ** -10 * (1 + 1e-6))


# ----------------------------------------------------------------------------
# combine
# ----------------------------------------------------------------------------

def _ulp_bf16(v):
    a = np.abs(np.asarray(v, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 7)


@pytest.mark.parametrize("name", ["tiny", "decode", "skew"])
def test_identity_round_trip(oracle, name):
    # the pages' own check: identity expert, combine(dispatch(x)) = x * sum(w)
    wl, inp, pl, d = _dispatch(oracle, WORKLOADS[name], 2, T=min(WORKLOADS[name].tokens, 256))
    out = oracle.combine(d["recv_x"], inp["weights"], inp["indices"], pl,
                         wl.experts_per_rank, wl.cap)
    exact = bf16_f32(inp["x"]).astype(np.float64) * inp["weights"].astype(np.float64).sum(1)[:, None]
    ref = bf16_f32(torch_bf16(exact.astype(np.float32)))  # fp64 -> fp32 is within 2^-24
    diff = np.abs(bf16_f32(out).astype(np.float64) - ref)
    assert np.all(diff <= _ulp_bf16(ref) * 1.0000001)


def test_combine_top1_unit_weight_and_one_hot(oracle):
    rng = np.random.default_rng(7)
    T, H, R, epr, cap = 40, 256, 4, 3, 64
    # top-1 with weight 1: the output is the token's own row, bit for bit
    idx = rng.integers(0, R * epr, size=(T, 1)).astype(np.int32)
    x = torch_bf16(rng.standard_normal((T, H)).astype(np.float32))
    w1 = np.ones((T, 1), np.float32)
    pl = oracle.plan(idx, R, epr, cap)
    d = oracle.dispatch(x, w1, idx, pl, R, epr, cap, False)
    assert np.array_equal(oracle.combine(d["recv_x"], w1, idx, pl, epr, cap), x)
    # top-4 with one-hot weights over random (non-identity) expert rows: the output
    # is exactly the row of the selected (token, expert) -- pins the gather index
    k = 4
    idx = np.stack([rng.permutation(R * epr)[:k] for _ in range(T)]).astype(np.int32)
    pl = oracle.plan(idx, R, epr, cap)
    y = torch_bf16(rng.standard_normal((R, cap, H)).astype(np.float32))
    for jsel in range(k):
        w = np.zeros((T, k), np.float32)
        w[:, jsel] = 1.0
        out = oracle.combine(y, w, idx, pl, epr, cap)
        for t in range(T):
            r = idx[t, jsel] // epr
            assert np.array_equal(out[t], y[r, pl["slot"][t, jsel]])


def test_combine_random_rows_error_bound(oracle):
    # random expert rows and weights: the fp32 chain of k fmas is within
    # k * 2^-24 * sum|w y| of the exact sum, then one bf16 rounding
    rng = np.random.default_rng(11)
    wl = WORKLOADS["decode"].with_tokens(64, cap=64)
    inp = make_inputs(wl, 3)
    pl = oracle.plan(inp["indices"], wl.ranks, wl.experts_per_rank, wl.cap)
    y = torch_bf16(rng.standard_normal((wl.ranks, wl.cap, 512)).astype(np.float32))
    w = rng.uniform(-1, 1, size=inp["weights"].shape).astype(np.float32)
    out = bf16_f32(oracle.combine(y, w, inp["indices"], pl, wl.experts_per_rank, wl.cap))
    yf = bf16_f32(y).astype(np.float64)
    r = inp["indices"] // wl.experts_per_rank
    rows = yf[r, pl["slot"]]                    # [T, k, H]
    terms = w.astype(np.float64)[:, :, None] * rows
    exact = terms.sum(1)
    bound = wl.topk * 2.0 ** -24 * np.abs(terms).sum(1) + 0.5 * _ulp_bf16(out) * 1.0000001
    assert np.all(np.abs(out - exact) <= bound + 1e-45)


def test_fp8_path_combine_bound(oracle):
    # prefill stand-in: expert = dequant * 0.5, so out ~ 0.5 * x * sum(w) within
    # the FP8 bound (2^-4 relative, or scale * 2^-10 near zero) plus bf16 rounding
    wl, inp, pl, d = _dispatch(oracle, WORKLOADS["prefill"], 0, T=64)
    y = oracle.expert_dequant(d["recv_x"], d["recv_scales"], 0.5)
    out = bf16_f32(oracle.combine(y, inp["weights"], inp["indices"], pl,
                                  wl.experts_per_rank, wl.cap)).astype(np.float64)
    x = bf16_f32(inp["x"]).astype(np.float64)
    sw = inp["weights"].astype(np.float64).sum(1)[:, None]
    amax = np.abs(x.reshape(wl.tokens, -1, 128)).max(2)
    s = np.repeat(amax / 448.0, 128, axis=1)
    q_err = np.maximum(2.0 ** -4 * np.abs(x), s * 2.0 ** -10) * 1.000001
    bound = 0.5 * sw * (q_err + 2.0 ** -8 * np.abs(x)) + _ulp_bf16(out)
    assert np.all(np.abs(out - 0.5 * x * sw) <= bound)


# ----------------------------------------------------------------------------
# expert-major layout
# ----------------------------------------------------------------------------

def test_expert_major_layout(oracle):
    # a source rank other than 0, so that source positions carry its offset
    wl = WORKLOADS["stdmoe"].with_tokens(300)
    inp = make_inputs(wl, 4)
    src = 3
    pl = oracle.plan(inp["indices"], wl.ranks, wl.experts_per_rank, wl.cap, src)
    d = oracle.dispatch(inp["x"], inp["weights"], inp["indices"], pl, wl.ranks,
                        wl.experts_per_rank, wl.cap, True)
    em = oracle.to_expert_major(d, pl, wl.ranks, wl.experts_per_rank, wl.cap, wl.tokens,
                                wl.cap_em, src, fill=0x5A)
    idx = inp["indices"]
    T, k, E = wl.tokens, wl.topk, wl.experts
    q_all = np.stack([oracle.quant_row(inp["x"][t])[0] for t in range(T)])
    assert em["status"] == 0
    cnt = np.bincount(idx.ravel(), minlength=E)
    assert np.array_equal(em["em_counts"], cnt)
    assert cnt.sum() == T * k
    padded = (cnt + 127) // 128 * 128
    assert np.array_equal(em["em_offsets"], np.concatenate([[0], np.cumsum(padded)]))
    assert np.all(em["em_offsets"] % 128 == 0)
    # rows of expert e: its tokens in ascending order (stable sort of (t, e) by e)
    flat_e = idx.ravel()
    flat_t = np.repeat(np.arange(T), k)
    order = np.argsort(flat_e, kind="stable")
    starts = np.concatenate([[0], np.cumsum(cnt)])
    for e in range(E):
        toks = flat_t[order][starts[e]:starts[e + 1]]
        o = em["em_offsets"][e]
        # source position: the plan's encoding, src_rank * (R * cap) + token
        assert np.array_equal(em["em_src_pos"][o:o + cnt[e]],
                              src * wl.ranks * wl.cap + toks)
        assert np.array_equal(em["em_x"][o:o + cnt[e]], q_all[toks])
        # padding rows untouched
        assert np.all(em["em_x"][o + cnt[e]:em["em_offsets"][e + 1]] == 0x5A)
        for i, t in enumerate(toks):
            j = int(np.nonzero(idx[t] == e)[0][0])
            assert em["tok_em_row"][t, j] == o + i


def test_expert_major_combine_equals_rank_major(oracle):
    # identity stand-in on both layouts gives the same values in the same fma order
    wl = WORKLOADS["stdmoe"].with_tokens(200)
    wl = type(wl)(**{**wl.__dict__, "quant": "none"})
    inp = make_inputs(wl, 6)
    pl = oracle.plan(inp["indices"], wl.ranks, wl.experts_per_rank, wl.cap)
    d = oracle.dispatch(inp["x"], inp["weights"], inp["indices"], pl, wl.ranks,
                        wl.experts_per_rank, wl.cap, False)
    em = oracle.to_expert_major(d, pl, wl.ranks, wl.experts_per_rank, wl.cap, wl.tokens,
                                wl.cap_em)
    a = oracle.combine(d["recv_x"], inp["weights"], inp["indices"], pl, wl.experts_per_rank,
                       wl.cap)
    b = oracle.combine_em(em["em_x"], inp["weights"], em["tok_em_row"])
    assert np.array_equal(a, b)


def test_expert_major_overflow_status(oracle):
    wl = WORKLOADS["stdmoe"].with_tokens(64)
    inp = make_inputs(wl, 0)
    pl = oracle.plan(inp["indices"], wl.ranks, wl.experts_per_rank, wl.cap)
    d = oracle.dispatch(inp["x"], inp["weights"], inp["indices"], pl, wl.ranks,
                        wl.experts_per_rank, wl.cap, True)
    em = oracle.to_expert_major(d, pl, wl.ranks, wl.experts_per_rank, wl.cap, wl.tokens, 1000)
    assert em["status"] == oracle.ST_EM_OVERFLOW
    assert np.all(em["em_src_pos"][:1000] >= -1)


def test_combine_is_fused_chain_in_top_k_order(oracle):
    # With y in bf16 (8 significant bits) and w in fp32 (24 bits), w*y is exact in
    # float64, and adding an fp32 accumulator of nearby magnitude is exact too, so
    # float32(float64(w)*float64(y) + float64(acc)) is exactly fmaf(w, y, acc).
    # Magnitudes are bounded (|y| in [0.5, 2), w in [0.1, 1)) to keep that true.
    rng = np.random.default_rng(13)
    T, H, R, epr, k, cap = 256, 2048, 4, 4, 8, 256
    idx = np.stack([rng.permutation(R * epr)[:k] for _ in range(T)]).astype(np.int32)
    pl = oracle.plan(idx, R, epr, cap)
    mag = rng.uniform(0.5, 2.0, size=(R, cap, H)) * rng.choice([-1.0, 1.0], size=(R, cap, H))
    y = torch_bf16(mag.astype(np.float32))
    w = rng.uniform(0.1, 1.0, size=(T, k)).astype(np.float32)
    out = oracle.combine(y, w, idx, pl, epr, cap)
    rows = bf16_f32(y)[idx // epr, pl["slot"]]          # [T, k, H] fp32 values
    fused = np.zeros((T, H), np.float32)
    unfused = np.zeros((T, H), np.float32)
    for j in range(k):
        fused = (w[:, j, None].astype(np.float64) * rows[:, j].astype(np.float64)
                 + fused.astype(np.float64)).astype(np.float32)
        unfused = (unfused + (w[:, j, None] * rows[:, j]).astype(np.float32)).astype(np.float32)
    ref = torch_bf16(fused)
    assert np.array_equal(out, ref)
    # the data does tell a fused chain from a multiply-then-add chain
    assert np.count_nonzero(torch_bf16(unfused) != ref) > 0


def test_expert_major_combine_is_fused_chain_in_top_k_order(oracle):
    # As for the rank-major combine: each (t, j) reads its own expert-major row
    # (here an arbitrary distinct row), and the chain of exact fp32 fmas in
    # top-k order is computed in float64 with one rounding per step.
    rng = np.random.default_rng(17)
    T, H, k = 256, 1024, 8
    tok = rng.permutation(T * k).reshape(T, k).astype(np.int32)
    mag = rng.uniform(0.5, 2.0, size=(T * k, H)) * rng.choice([-1.0, 1.0], size=(T * k, H))
    y = torch_bf16(mag.astype(np.float32))
    w = rng.uniform(0.1, 1.0, size=(T, k)).astype(np.float32)
    out = oracle.combine_em(y, w, tok)
    rows = bf16_f32(y)[tok]                               # [T, k, H] fp32 values

    def chain(order, fused=True):
        acc = np.zeros((T, H), np.float32)
        for j in order:
            p = w[:, j, None].astype(np.float64) * rows[:, j].astype(np.float64)
            if fused:
                acc = (p + acc.astype(np.float64)).astype(np.float32)
            else:
                acc = (acc + p.astype(np.float32)).astype(np.float32)
        return torch_bf16(acc)

    ref = chain(range(k))
    assert np.array_equal(out, ref)
    # the data tells the top-k order and the fused chain from the alternatives
    assert np.count_nonzero(chain(range(k - 1, -1, -1)) != ref) > 0
    assert np.count_nonzero(chain(range(k), fused=False) != ref) > 0


# ----------------------------------------------------------------------------
# already-quantized FP8 payloads (carry) and standard-MoE dispatch
# ----------------------------------------------------------------------------

def test_carry_of_prequantized_rows_equals_quantising_dispatch(oracle):
    # Carrying rows that were quantised beforehand must land exactly what the
    # quantising dispatch writes: the two modes differ only in where R5 runs.
    wl = WORKLOADS["prefill"].with_tokens(160)
    inp = make_inputs(wl, 21)
    R, epr, cap = wl.ranks, wl.experts_per_rank, wl.cap
    pl = oracle.plan(inp["indices"], R, epr, cap)
    dq = oracle.dispatch(inp["x"], inp["weights"], inp["indices"], pl, R, epr, cap, 1, fill=0x33)
    rows = [oracle.quant_row(inp["x"][t]) for t in range(wl.tokens)]
    q = np.stack([r[0] for r in rows])
    s = np.stack([r[1] for r in rows])
    dc = oracle.dispatch(q, inp["weights"], inp["indices"], pl, R, epr, cap, 2, fill=0x33,
                         scales=s)
    for key in ("recv_x", "recv_scales", "recv_weights", "recv_indices"):
        assert np.array_equal(dq[key], dc[key]), key


@pytest.mark.parametrize("sd", [0, 3, 56])
def test_carry_copies_bytes_and_scale_rows(oracle, sd):
    # Any bytes (NaN and inf codes included) and any scale width travel unchanged
    # to the row of every distinct destination rank; other rows keep the fill.
    rng = np.random.default_rng(5 + sd)
    T, H, R, epr, k, cap = 70, 256, 4, 3, 3, 80
    idx = np.stack([rng.choice(R * epr, k, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k), dtype=np.float32)
    x = rng.integers(0, 256, (T, H), dtype=np.uint8)
    s = rng.standard_normal((T, sd)).astype(np.float32)
    pl = oracle.plan(idx, R, epr, cap)
    d = oracle.dispatch(x, w, idx, pl, R, epr, cap, 2, fill=0x77, scales=s)
    written = np.zeros((R, cap), dtype=bool)
    for t in range(T):
        for j in range(k):
            r = idx[t, j] // epr
            row = pl["slot"][t, j]
            written[r, row] = True
            assert np.array_equal(d["recv_x"][r, row], x[t])
            if sd:
                assert np.array_equal(d["recv_scales"][r, row], s[t])
            assert np.array_equal(d["recv_indices"][r, row], idx[t])
    assert np.all(d["recv_x"][~written] == 0x77)
    assert (d["recv_scales"] is None) == (sd == 0)


def test_standard_moe_by_brute_force(oracle):
    # Tiny case written out by hand: expert e's rows are the valid tokens naming
    # e, ascending, each once (a repeated id maps the first position); segments
    # start at multiples of 128; a token with an id outside [0, E) goes nowhere.
    rng = np.random.default_rng(8)
    T, H, R, epr, k, cap = 90, 128, 3, 2, 3, 96
    E = R * epr
    idx = rng.integers(0, E, (T, k)).astype(np.int32)  # repeats allowed
    idx[7, 1] = E          # bad id
    idx[40, 0] = -1        # bad id
    w = rng.random((T, k), dtype=np.float32)
    x = rng.integers(0, 1 << 16, (T, H), dtype=np.uint16)
    x &= np.uint16(0xBFFF)  # keep away from inf/NaN patterns
    cap_em = T * k + 127 * E
    em = oracle.dispatch_standard_moe(x, w, idx, R, epr, cap, 0, cap_em, fill=0x11)
    valid = [t for t in range(T) if np.all((idx[t] >= 0) & (idx[t] < E))]
    assert em["status"] & oracle.ST_BAD_INDEX
    assert em["status"] & oracle.ST_DUP_EXPERT
    off = 0
    for e in range(E):
        toks = [t for t in valid if e in idx[t]]
        assert em["em_counts"][e] == len(toks)
        assert em["em_offsets"][e] == off
        for i, t in enumerate(toks):
            assert em["em_src_pos"][off + i] == t
            assert np.array_equal(em["em_x"][off + i], x[t])
            j = int(np.nonzero(idx[t] == e)[0][0])
            assert em["tok_em_row"][t, j] == off + i
        off += (len(toks) + 127) // 128 * 128
    assert em["em_offsets"][E] == off
    for t in range(T):
        for j in range(k):
            first = t in valid and idx[t, j] not in idx[t, :j]
            assert (em["tok_em_row"][t, j] >= 0) == first


# ----------------------------------------------------------------------------
# FP4 (OCP MX: E2M1 elements, E8M0 block scales) and the FP8 direct cast
# ----------------------------------------------------------------------------

E2M1_MAGNITUDES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]  # OCP MX spec, FP4 E2M1


def test_e2m1_decode_table(oracle):
    tab = oracle.e2m1_decode_table()
    assert list(tab[:8]) == E2M1_MAGNITUDES
    assert list(tab[8:]) == [-m for m in E2M1_MAGNITUDES]
    assert np.signbit(tab[8])


def _e2m1_nearest(v):
    # brute force: the closest magnitude; on a tie the even code; sign kept
    mags = np.array(E2M1_MAGNITUDES)
    a = min(abs(v), 6.0)
    d = np.abs(mags - a)
    best = np.flatnonzero(d == d.min())
    c = int(best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0])
    return c | (8 if np.signbit(v) else 0)


def test_e2m1_encode_matches_brute_force(oracle):
    grid = np.arange(-8 * 64, 8 * 64 + 1) / 64.0  # every midpoint lies on this grid
    rng = np.random.default_rng(3)
    vals = np.concatenate([grid, rng.standard_normal(2000) * 3, [-0.0, 1e-30, -1e-30, 7.9, 100.0]])
    for v in vals:
        assert oracle.e2m1_encode(v) == _e2m1_nearest(v), v


def _bf16_of(v64):
    return torch_bf16(np.asarray(v64, dtype=np.float32))


def test_mx4_exact_blocks_round_trip(oracle):
    # Blocks built from E2M1 codes times 2^s, with a largest magnitude of 4 or 6,
    # quantise back to the same codes and to scale byte s + 127.
    rng = np.random.default_rng(17)
    H = 32 * 24
    codes = rng.integers(0, 16, H).astype(np.uint8)
    s = rng.integers(-100, 100, H // 32)
    for b in range(H // 32):
        codes[b * 32 + rng.integers(0, 32)] = rng.choice([6, 7, 14, 15])
    vals = np.array([oracle.e2m1_decode_table()[c] for c in codes]) * np.repeat(2.0 ** s, 32)
    x = _bf16_of(vals)
    assert np.array_equal(bf16_f32(x).astype(np.float64), vals)  # exact in bf16
    q, e8 = oracle.mx4_quant_row(x)
    assert np.array_equal(e8, (s + 127).astype(np.uint8))
    lo, hi = q & 0xF, q >> 4
    # a code of 8 (negative zero) decodes like 0: compare values, then signs
    assert np.array_equal(np.stack([lo, hi], 1).reshape(-1) & 7, codes & 7)
    assert np.array_equal(oracle.mx4_decode_row(q, e8), vals)


def test_mx4_scale_and_error_bound(oracle):
    wl = WORKLOADS["prefill"].with_tokens(24)
    x = make_inputs(wl, 9)["x"]
    rng = np.random.default_rng(2)
    x[3, :32] = 0                                       # zero block
    x[3, 32:64] = 0x8000                                # negative zeros
    x[4, :32] = _bf16_of(rng.standard_normal(32) * 2.0 ** -130)  # below the lowest scale
    x[5, :32] = _bf16_of(rng.standard_normal(32) * 2.0 ** 120)
    for t in range(wl.tokens):
        q, e8 = oracle.mx4_quant_row(x[t])
        v = bf16_f32(x[t]).astype(np.float64).reshape(-1, 32)
        amax = np.abs(v).max(1)
        with np.errstate(divide="ignore"):
            se = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1))) - 2, -127)
        se = np.clip(se, -127, 127)
        assert np.array_equal(e8.astype(np.int64), (se + 127).astype(np.int64))
        X = np.repeat(2.0 ** se, 32)
        dq = oracle.mx4_decode_row(q, e8)
        a = np.abs(v.reshape(-1)) / X
        half_step = np.where(a < 2, 0.25, np.where(a < 4, 0.5, 1.0))
        bound = np.where(a > 6, a - 6, half_step) * X
        assert np.all(np.abs(dq - v.reshape(-1)) <= bound)
        assert np.all(np.abs(dq) <= 6 * X)
    q, e8 = oracle.mx4_quant_row(x[3])
    assert e8[0] == 0 and e8[1] == 0
    assert np.all(q[:16] == 0) and np.all(q[16:32] == 0x88)


def test_mxfp4_dispatch_and_fp4_carry(oracle):
    wl = WORKLOADS["prefill"].with_tokens(96)
    inp = make_inputs(wl, 23)
    R, epr, cap = wl.ranks, wl.experts_per_rank, wl.cap
    pl = oracle.plan(inp["indices"], R, epr, cap)
    d4 = oracle.dispatch(inp["x"], inp["weights"], inp["indices"], pl, R, epr, cap, 4,
                         fill=0x3C)
    rows = [oracle.mx4_quant_row(inp["x"][t]) for t in range(wl.tokens)]
    assert d4["recv_x"].shape == (R, cap, wl.hidden // 2)
    assert d4["recv_scales"].shape == (R, cap, wl.hidden // 128)
    written = np.zeros((R, cap), bool)
    for t in range(wl.tokens):
        for j in range(wl.topk):
            r, s = inp["indices"][t, j] // epr, pl["slot"][t, j]
            written[r, s] = True
            assert np.array_equal(d4["recv_x"][r, s], rows[t][0])
            assert np.array_equal(d4["recv_scales"][r, s].view(np.uint8), rows[t][1])
    assert np.all(d4["recv_x"][~written] == 0x3C)
    # carrying the pre-quantised rows lands the same bytes
    q = np.stack([r[0] for r in rows])
    sw = np.stack([r[1] for r in rows]).view(np.float32)
    dc = oracle.dispatch(q, inp["weights"], inp["indices"], pl, R, epr, cap, 3, fill=0x3C,
                         scales=sw)
    assert np.array_equal(dc["recv_x"], d4["recv_x"])
    assert np.array_equal(dc["recv_scales"].view(np.uint32), d4["recv_scales"].view(np.uint32))


def test_fp8_direct_cast_combine(oracle):
    # Expert outputs that are E4M3 values already survive the cast, so the
    # combine of the cast rows equals the bf16 combine bit for bit; other
    # outputs stay within the cast's error: 2^-4 relative, 2^-10 absolute
    # below the smallest normal (half a subnormal step).
    wl = dataclasses.replace(WORKLOADS["decode"].with_tokens(64), ranks=4, experts_per_rank=8,
                             cap=64, hidden=1024)
    inp = make_inputs(wl, 31)
    R, epr, cap = wl.ranks, wl.experts_per_rank, wl.cap
    pl = oracle.plan(inp["indices"], R, epr, cap)
    rng = np.random.default_rng(4)
    codes = rng.integers(0, 254, (R, cap, wl.hidden)).astype(np.uint8)
    codes[codes >= 0x7F] += 1
    y = oracle.e4m3_to_bf16(codes)
    assert np.array_equal(oracle.cast_fp8_direct(y), codes)
    a = oracle.combine(y, inp["weights"], inp["indices"], pl, epr, cap)
    b = oracle.combine(oracle.e4m3_to_bf16(oracle.cast_fp8_direct(y)), inp["weights"],
                       inp["indices"], pl, epr, cap)
    assert np.array_equal(a, b)
    d = oracle.dispatch(inp["x"], inp["weights"], inp["indices"], pl, R, epr, cap, False)
    y2 = d["recv_x"]
    ref = bf16_f32(oracle.combine(y2, inp["weights"], inp["indices"], pl, epr, cap))
    got = bf16_f32(oracle.combine(oracle.e4m3_to_bf16(oracle.cast_fp8_direct(y2)),
                                  inp["weights"], inp["indices"], pl, epr, cap))
    wsum = np.abs(inp["weights"]).sum(1)[:, None]
    yabs = np.abs(bf16_f32(inp["x"]))
    bound = 2.0 ** -4 * wsum * yabs + 2.0 ** -10 * wsum + _ulp_bf16(ref) + _ulp_bf16(got)
    assert np.all(np.abs(got - ref) <= bound)
    big = oracle.cast_fp8_direct(_bf16_of(np.array([1000.0, -1000.0, 448.0, 464.0])))
    assert list(big) == [0x7E, 0xFE, 0x7E, 0x7E]  # saturates at +-448


# ----------------------------------------------------------------------------
# expert-major expert outputs back to the combine input (convert_combine_input)
# and the combine of converted rows ("MORI-EP User Guide" section 4)
# ----------------------------------------------------------------------------

def _read_golden_rows(name):
    """Golden file with float values; keys that repeat collect a row each."""
    d = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            d.setdefault(key, []).append([float(v) for v in vals])
    return d


def _em_of(oracle, idx, w, R, epr, cap, src=0, H=8, x=None):
    """Plan, bf16 dispatch and expert-major layout of the given routing."""
    T = idx.shape[0]
    if x is None:
        x = np.zeros((T, H), np.uint16)
    pl = oracle.plan(idx, R, epr, cap, src)
    d = oracle.dispatch(x, w, idx, pl, R, epr, cap, False)
    cap_em = T * idx.shape[1] + 127 * R * epr
    em = oracle.to_expert_major(d, pl, R, epr, cap, T, cap_em, src)
    return pl, d, em


def test_convert_combine_hand_worked_example(oracle):
    g = _read_golden_rows("convert_combine_tiny.txt")
    R, epr, k, cap, src = (int(g[n][0][0]) for n in ("R", "epr", "k", "cap", "src_rank"))
    idx = np.array(g["indices"][0], np.int32).reshape(-1, k)
    w = np.array(g["weights"][0], np.float32).reshape(-1, k)
    T, H = idx.shape[0], 2
    pl, d, em = _em_of(oracle, idx, w, R, epr, cap, src, H)
    # the layout the hand-worked rows assume
    assert list(em["em_counts"]) == [int(v) for v in g["em_counts"][0]]
    assert list(em["em_offsets"]) == [int(v) for v in g["em_offsets"][0]]
    for e in range(R * epr):
        toks = [int(v) for v in g[f"em_tokens_e{e}"][0]]
        o = em["em_offsets"][e]
        assert list(em["em_src_pos"][o:o + len(toks)]) == [src * R * cap + t for t in toks]
    # expert outputs at their rows; every other row is a NaN that would show
    y_em = np.full(em["em_x"].shape, 0x7FC0, np.uint16)
    for e, t, *v in g["y"]:
        e, t = int(e), int(t)
        toks = [int(u) for u in g[f"em_tokens_e{e}"][0]]
        y_em[em["em_offsets"][e] + toks.index(t)] = torch_bf16(np.array(v, np.float32))
    conv = oracle.convert_combine_input(y_em, em, d, pl, R, epr, cap, fill=0x7F80)
    for r, s, *v in g["conv"]:
        assert np.array_equal(conv[int(r), int(s)], torch_bf16(np.array(v, np.float32))), (r, s)
    assert np.all(conv[:, T:] == 0x7F80)  # rows past the counts are not written
    out = oracle.combine_rank_sum(conv, idx, pl, epr, cap)
    for t, *v in g["out"]:
        assert np.array_equal(out[int(t)], torch_bf16(np.array(v, np.float32))), t


def test_convert_combine_input_is_fused_chain_per_rank(oracle):
    # Each converted row is the chain of exact fp32 fmas, in top-k order, over
    # the row's positions on its own rank, with the dispatched weights.  The
    # reference reaches the expert-major rows through the token-side map
    # (tok_em_row), not through the source info the oracle searches, and forms
    # each step in float64 with one rounding to float32 (w*y is exact in
    # float64 and the magnitudes are bounded, so that is exactly fmaf).
    rng = np.random.default_rng(23)
    T, H, R, epr, k, cap, src = 256, 512, 4, 4, 8, 256, 2
    idx = np.stack([rng.permutation(R * epr)[:k] for _ in range(T)]).astype(np.int32)
    w = rng.uniform(0.1, 1.0, size=(T, k)).astype(np.float32)
    pl, d, em = _em_of(oracle, idx, w, R, epr, cap, src, H)
    mag = rng.uniform(0.5, 2.0, size=(em["em_x"].shape[0], H))
    y_em = torch_bf16((mag * rng.choice([-1.0, 1.0], size=mag.shape)).astype(np.float32))
    conv = oracle.convert_combine_input(y_em, em, d, pl, R, epr, cap)
    yv = bf16_f32(y_em)
    ranks = idx // epr

    def chain(order, fused=True):
        ref = {}
        for t in range(T):
            for r in np.unique(ranks[t]):
                acc = np.zeros(H, np.float32)
                for j in order:
                    if ranks[t, j] != r:
                        continue
                    p = np.float64(w[t, j]) * yv[em["tok_em_row"][t, j]].astype(np.float64)
                    if fused:
                        acc = (p + acc.astype(np.float64)).astype(np.float32)
                    else:
                        acc = (acc + p.astype(np.float32)).astype(np.float32)
                ref[(int(r), int(pl["slot"][t, list(ranks[t]).index(r)]))] = torch_bf16(acc)
        return ref

    ref = chain(range(k))
    assert len(ref) == int(pl["recv_counts"].sum())
    for (r, s), v in ref.items():
        assert np.array_equal(conv[r, s], v), (r, s)
    # the data tells the top-k order and the fused chain from the alternatives
    rev, unf = chain(range(k - 1, -1, -1)), chain(range(k), fused=False)
    assert any(not np.array_equal(rev[key], v) for key, v in ref.items())
    assert any(not np.array_equal(unf[key], v) for key, v in ref.items())


def test_convert_undoes_the_expert_major_layout(oracle):
    # Unit weights and every token's experts on distinct ranks: a received row
    # holds one expert, so converting the expert-major copies of the received
    # rows gives the received rows back bit for bit (fmaf(1, y, +0) = y).
    rng = np.random.default_rng(29)
    T, H, R, epr, k, cap = 300, 256, 8, 4, 4, 300
    ranks = np.stack([rng.permutation(R)[:k] for _ in range(T)])
    idx = (ranks * epr + rng.integers(0, epr, size=(T, k))).astype(np.int32)
    x = torch_bf16(rng.standard_normal((T, H)).astype(np.float32))
    w = np.ones((T, k), np.float32)
    pl, d, em = _em_of(oracle, idx, w, R, epr, cap, 0, H, x)
    conv = oracle.convert_combine_input(em["em_x"], em, d, pl, R, epr, cap, fill=0x5A5A)
    for r in range(R):
        n = int(pl["recv_counts"][r])
        assert np.array_equal(conv[r, :n], d["recv_x"][r, :n])
        assert np.all(conv[r, n:] == 0x5A5A)


def test_convert_then_rank_sum_equals_expert_major_combine_on_exact_data(oracle):
    # With dyadic values of few bits every fp32 step is exact, so converting and
    # adding the rank rows must give exactly the expert-major combine (the top-k
    # weighted sum over the experts each token names once).  Tokens naming one
    # expert twice are included: the expert counts once on both sides.
    rng = np.random.default_rng(31)
    T, H, R, epr, k, cap = 200, 64, 4, 3, 6, 200
    idx = np.stack([rng.permutation(R * epr)[:k] for _ in range(T)]).astype(np.int32)
    idx[::7, 3] = idx[::7, 1]                      # repeated experts
    w = rng.choice([0.125, 0.25, 0.375, 0.5, 0.75], size=(T, k)).astype(np.float32)
    pl, d, em = _em_of(oracle, idx, w, R, epr, cap, 1, H)
    assert pl["status"] == oracle.ST_DUP_EXPERT
    vals = np.array([-3, -2, -1.5, -1, -0.5, 0, 0.5, 1, 1.5, 2, 3, 4], np.float32)
    y_em = torch_bf16(rng.choice(vals, size=(em["em_x"].shape[0], H)))
    conv = oracle.convert_combine_input(y_em, em, d, pl, R, epr, cap)
    got = oracle.combine_rank_sum(conv, idx, pl, epr, cap)
    ref = oracle.combine_em(y_em, w, em["tok_em_row"])
    assert np.array_equal(got, ref)
    # and it is the plain weighted sum, each named expert once
    yv = bf16_f32(y_em).astype(np.float64)
    for t in range(T):
        s = np.zeros(H)
        for j in range(k):
            if idx[t, j] not in idx[t, :j]:
                s += np.float64(w[t, j]) * yv[em["tok_em_row"][t, j]]
        assert np.array_equal(bf16_f32(got[t]).astype(np.float64), s), t


def test_convert_then_rank_sum_identity_round_trip(oracle):
    # Identity experts: every output is x * (sum of the token's weights) up to
    # the two roundings of the path (each within half a bf16 ulp of a term of
    # one sign), so within 2 ulp of the float64 value.
    wl = WORKLOADS["stdmoe"].with_tokens(256)
    wl = dataclasses.replace(wl, quant="none", ranks=8, experts_per_rank=4, hidden=256)
    inp = make_inputs(wl, 5)
    idx, w = inp["indices"], inp["weights"]
    pl, d, em = _em_of(oracle, idx, w, wl.ranks, wl.experts_per_rank, wl.cap, 0, wl.hidden,
                       inp["x"])
    conv = oracle.convert_combine_input(em["em_x"], em, d, pl, wl.ranks, wl.experts_per_rank,
                                        wl.cap)
    out = bf16_f32(oracle.combine_rank_sum(conv, idx, pl, wl.experts_per_rank, wl.cap))
    want = bf16_f32(inp["x"]).astype(np.float64) * w.astype(np.float64).sum(1)[:, None]
    ulp = np.exp2(np.floor(np.log2(np.abs(want) + 1e-300)) - 7)
    assert np.all(np.abs(out - want) <= 2 * ulp)


def test_combine_rank_sum_adds_rank_rows_in_first_position_order(oracle):
    # Rows of widely different magnitudes, so that fp32 addition order shows:
    # the reference adds each token's distinct rank rows with float32 numpy
    # additions (one rounding each) in the order of their first top-k position.
    rng = np.random.default_rng(37)
    T, H, R, epr, k, cap = 128, 64, 8, 2, 6, 128
    idx = np.stack([rng.permutation(R * epr)[:k] for _ in range(T)]).astype(np.int32)
    pl = oracle.plan(idx, R, epr, cap)
    big = rng.choice([2.0 ** 30, -2.0 ** 30, 1.0, -1.0, 2.0 ** 12], size=(R, cap, H))
    y_rm = torch_bf16(big.astype(np.float32))
    out = oracle.combine_rank_sum(y_rm, idx, pl, epr, cap)
    yv = bf16_f32(y_rm)

    def ref(order):
        res = np.empty((T, H), np.uint16)
        for t in range(T):
            rs = []
            for j in range(k):
                r = int(idx[t, j]) // epr
                if r not in [q for q, _ in rs]:
                    rs.append((r, int(pl["slot"][t, j])))
            acc = np.zeros(H, np.float32)
            for i in order(len(rs)):
                acc = acc + yv[rs[i][0], rs[i][1]]
            res[t] = torch_bf16(acc)
        return res

    fwd = ref(lambda n: range(n))
    assert np.array_equal(out, fwd)
    assert np.count_nonzero(ref(lambda n: range(n - 1, -1, -1)) != fwd) > 0
