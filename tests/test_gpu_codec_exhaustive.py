"""The device conversions of the path over every input they take.

The kernels' fp32 -> bf16 round-to-nearest-even (every combine output) and
fp32 -> OCP E4M3 (every quantised dispatch code) run through the library's
codec probes over all fp32 bit patterns in their domain, chunk by chunk on the
device; the FP8 block encoder (every MEP_QUANT_FP8_E4M3_BLOCK128 dispatch
code and scale) over every pair of a finite bf16 value and a bf16 block amax
at least its magnitude, and the MX FP4 block encoder (every MEP_QUANT_MXFP4
dispatch code and scale) over every finite bf16 value under every block
exponent it can take.  The sampled probe tests compare against the oracle; here the
references are definitions that need no sampling:

- bf16: round to nearest even on the bit pattern of a finite float (add
  0x7FFF plus the lowest kept bit, keep the top 16 bits), which also rounds
  the largest finite values to infinity;
- E4M3: torch's CPU cast to float8_e4m3fn (round to nearest even; an oracle
  pin checks the oracle's encoder against the same cast), for every pattern
  whose magnitude is at most 448 * (1 + 2^-23) -- the largest quotient a
  quantising dispatch can form (amax / (amax / 448));
- FP8 blocks: scale = fp32(amax / 448) and quotient = fp32(x / scale), both
  formed in fp64 and rounded once to fp32 -- which is the correctly rounded
  fp32 result here, because an 8-bit bf16 numerator over an fp32 denominator
  (or over 448) never comes within 2^-53 of an fp32 rounding midpoint
  without being one, and never is one -- then the device E4M3 conversion
  checked above;
- MX FP4: the oracle's block quantiser (its E2M1 encoder is pinned against
  the format's table and exact midpoints on the CPU).

Source: "Choosing an EP API and backend" (OCP E4M3 on gfx950; the HIP
backend's combine gathers in BF16 or FP32).
"""

import numpy as np
import pytest
import torch

import combine_mep_plan_amd as M
from oracle import oracle as O

pytestmark = pytest.mark.gpu


def _floats(bits64):
    """fp32 values with the given bit patterns (int64 in [0, 2^32))."""
    return (bits64 - (bits64 >= 2**31).to(torch.int64) * 2**32).to(torch.int32).view(torch.float32)


def test_bf16_conversion_every_finite_input():
    step = 1 << 27
    for lo in range(0, 1 << 32, step):
        b = torch.arange(lo, lo + step, dtype=torch.int64, device="cuda")
        v = _floats(b)
        out = torch.empty(step, dtype=torch.int16, device="cuda")
        M.mep_probe_bf16(v, out, step)
        finite = (b & 0x7F800000) != 0x7F800000
        inf = ((b & 0x7FFFFFFF) == 0x7F800000)
        ref = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) & 0xFFFF
        ref = torch.where(inf, b >> 16, ref)
        got = out.to(torch.int64) & 0xFFFF
        bad = ((got != ref) & (finite | inf)).nonzero()
        assert bad.numel() == 0, [(hex(int(b[i])), hex(int(got[i])), hex(int(ref[i])))
                                  for i in bad[:8, 0].tolist()]
        del b, v, out, finite, inf, ref, got
    torch.cuda.synchronize()


def test_e4m3_conversion_every_input_in_the_quotient_range():
    top = int(np.float32(448.0).view(np.uint32)) + 1  # 448 * (1 + 2^-23)
    step = 1 << 26
    for sign in (0, 1 << 31):
        for lo in range(0, top + 1, step):
            hi = min(lo + step, top + 1)
            b = torch.arange(lo, hi, dtype=torch.int64, device="cuda") + sign
            v = _floats(b)
            n = hi - lo
            out = torch.empty(n, dtype=torch.uint8, device="cuda")
            M.mep_probe_e4m3(v, out, n)
            ref = v.cpu().to(torch.float8_e4m3fn).view(torch.uint8)
            got = out.cpu()
            bad = (got != ref).nonzero()
            assert bad.numel() == 0, [(float(v[i]), hex(int(got[i])), hex(int(ref[i])))
                                      for i in bad[:8, 0].tolist()]
            del b, v, out, ref, got
    torch.cuda.synchronize()


def test_mxfp4_block_encoder_every_value_under_every_exponent():
    """Blocks [A, v1..v31]: A = the largest bf16 magnitude of binade B sets the
    block exponent (B = 0..254: every exponent -127..125, subnormal amax
    included); the v run over every finite bf16 value with |v| <= A, both signs,
    so each value meets every exponent under which it can occur, saturation
    range [6, 8) included."""
    blocks = []
    for B in range(255):
        A = (B << 7) | 0x7F
        mags = np.arange(A + 1, dtype=np.uint16)
        vals = np.concatenate([mags, mags | np.uint16(0x8000)])
        pad = (-vals.size) % 31
        vals = np.concatenate([vals, np.zeros(pad, np.uint16)]).reshape(-1, 31)
        head = np.full((vals.shape[0], 1), A, np.uint16)
        blocks.append(np.concatenate([head, vals], axis=1))
    x = np.ascontiguousarray(np.concatenate(blocks))  # [nblocks, 32] bf16 bits
    nb = x.shape[0]
    q_ref, e8_ref = O.mx4_quant_row(x.reshape(-1))
    xd = torch.from_numpy(x.view(np.int16)).cuda()
    q = torch.empty(nb * 16, dtype=torch.uint8, device="cuda")
    e8 = torch.empty(nb, dtype=torch.uint8, device="cuda")
    M.mep_probe_mxfp4(xd, q, e8, nb)
    torch.cuda.synchronize()
    got_q, got_e8 = q.cpu().numpy(), e8.cpu().numpy()
    bad = np.nonzero(got_e8 != np.asarray(e8_ref).reshape(-1))[0]
    assert bad.size == 0, [(int(i), int(got_e8[i]), int(e8_ref[i])) for i in bad[:8]]
    bad = np.nonzero(got_q != np.asarray(q_ref).reshape(-1))[0]
    assert bad.size == 0, [(int(i) // 16, hex(int(got_q[i])), hex(int(q_ref[i]))) for i in bad[:8]]


def _fp8_blocks(A):
    """Blocks [A, v1..v127] for amax patterns A (int64, positive finite bf16):
    the v run over every bf16 value with |v| <= A, both signs, zero-padded."""
    nb = (2 * (A + 1) + 126) // 127
    total = int(nb.sum())
    blk_a = torch.repeat_interleave(A, nb)
    start = torch.repeat_interleave(torch.cumsum(nb, 0) - nb, nb)
    within = torch.arange(total, device=A.device) - start
    idx = within[:, None] * 127 + torch.arange(127, device=A.device)[None, :]
    a = blk_a[:, None]
    v = torch.where(idx <= a, idx, 0x8000 + idx - a - 1)
    v = torch.where(idx < 2 * (a + 1), v, torch.zeros_like(v))
    return torch.cat([a, v], dim=1)  # [blocks, 128] bf16 bit patterns as int64


def test_fp8_block_encoder_every_value_under_every_amax():
    """1.07e9 (value, amax) pairs: every positive finite bf16 amax (and zero),
    with every bf16 value of magnitude up to it, through the dispatch's block
    encoder (which divides by the scale through its reciprocal and two
    remainder corrections for scales >= 2^-60, by IEEE division below)."""
    amax_all = np.arange(0, 0x7F80, dtype=np.int64)
    nb_all = (2 * (amax_all + 1) + 126) // 127
    per_chunk = 1 << 20  # blocks per device pass
    lo = 0
    while lo < amax_all.size:
        hi = lo + max(1, int(np.searchsorted(np.cumsum(nb_all[lo:]), per_chunk, side="right")))
        bits = _fp8_blocks(torch.from_numpy(amax_all[lo:hi]).cuda())
        nb = bits.shape[0]
        x = _floats(bits << 16)  # [nb,128] fp32 values of the bf16 patterns
        s_ref = (x[:, 0].double() / 448.0).float()
        q_ref = (x.double() / s_ref.double()[:, None]).float()
        q_ref = torch.where(s_ref[:, None] == 0, x, q_ref)  # all-zero block: signed zeros
        codes_ref = torch.empty(q_ref.shape, dtype=torch.uint8, device="cuda")
        M.mep_probe_e4m3(q_ref.contiguous(), codes_ref, q_ref.numel())
        x16 = (bits - 65536 * (bits >= 32768).to(torch.int64)).to(torch.int16).contiguous()
        codes = torch.empty((nb, 128), dtype=torch.uint8, device="cuda")
        scales = torch.empty(nb, dtype=torch.float32, device="cuda")
        M.mep_probe_fp8_block(x16, codes, scales, nb)
        bad = (scales.view(torch.int32) != s_ref.view(torch.int32)).nonzero()
        assert bad.numel() == 0, [(hex(int(bits[i, 0])), float(scales[i]), float(s_ref[i]))
                                  for i in bad[:8, 0].tolist()]
        bad = (codes != codes_ref).nonzero()
        assert bad.numel() == 0, [(hex(int(bits[i, 0])), hex(int(bits[i, j])), hex(int(codes[i, j])),
                                   hex(int(codes_ref[i, j])))
                                  for i, j in bad[:8].tolist()]
        del bits, x, s_ref, q_ref, codes_ref, x16, codes, scales
        lo = hi
    torch.cuda.synchronize()
