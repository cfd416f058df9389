"""The device conversions of the path over every input they take.

The kernels' fp32 -> bf16 round-to-nearest-even (every combine output) and
fp32 -> OCP E4M3 (every quantised dispatch code) run through the library's
codec probes over all fp32 bit patterns in their domain, chunk by chunk on the
device; the MX FP4 block encoder (every MEP_QUANT_MXFP4 dispatch code and
scale) runs over every finite bf16 value under every block exponent it can
take.  The sampled probe tests compare against the oracle; here the
references are definitions that need no sampling:

- bf16: round to nearest even on the bit pattern of a finite float (add
  0x7FFF plus the lowest kept bit, keep the top 16 bits), which also rounds
  the largest finite values to infinity;
- E4M3: torch's CPU cast to float8_e4m3fn (round to nearest even; an oracle
  pin checks the oracle's encoder against the same cast), for every pattern
  whose magnitude is at most 448 * (1 + 2^-23) -- the largest quotient a
  quantising dispatch can form (amax / (amax / 448));
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
