"""The two device conversions of the path over every input they take.

The kernels' fp32 -> bf16 round-to-nearest-even (every combine output) and
fp32 -> OCP E4M3 (every quantised dispatch code) run through the library's
codec probes over all fp32 bit patterns in their domain, chunk by chunk on the
device.  The sampled probe tests compare against the oracle; here the
references are definitions that need no sampling:

- bf16: round to nearest even on the bit pattern of a finite float (add
  0x7FFF plus the lowest kept bit, keep the top 16 bits), which also rounds
  the largest finite values to infinity;
- E4M3: torch's CPU cast to float8_e4m3fn (round to nearest even; an oracle
  pin checks the oracle's encoder against the same cast), for every pattern
  whose magnitude is at most 448 * (1 + 2^-23) -- the largest quotient a
  quantising dispatch can form (amax / (amax / 448)).

Source: "Choosing an EP API and backend" (OCP E4M3 on gfx950; the HIP
backend's combine gathers in BF16 or FP32).
"""

import numpy as np
import pytest
import torch

import combine_mep_plan_amd as M

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
