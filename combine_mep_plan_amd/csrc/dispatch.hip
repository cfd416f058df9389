// Dispatch: scatter each token's row (bf16 copy, or OCP E4M3 codes with one
// fp32 scale per 128 columns) plus its k weights and k expert ids into the
// receive buffer of every distinct destination rank, at the slot the plan
// assigned.
//
// Source: "MORI-EP User Guide", section 3 dispatch() (outputs: received rows,
// weights, scales, indices); "Choosing an EP API and backend": the gfx950 FP8
// flavour is OCP E4M3.  The block-scale rule (scale = amax / 448 per 128
// columns, code = E4M3(x / scale), round to nearest even) is this library's
// reading; the pages do not print the format.
//
// One wavefront per token.  The row is read from HBM once and held in
// registers; each destination then receives 16-byte-per-lane stores (1 KiB
// per wave instruction, fully coalesced).  Receive rows are written with
// non-temporal stores: they are not read again by this launch.
#include "dev.h"
#include "mep_internal.h"

namespace mep {

namespace {

// Token row metadata: k weights and k expert ids, one lane per top-k entry.
__device__ __forceinline__ void store_meta(const DispatchArgs& a, int t, int row, int lane) {
  if (lane < a.k) {
    a.recv_w[(size_t)row * a.k + lane] = a.w[(size_t)t * a.k + lane];
    a.recv_idx[(size_t)row * a.k + lane] = a.idx[(size_t)t * a.k + lane];
  }
}

template <int UNROLL>
__global__ __launch_bounds__(256) void dispatch_bf16_kernel(DispatchArgs a) {
  const int lane = threadIdx.x & 63;
  int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  t = first_lane(t);
  const uint32_t first = a.ufirst[t];
  if (first == 0) return;  // token not dispatched (bad expert id)
  const int nv = a.H / 8;  // 16-byte vectors per row
  const u32x4* src = reinterpret_cast<const u32x4*>(a.x) + (size_t)t * nv;
  const int32_t* rr = a.rrow + (size_t)t * a.k;
  u32x4* dst_base = reinterpret_cast<u32x4*>(a.recv_x);
  for (int v0 = 0; v0 < nv; v0 += kWave * UNROLL) {
    u32x4 buf[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int v = v0 + u * kWave + lane;
      if (v < nv) buf[u] = src[v];
    }
    for (uint32_t m = first; m; m &= m - 1) {
      const int row = rr[__builtin_ctz(m)];
      u32x4* dst = dst_base + (size_t)row * nv;
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const int v = v0 + u * kWave + lane;
        if (v < nv) store_nt(dst + v, buf[u]);
      }
    }
  }
  for (uint32_t m = first; m; m &= m - 1) store_meta(a, t, rr[__builtin_ctz(m)], lane);
}

// FP8: each lane owns 16 consecutive columns (32 input bytes -> 16 code bytes);
// 8 neighbouring lanes cover one 128-column scale block.
template <int UNROLL>
__global__ __launch_bounds__(256) void dispatch_fp8_kernel(DispatchArgs a) {
  const int lane = threadIdx.x & 63;
  int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  t = first_lane(t);
  const uint32_t first = a.ufirst[t];
  if (first == 0) return;
  const int nu = a.H / 16;   // 16-column units per row
  const int nb = a.H / 128;  // scale blocks per row
  const u32x4* src = reinterpret_cast<const u32x4*>(a.x) + (size_t)t * (a.H / 8);
  const int32_t* rr = a.rrow + (size_t)t * a.k;
  u32x4* qbase = reinterpret_cast<u32x4*>(a.recv_x);
  for (int v0 = 0; v0 < nu; v0 += kWave * UNROLL) {
    u32x4 in0[UNROLL], in1[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int v = v0 + u * kWave + lane;
      if (v < nu) { in0[u] = src[2 * v]; in1[u] = src[2 * v + 1]; }
      else { in0[u] = u32x4{0, 0, 0, 0}; in1[u] = u32x4{0, 0, 0, 0}; }
    }
    u32x4 q[UNROLL];
    float scale[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      float f[16];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f[2 * i] = bf16_lo(in0[u][i]);
        f[2 * i + 1] = bf16_hi(in0[u][i]);
        f[8 + 2 * i] = bf16_lo(in1[u][i]);
        f[8 + 2 * i + 1] = bf16_hi(in1[u][i]);
      }
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(f[i]));
      // lanes 8m..8m+7 share a block; units past the row end hold amax 0 and
      // never leave their own 8-lane group (nu is a multiple of 8)
      amax = fmaxf(amax, __shfl_xor(amax, 1));
      amax = fmaxf(amax, __shfl_xor(amax, 2));
      amax = fmaxf(amax, __shfl_xor(amax, 4));
      const float s = amax / 448.0f;
      scale[u] = s;
      uint32_t w[4];
      if (s == 0.0f) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          w[i] = ((__float_as_uint(f[4 * i]) >> 31) << 7) |
                 ((__float_as_uint(f[4 * i + 1]) >> 31) << 15) |
                 ((__float_as_uint(f[4 * i + 2]) >> 31) << 23) |
                 ((__float_as_uint(f[4 * i + 3]) >> 31) << 31);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          w[i] = pack_e4m3x4(f[4 * i] / s, f[4 * i + 1] / s, f[4 * i + 2] / s, f[4 * i + 3] / s);
      }
      q[u] = u32x4{w[0], w[1], w[2], w[3]};
    }
    for (uint32_t m = first; m; m &= m - 1) {
      const int row = rr[__builtin_ctz(m)];
      u32x4* dq = qbase + (size_t)row * nu;
      float* ds = a.recv_scales + (size_t)row * nb;
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const int v = v0 + u * kWave + lane;
        if (v < nu) {
          store_nt(dq + v, q[u]);
          if ((v & 7) == 0) ds[v >> 3] = scale[u];
        }
      }
    }
  }
  for (uint32_t m = first; m; m &= m - 1) store_meta(a, t, rr[__builtin_ctz(m)], lane);
}

}  // namespace

hipError_t launch_dispatch(const DispatchArgs& a, bool fp8, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const int blocks = (a.T + 3) / 4;
  if (fp8) dispatch_fp8_kernel<7><<<blocks, 256, 0, s>>>(a);
  else dispatch_bf16_kernel<14><<<blocks, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mep
