// Small launches: a device copy for route inspection, probes that run the
// kernels' own device conversions over caller arrays, and a streaming probe
// that measures what HBM gives a given mix of reads and writes.
#include "dev.h"
#include "mep_internal.h"
#include "payload.h"

namespace mep {

namespace {

__global__ void copy_i32_kernel(const int32_t* src, int32_t* dst, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

__global__ void probe_e4m3_kernel(const float* in, uint8_t* out, int64_t n) {
  const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i + 3 < n) {
    const uint32_t w = pack_e4m3x4(in[i], in[i + 1], in[i + 2], in[i + 3]);
    for (int b = 0; b < 4; ++b) out[i + b] = (uint8_t)(w >> (8 * b));
  } else {
    for (int64_t j = i; j < n; ++j) out[j] = (uint8_t)pack_e4m3x4(in[j], 0.0f, 0.0f, 0.0f);
  }
}

// MX FP4 blocks (32 bf16 columns) through the dispatch's own block encoder:
// 2 lanes per block, 16 columns each, as in a dispatch wave; 16 code bytes
// and one scale byte per block.
__global__ void probe_mxfp4_kernel(const u32x4* in, u32x2* q, uint8_t* e8, int64_t nblocks) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t b = g >> 1;
  const int part = (int)(g & 1);
  if (b >= nblocks) return;  // both lanes of a block leave together
  uint32_t e = 0;
  q[g] = quant_mx4_half(in[2 * g], in[2 * g + 1], e);
  if (part == 0) e8[b] = (uint8_t)e;
}

// FP8 blocks (128 bf16 columns) through the dispatch's own block encoder:
// 8 lanes per block, 16 columns each, as in a dispatch wave; 128 code bytes
// and one fp32 scale per block.
__global__ void probe_fp8_block_kernel(const u32x4* in, u32x4* q, float* scales,
                                       int64_t nblocks) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t b = g >> 3;
  const int part = (int)(g & 7);
  if (b >= nblocks) return;  // all 8 lanes of a block leave together
  float scale = 0.0f;
  q[b * 8 + part] = quant16(in[b * 16 + part * 2], in[b * 16 + part * 2 + 1], scale);
  if (part == 0) scales[b] = scale;
}

__global__ void probe_bf16_kernel(const float* in, uint16_t* out, int64_t n) {
  const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 2;
  if (i + 1 < n) {
    const uint32_t w = pack_bf16_rne(in[i], in[i + 1]);
    out[i] = (uint16_t)w;
    out[i + 1] = (uint16_t)(w >> 16);
  } else if (i < n) {
    out[i] = (uint16_t)pack_bf16_rne(in[i], 0.0f);
  }
}

// Streaming probe: `waves` waves share rd reads and wr writes of 1 KiB units
// (64 lanes x 16 bytes) as evenly as the counts allow: with rd = rq*waves + rr,
// wave g reads rq units, plus one if g < rr, from a contiguous run of src
// starting at unit g*rq + min(g, rr); writes likewise (quotients and
// remainders come from the host, so no wave divides).  Loads are non-temporal
// and all issued before the stores (at most kProbeMaxRd units per wave,
// checked on the host); the stored words fold in every loaded word, so no
// load can be dropped.
constexpr int kProbeMaxRd = 16;

struct ProbeShare {
  int64_t q, r;  // units per wave and waves taking one more
  __device__ __forceinline__ void range(int64_t g, int64_t& u0, int64_t& u1) const {
    u0 = g * q + (g < r ? g : r);
    u1 = u0 + q + (g < r ? 1 : 0);
  }
};

__global__ __launch_bounds__(256) void stream_probe_kernel(const u32x4* src, u32x4* dst,
                                                           int64_t waves, ProbeShare rd,
                                                           ProbeShare wr) {
  const int lane = threadIdx.x & 63;
  const int64_t g = first_lane(blockIdx.x * 4 + (threadIdx.x >> 6));
  if (g >= waves) return;
  int64_t r0, r1, w0, w1;
  rd.range(g, r0, r1);
  wr.range(g, w0, w1);
  u32x4 in[kProbeMaxRd];
#pragma unroll
  for (int i = 0; i < kProbeMaxRd; ++i) {
    in[i] = u32x4{0, 0, 0, 0};
    if (r0 + i < r1) in[i] = __builtin_nontemporal_load(src + (r0 + i) * kWave + lane);
  }
  u32x4 acc = u32x4{(uint32_t)g, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < kProbeMaxRd; ++i) acc ^= in[i];
  for (int64_t u = w0; u < w1; ++u) {
    acc[1] += 1u;
    store_nt(dst + u * kWave + lane, acc);
  }
  if (w0 == w1 && lane == 0 && acc[0] == 0xFFFFFFFFu && acc[1] == 0xFFFFFFFFu)
    dst[0] = acc;  // a read-only wave's loads must stay live; practically never taken
}

}  // namespace

hipError_t launch_stream_probe(const void* src, void* dst, int64_t waves, int64_t rd_units,
                               int64_t wr_units, hipStream_t s) {
  if (waves == 0) return hipSuccess;
  const int64_t blocks = (waves + 3) / 4;
  const ProbeShare rd{rd_units / waves, rd_units % waves};
  const ProbeShare wr{wr_units / waves, wr_units % waves};
  stream_probe_kernel<<<(unsigned)blocks, 256, 0, s>>>(reinterpret_cast<const u32x4*>(src),
                                                        reinterpret_cast<u32x4*>(dst), waves, rd,
                                                        wr);
  return hipGetLastError();
}

int stream_probe_max_units() { return kProbeMaxRd; }

hipError_t launch_copy_i32(const int32_t* src, int32_t* dst, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int blocks = (int)std::min<int64_t>((n + 255) / 256, 1024);
  copy_i32_kernel<<<blocks, 256, 0, s>>>(src, dst, n);
  return hipGetLastError();
}

hipError_t launch_probe_e4m3(const float* in, uint8_t* out, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int64_t threads = (n + 3) / 4;
  probe_e4m3_kernel<<<(unsigned)((threads + 255) / 256), 256, 0, s>>>(in, out, n);
  return hipGetLastError();
}

hipError_t launch_probe_mxfp4(const uint16_t* in, uint8_t* q, uint8_t* e8, int64_t nblocks,
                              hipStream_t s) {
  if (nblocks == 0) return hipSuccess;
  const int64_t threads = nblocks * 2;
  probe_mxfp4_kernel<<<(unsigned)((threads + 255) / 256), 256, 0, s>>>(
      reinterpret_cast<const u32x4*>(in), reinterpret_cast<u32x2*>(q), e8, nblocks);
  return hipGetLastError();
}

hipError_t launch_probe_fp8_block(const uint16_t* in, uint8_t* q, float* scales, int64_t nblocks,
                                  hipStream_t s) {
  if (nblocks == 0) return hipSuccess;
  const int64_t threads = nblocks * 8;
  probe_fp8_block_kernel<<<(unsigned)((threads + 255) / 256), 256, 0, s>>>(
      reinterpret_cast<const u32x4*>(in), reinterpret_cast<u32x4*>(q), scales, nblocks);
  return hipGetLastError();
}

hipError_t launch_probe_bf16(const float* in, uint16_t* out, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int64_t threads = (n + 1) / 2;
  probe_bf16_kernel<<<(unsigned)((threads + 255) / 256), 256, 0, s>>>(in, out, n);
  return hipGetLastError();
}

}  // namespace mep
