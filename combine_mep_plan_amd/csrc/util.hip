// Small launches: a device copy for route inspection, the status-word clear of
// captured iterations, and probes that run the kernels' own device conversions
// over caller arrays.
#include "dev.h"
#include "mep_internal.h"

namespace mep {

namespace {

__global__ void copy_i32_kernel(const int32_t* src, int32_t* dst, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

__global__ void clear_word_kernel(uint32_t* word) { *word = 0u; }

__global__ void probe_e4m3_kernel(const float* in, uint8_t* out, int64_t n) {
  const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i + 3 < n) {
    const uint32_t w = pack_e4m3x4(in[i], in[i + 1], in[i + 2], in[i + 3]);
    for (int b = 0; b < 4; ++b) out[i + b] = (uint8_t)(w >> (8 * b));
  } else {
    for (int64_t j = i; j < n; ++j) out[j] = (uint8_t)pack_e4m3x4(in[j], 0.0f, 0.0f, 0.0f);
  }
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

}  // namespace

hipError_t launch_copy_i32(const int32_t* src, int32_t* dst, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int blocks = (int)std::min<int64_t>((n + 255) / 256, 1024);
  copy_i32_kernel<<<blocks, 256, 0, s>>>(src, dst, n);
  return hipGetLastError();
}

hipError_t launch_clear_word(uint32_t* word, hipStream_t s) {
  clear_word_kernel<<<1, 1, 0, s>>>(word);
  return hipGetLastError();
}

hipError_t launch_probe_e4m3(const float* in, uint8_t* out, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int64_t threads = (n + 3) / 4;
  probe_e4m3_kernel<<<(unsigned)((threads + 255) / 256), 256, 0, s>>>(in, out, n);
  return hipGetLastError();
}

hipError_t launch_probe_bf16(const float* in, uint16_t* out, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int64_t threads = (n + 1) / 2;
  probe_bf16_kernel<<<(unsigned)((threads + 255) / 256), 256, 0, s>>>(in, out, n);
  return hipGetLastError();
}

}  // namespace mep
