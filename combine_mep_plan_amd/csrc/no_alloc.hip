// The fused routing plan + dispatch for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid allocation): no handle and no workspace argument.  The plan's
// scratch -- per-token rank masks, the per-chunk and per-block count
// prefixes, the receive row of every (token, top-k position), first-occurrence
// bits and two status words -- lives in a file-scope device array of
// kScratchBytes that every GPU the library runs on holds until the process
// ends.  The kernels are those of mep_plan_dispatch.
#include <mutex>

#include "mep_internal.h"

namespace {

constexpr size_t kScratchBytes = (size_t)2 << 20;  // 2 MiB per GPU
constexpr int kMaxDevices = 64;

// In host code this name is a host-side stand-in, not a device address: the
// kernels get the address hipGetSymbolAddress returns for the current GPU.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_lock;
void* g_scratch[kMaxDevices];  // device address of each GPU's copy, looked up once

// The device address of GPU dev's scratch, looked up on first use with that
// GPU current (the caller's current device is restored).
int scratch_address(int dev, unsigned char** out) {
  if (dev < 0 || dev >= kMaxDevices) return MEP_ERR_HIP;
  std::lock_guard<std::mutex> guard(g_lock);
  if (!g_scratch[dev]) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return MEP_ERR_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return MEP_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return MEP_ERR_HIP;
    if (e != hipSuccess || !p) return MEP_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = static_cast<unsigned char*>(g_scratch[dev]);
  return MEP_OK;
}

// Sections of the scratch for a batch of T tokens (each 256-byte aligned);
// the kernels index them by token and chunk only, never by capacity.
struct ScratchLayout {
  size_t status, chunk_cnt, block_cnt, mask, rrow, ufirst, total;
};

ScratchLayout scratch_layout(int64_t T, int64_t k, int64_t R) {
  ScratchLayout L{};
  const int64_t C = (T + mep::kChunk - 1) / mep::kChunk;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = (off + bytes + 255) & ~(size_t)255;
    return o;
  };
  L.status = take(2 * sizeof(uint32_t));
  L.chunk_cnt = take((size_t)(C * R) * sizeof(int32_t));
  L.block_cnt = take((size_t)((C + mep::kMinBlockChunks - 1) / mep::kMinBlockChunks * R) * sizeof(int32_t));
  L.mask = take((size_t)T * sizeof(uint64_t));
  L.rrow = take((size_t)(T * k) * sizeof(int32_t));
  L.ufirst = take((size_t)T * sizeof(uint32_t));
  L.total = off;
  return L;
}

}  // namespace

extern "C" int mep_plan_dispatch_noalloc(const mep_config* cfg, const int32_t* indices, int32_t T,
                                         int32_t* recv_counts, int32_t* src_token_pos,
                                         const void* x, const float* weights, const float* scales,
                                         void* recv_x, float* recv_scales, float* recv_weights,
                                         int32_t* recv_indices, void* stream) {
  int rc = mep::check_config(cfg);
  if (rc != MEP_OK) return rc;
  const mep::RankDiv rd = mep::make_rdiv(cfg->num_experts_per_rank);
  if (mep::check_rank_map(*cfg, rd) != MEP_OK) return MEP_ERR_CONFIG;
  rc = mep::check_plan_args(*cfg, indices, T, recv_counts, src_token_pos);
  if (rc != MEP_OK) return rc;
  rc = mep::check_dispatch_args(*cfg, T, x, weights, scales, indices, recv_x, recv_scales,
                                recv_weights, recv_indices);
  if (rc != MEP_OK) return rc;
  const ScratchLayout L =
      scratch_layout(T, cfg->num_experts_per_token, cfg->world_size);
  if (L.total > kScratchBytes) return MEP_ERR_SHAPE;
  const hipStream_t s = (hipStream_t)stream;
  int dev = -1;
  if ((s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev)) != hipSuccess) return MEP_ERR_HIP;
  unsigned char* base = nullptr;
  rc = scratch_address(dev, &base);
  if (rc != MEP_OK) return rc;
  mep::WsPtrs w{};
  w.status = reinterpret_cast<uint32_t*>(base + L.status);  // ORed into, never read back
  w.status_next = w.status + 1;                             // cleared by the plan
  w.tok_status = nullptr;
  w.chunk_cnt = reinterpret_cast<int32_t*>(base + L.chunk_cnt);
  w.block_cnt = reinterpret_cast<int32_t*>(base + L.block_cnt);
  w.mask = reinterpret_cast<uint64_t*>(base + L.mask);
  w.rrow = reinterpret_cast<int32_t*>(base + L.rrow);
  w.ufirst = reinterpret_cast<uint32_t*>(base + L.ufirst);
  const mep::PlanArgs p = mep::plan_args(*cfg, rd, w, indices, T, recv_counts, src_token_pos);
  mep::DispatchArgs a = mep::dispatch_args(*cfg, rd, w, T, x, weights, scales, indices, recv_x,
                                           recv_scales, recv_weights, recv_indices);
  a.recv_counts = recv_counts;
  a.spos = src_token_pos;
  return mep::launch_plan_dispatch(p, a, s) == hipSuccess ? MEP_OK : MEP_ERR_HIP;
}
