// The C ABI used from a plain host program, without Python or torch: device
// memory comes from the HIP runtime, the routing plan, dispatch and combine
// run through the mep_* entry points on the default stream, and every output
// is compared with the CPU oracle (test infrastructure, linked into this test
// program only).  Inputs come from a splitmix64 counter generator (Steele,
// Lea and Flood, "Fast Splittable Pseudorandom Number Generators", 2014), used
// for the inputs only.
//
// Exit status 0 when every case matches: counts, source positions, receive
// rows, weights, ids and scales bit for bit (unwritten receive rows keep their
// fill byte), combine within 1 bf16 ulp.
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <chrono>
#include <vector>

#include "mep.h"

extern "C" {
int32_t oracle_plan(const int32_t* idx, int32_t T, int32_t k, int32_t R, int32_t epr, int32_t cap,
                    int32_t src_rank, int32_t* recv_counts, int32_t* src_token_pos,
                    int32_t* slot);
void oracle_dispatch(const void* x, const float* xs, int32_t sd, const float* w,
                     const int32_t* idx, const int32_t* slot, int32_t T, int32_t H, int32_t k,
                     int32_t R, int32_t epr, int32_t cap, int32_t quant, void* recv_x,
                     float* recv_scales, float* recv_w, int32_t* recv_idx, uint8_t* q_tmp,
                     float* s_tmp);
void oracle_combine(const uint16_t* y, const float* w, const int32_t* idx, const int32_t* slot,
                    int32_t T, int32_t H, int32_t k, int32_t epr, int32_t cap, uint16_t* out);
}

static uint64_t g_state;
static uint64_t next64() {
  uint64_t z = (g_state += 0x9e3779b97f4a7c15ull);
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}
static uint32_t below(uint32_t n) { return (uint32_t)(next64() % n); }

#define HIP_OK(x)                                                         \
  do {                                                                    \
    hipError_t e_ = (x);                                                  \
    if (e_ != hipSuccess) {                                               \
      fprintf(stderr, "HIP error %s at %s:%d\n", hipGetErrorString(e_), \
              __FILE__, __LINE__);                                        \
      exit(2);                                                            \
    }                                                                     \
  } while (0)

template <class T>
static T* dev_alloc(size_t n, int fill) {
  void* p = nullptr;
  const size_t bytes = n * sizeof(T) > 0 ? n * sizeof(T) : 16;
  HIP_OK(hipMalloc(&p, bytes));
  HIP_OK(hipMemset(p, fill, bytes));
  return (T*)p;
}

template <class T>
static std::vector<T> to_host(const T* d, size_t n) {
  std::vector<T> h(n);
  if (n) HIP_OK(hipMemcpy(h.data(), d, n * sizeof(T), hipMemcpyDeviceToHost));
  return h;
}

static int bf16_ulp(uint16_t a, uint16_t b) {
  const int ia = (a & 0x8000) ? -(int)(a & 0x7fff) : (int)(a & 0x7fff);
  const int ib = (b & 0x8000) ? -(int)(b & 0x7fff) : (int)(b & 0x7fff);
  return abs(ia - ib);
}

// One case; returns the number of mismatches found.
static int run_case(const char* name, int H, int T, int R, int epr, int k, int cap, int quant,
                    int src_rank, bool fused, uint64_t seed) {
  g_state = seed;
  const int E = R * epr;
  const bool fp8 = quant == MEP_QUANT_FP8_E4M3_BLOCK128;
  const int nb = fp8 ? H / 128 : 0;
  const size_t rowb = fp8 ? (size_t)H : (size_t)H * 2;

  // inputs: finite bf16 values of magnitude in [2^-7, 2^8), k distinct
  // experts per token, positive weights
  std::vector<uint16_t> x((size_t)T * H);
  for (auto& v : x)
    v = (uint16_t)(((next64() & 1) << 15) | ((120 + below(15)) << 7) | below(128));
  std::vector<int32_t> idx((size_t)T * k);
  for (int t = 0; t < T; ++t)
    for (int j = 0; j < k; ++j) {
      int e;
      bool again;
      do {
        e = (int)below((uint32_t)E);
        again = false;
        for (int jj = 0; jj < j; ++jj) again |= idx[(size_t)t * k + jj] == e;
      } while (again);
      idx[(size_t)t * k + j] = e;
    }
  std::vector<float> w((size_t)T * k);
  for (auto& v : w) v = (float)((next64() >> 40) + 1) / (float)(1ull << 24);

  // GPU
  mep_config cfg{H, nb, epr, k, cap, R, src_rank, quant};
  const size_t wsb = mep_workspace_bytes(&cfg);
  if (wsb == 0) { fprintf(stderr, "%s: config rejected\n", name); return 1; }
  unsigned char* ws = dev_alloc<unsigned char>(wsb, 0);
  mep_handle* h = nullptr;
  if (mep_create(&cfg, ws, wsb, &h) != MEP_OK) { fprintf(stderr, "%s: create\n", name); return 1; }
  uint16_t* d_x = dev_alloc<uint16_t>(x.size(), 0);
  int32_t* d_idx = dev_alloc<int32_t>(idx.size(), 0);
  float* d_w = dev_alloc<float>(w.size(), 0);
  HIP_OK(hipMemcpy(d_x, x.data(), x.size() * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_idx, idx.data(), idx.size() * 4, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_w, w.data(), w.size() * 4, hipMemcpyHostToDevice));
  int32_t* d_counts = dev_alloc<int32_t>(R, 0xA5);
  int32_t* d_spos = dev_alloc<int32_t>((size_t)R * cap, 0xA5);
  unsigned char* d_rx = dev_alloc<unsigned char>((size_t)R * cap * rowb, 0xA5);
  float* d_rs = fp8 ? dev_alloc<float>((size_t)R * cap * nb, 0xA5) : nullptr;
  float* d_rw = dev_alloc<float>((size_t)R * cap * k, 0xA5);
  int32_t* d_ri = dev_alloc<int32_t>((size_t)R * cap * k, 0xA5);
  uint16_t* d_out = dev_alloc<uint16_t>((size_t)T * H, 0xA5);
  int rc;
  if (fused) {
    rc = mep_plan_dispatch(h, d_idx, T, d_counts, d_spos, d_x, d_w, nullptr, d_rx, d_rs, d_rw,
                           d_ri, nullptr);
  } else {
    rc = mep_plan(h, d_idx, T, d_counts, d_spos, nullptr);
    if (rc == MEP_OK)
      rc = mep_dispatch(h, d_x, d_w, nullptr, d_idx, d_rx, d_rs, d_rw, d_ri, nullptr);
  }
  if (rc != MEP_OK) { fprintf(stderr, "%s: dispatch rc %d\n", name, rc); return 1; }
  // identity expert on bf16 rows: the combine reads the receive buffer itself
  if (!fp8) {
    rc = mep_combine(h, MEP_RANK_MAJOR, d_rx, d_w, d_out, nullptr);
    if (rc != MEP_OK) { fprintf(stderr, "%s: combine rc %d\n", name, rc); return 1; }
  }
  int32_t st = -1;
  rc = mep_get_status(h, nullptr, &st);
  if (rc != MEP_OK || st != 0) { fprintf(stderr, "%s: status %d/%d\n", name, rc, st); return 1; }
  auto g_counts = to_host(d_counts, R);
  auto g_spos = to_host(d_spos, (size_t)R * cap);
  auto g_rx = to_host(d_rx, (size_t)R * cap * rowb);
  auto g_rs = fp8 ? to_host(d_rs, (size_t)R * cap * nb) : std::vector<float>();
  auto g_rw = to_host(d_rw, (size_t)R * cap * k);
  auto g_ri = to_host(d_ri, (size_t)R * cap * k);
  auto g_out = to_host(d_out, (size_t)T * H);
  mep_reset(h, nullptr);
  mep_destroy(h);
  for (void* p : {(void*)ws, (void*)d_x, (void*)d_idx, (void*)d_w, (void*)d_counts,
                  (void*)d_spos, (void*)d_rx, (void*)d_rs, (void*)d_rw, (void*)d_ri,
                  (void*)d_out})
    if (p) HIP_OK(hipFree(p));

  // oracle
  std::vector<int32_t> o_counts(R), o_spos((size_t)R * cap, 0), slot((size_t)T * k);
  const int32_t ost = oracle_plan(idx.data(), T, k, R, epr, cap, src_rank, o_counts.data(),
                                  o_spos.data(), slot.data());
  std::vector<unsigned char> o_rx((size_t)R * cap * rowb, 0);
  std::vector<float> o_rs((size_t)R * cap * (nb ? nb : 1)), o_rw((size_t)R * cap * k);
  std::vector<int32_t> o_ri((size_t)R * cap * k);
  std::vector<uint8_t> q_tmp(H);
  std::vector<float> s_tmp(nb ? nb : 1);
  oracle_dispatch(x.data(), nullptr, 0, w.data(), idx.data(), slot.data(), T, H, k, R, epr, cap,
                  fp8 ? 1 : 0, o_rx.data(), o_rs.data(), o_rw.data(), o_ri.data(), q_tmp.data(),
                  s_tmp.data());
  std::vector<uint16_t> o_out((size_t)T * H);
  if (!fp8)
    oracle_combine((const uint16_t*)o_rx.data(), w.data(), idx.data(), slot.data(), T, H, k, epr,
                   cap, o_out.data());

  // compare
  int bad = ost != 0;
  for (int r = 0; r < R; ++r) {
    if (g_counts[r] != o_counts[r]) { ++bad; continue; }
    for (int s = 0; s < cap; ++s) {
      const size_t row = (size_t)r * cap + s;
      const bool written = s < o_counts[r];
      const unsigned char* gr = g_rx.data() + row * rowb;
      if (!written) {
        for (size_t b = 0; b < rowb; ++b) bad += gr[b] != 0xA5;
        continue;
      }
      bad += g_spos[row] != o_spos[row];
      bad += memcmp(gr, o_rx.data() + row * rowb, rowb) != 0;
      bad += memcmp(&g_rw[row * k], &o_rw[row * k], 4 * (size_t)k) != 0;
      bad += memcmp(&g_ri[row * k], &o_ri[row * k], 4 * (size_t)k) != 0;
      if (fp8) bad += memcmp(&g_rs[row * nb], &o_rs[row * nb], 4 * (size_t)nb) != 0;
    }
  }
  int max_ulp = 0;
  if (!fp8)
    for (size_t i = 0; i < g_out.size(); ++i) {
      const int u = bf16_ulp(g_out[i], o_out[i]);
      if (u > max_ulp) max_ulp = u;
    }
  bad += max_ulp > 1;
  int U = 0;
  for (int r = 0; r < R; ++r) U += o_counts[r];
  printf("%-28s H=%d T=%d R=%d k=%d %s %s: U=%d mismatches=%d combine max ulp=%s\n", name, H, T,
         R, k, fp8 ? "fp8" : "bf16", fused ? "fused" : "separate", U, bad,
         fp8 ? "-" : (max_ulp ? "1" : "0"));
  fflush(stdout);
  return bad;
}

// Host time of the C ABI calls themselves (argument checks and kernel
// submission, no Python): 100 back-to-back calls of the 128-token x 7168 decode
// shape, few enough that the queue never blocks the host; the GPU work is
// waited for outside the timed region.  Median of 20 repeats, microseconds per
// call.
static void host_cost() {
  const int H = 7168, T = 128, R = 8, epr = 32, k = 8, cap = 128, n = 100;
  g_state = 5;
  std::vector<uint16_t> x((size_t)T * H, 0x3f80);
  std::vector<int32_t> idx((size_t)T * k);
  for (int t = 0; t < T; ++t)
    for (int j = 0; j < k; ++j) idx[(size_t)t * k + j] = (t * 37 + j * 32) % (R * epr);
  std::vector<float> w((size_t)T * k, 0.125f);
  mep_config cfg{H, 0, epr, k, cap, R, 0, MEP_QUANT_NONE};
  const size_t wsb = mep_workspace_bytes(&cfg);
  unsigned char* ws = dev_alloc<unsigned char>(wsb, 0);
  mep_handle* h = nullptr;
  if (mep_create(&cfg, ws, wsb, &h) != MEP_OK) { fprintf(stderr, "create\n"); exit(1); }
  uint16_t* d_x = dev_alloc<uint16_t>(x.size(), 0);
  int32_t* d_idx = dev_alloc<int32_t>(idx.size(), 0);
  float* d_w = dev_alloc<float>(w.size(), 0);
  HIP_OK(hipMemcpy(d_x, x.data(), x.size() * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_idx, idx.data(), idx.size() * 4, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_w, w.data(), w.size() * 4, hipMemcpyHostToDevice));
  int32_t* d_counts = dev_alloc<int32_t>(R, 0);
  int32_t* d_spos = dev_alloc<int32_t>((size_t)R * cap, 0);
  uint16_t* d_rx = dev_alloc<uint16_t>((size_t)R * cap * H, 0);
  float* d_rw = dev_alloc<float>((size_t)R * cap * k, 0);
  int32_t* d_ri = dev_alloc<int32_t>((size_t)R * cap * k, 0);
  uint16_t* d_out = dev_alloc<uint16_t>((size_t)T * H, 0);
  auto pd = [&]() {
    return mep_plan_dispatch(h, d_idx, T, d_counts, d_spos, d_x, d_w, nullptr, d_rx, nullptr,
                             d_rw, d_ri, nullptr);
  };
  auto cb = [&]() { return mep_combine(h, MEP_RANK_MAJOR, d_rx, d_w, d_out, nullptr); };
  for (int i = 0; i < 50; ++i)
    if (pd() != MEP_OK || cb() != MEP_OK) { fprintf(stderr, "call failed\n"); exit(1); }
  HIP_OK(hipDeviceSynchronize());
  std::vector<double> t_pd, t_cb;
  for (int rep = 0; rep < 20; ++rep) {
    auto t0 = std::chrono::steady_clock::now();
    for (int i = 0; i < n; ++i) pd();
    auto t1 = std::chrono::steady_clock::now();
    HIP_OK(hipDeviceSynchronize());
    auto t2 = std::chrono::steady_clock::now();
    for (int i = 0; i < n; ++i) cb();
    auto t3 = std::chrono::steady_clock::now();
    HIP_OK(hipDeviceSynchronize());
    t_pd.push_back(std::chrono::duration<double, std::micro>(t1 - t0).count() / n);
    t_cb.push_back(std::chrono::duration<double, std::micro>(t3 - t2).count() / n);
  }
  std::sort(t_pd.begin(), t_pd.end());
  std::sort(t_cb.begin(), t_cb.end());
  printf("host us per call (C, decode 128 x 7168): plan_dispatch %.2f combine %.2f\n",
         t_pd[t_pd.size() / 2], t_cb[t_cb.size() / 2]);
  mep_destroy(h);
  for (void* p : {(void*)ws, (void*)d_x, (void*)d_idx, (void*)d_w, (void*)d_counts,
                  (void*)d_spos, (void*)d_rx, (void*)d_rw, (void*)d_ri, (void*)d_out})
    HIP_OK(hipFree(p));
}

int main(int argc, char** argv) {
  if (argc > 1 && strcmp(argv[1], "--host-cost") == 0) {
    host_cost();
    return 0;
  }
  int bad = 0;
  bad += run_case("ragged bf16", 256, 37, 4, 2, 2, 40, MEP_QUANT_NONE, 1, true, 1);
  bad += run_case("ragged bf16", 256, 37, 4, 2, 2, 40, MEP_QUANT_NONE, 1, false, 2);
  bad += run_case("fp8 two-launch plan", 512, 300, 8, 4, 4, 300, MEP_QUANT_FP8_E4M3_BLOCK128, 7,
                  true, 3);
  bad += run_case("decode 128 x 7168", 7168, 128, 8, 32, 8, 128, MEP_QUANT_NONE, 0, true, 4);
  printf(bad ? "c_abi FAILED\n" : "c_abi ok\n");
  return bad ? 1 : 0;
}
