// Host-side driver for the C ABI's argument and state checks, built with the
// host sanitizers (AddressSanitizer, UndefinedBehaviorSanitizer) on the host
// code only.  Without a GPU it runs every check that precedes a device call;
// with one it also drives a small cache through create, prefill, decode, read
// and destroy.  Prints "abi checks ok" and exits 0 when every status matches.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstring>
#include <vector>

#include "h2o.h"

static int g_fail = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      std::printf("FAILED %s:%d: %s\n", __FILE__, __LINE__, #cond);    \
      ++g_fail;                                                        \
    }                                                                  \
  } while (0)

static h2o_params base() {
  h2o_params p;
  std::memset(&p, 0, sizeof(p));
  p.batch = 2;
  p.heads = 3;
  p.head_dim = 128;
  p.heavy_budget = 8;
  p.recent_budget = 8;
  p.dtype = H2O_BF16;
  p.scale = 0.f;
  p.max_prompt = 64;
  p.rope_base = 0.f;
  return p;
}

int main() {
  // parameter validation (no device call)
  size_t kv = 0, tot = 0;
  h2o_params p = base();
  EXPECT(h2o_cache_bytes(&p, &kv, &tot) == H2O_OK && kv == size_t{2} * 6 * 16 * 128 * 2 && tot > kv);
  EXPECT(h2o_cache_bytes(nullptr, &kv, &tot) == H2O_ERR_INVALID_ARG);
  p = base(); p.batch = 0;            EXPECT(h2o_cache_bytes(&p, nullptr, nullptr) == H2O_ERR_INVALID_ARG);
  p = base(); p.head_dim = 96;        EXPECT(h2o_cache_bytes(&p, nullptr, nullptr) == H2O_ERR_UNSUPPORTED);
  p = base(); p.heavy_budget = -1;    EXPECT(h2o_cache_bytes(&p, nullptr, nullptr) == H2O_ERR_INVALID_ARG);
  p = base(); p.heavy_budget = 0; p.recent_budget = 0;
  EXPECT(h2o_cache_bytes(&p, nullptr, nullptr) == H2O_ERR_INVALID_ARG);
  p = base(); p.heavy_budget = 12288; EXPECT(h2o_cache_bytes(&p, nullptr, nullptr) == H2O_ERR_UNSUPPORTED);
  p = base(); p.dtype = (h2o_dtype)7; EXPECT(h2o_cache_bytes(&p, nullptr, nullptr) == H2O_ERR_INVALID_ARG);
  p = base(); p.scale = 1.f / 0.f;    EXPECT(h2o_cache_bytes(&p, nullptr, nullptr) == H2O_ERR_INVALID_ARG);
  p = base(); p.max_prompt = -1;      EXPECT(h2o_cache_bytes(&p, nullptr, nullptr) == H2O_ERR_INVALID_ARG);
  p = base(); p.rope_base = -2.f;     EXPECT(h2o_cache_bytes(&p, nullptr, nullptr) == H2O_ERR_INVALID_ARG);
  p = base(); p.batch = 1 << 16; p.heads = 1 << 10; p.max_prompt = 4096;
  EXPECT(h2o_cache_bytes(&p, nullptr, nullptr) == H2O_ERR_INVALID_ARG);
  p = base(); p.max_prompt = 1 << 24; EXPECT(h2o_cache_bytes(&p, nullptr, nullptr) == H2O_ERR_INVALID_ARG);
  p = base(); p.rope_base = 10000.f;  EXPECT(h2o_cache_bytes(&p, nullptr, &tot) == H2O_OK);
  EXPECT(std::strlen(h2o_last_error()) > 0);
  for (int s = 0; s <= 6; ++s) EXPECT(h2o_status_str((h2o_status)s) != nullptr);

  // NULL handles: rejected before any device call
  h2o_cache* c = nullptr;
  EXPECT(h2o_cache_create(nullptr, -1, &c) == H2O_ERR_INVALID_ARG && c == nullptr);
  p = base();
  EXPECT(h2o_cache_create(&p, -1, nullptr) == H2O_ERR_INVALID_ARG);
  EXPECT(h2o_cache_create(&p, -3, &c) == H2O_ERR_INVALID_ARG && c == nullptr);
  EXPECT(h2o_cache_destroy(nullptr) == H2O_OK);
  EXPECT(h2o_prefill(nullptr, nullptr, nullptr, nullptr, 0, nullptr, nullptr) == H2O_ERR_INVALID_ARG);
  EXPECT(h2o_decode_step(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == H2O_ERR_INVALID_ARG);
  EXPECT(h2o_decode_steps(nullptr, nullptr, nullptr, nullptr, 1, nullptr, 0, nullptr, nullptr) ==
         H2O_ERR_INVALID_ARG);
  EXPECT(h2o_cache_read(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == H2O_ERR_INVALID_ARG);
  EXPECT(h2o_prefill_stats_read(nullptr, nullptr, nullptr, nullptr) == H2O_ERR_INVALID_ARG);
  EXPECT(h2o_cache_info(nullptr, nullptr, nullptr, nullptr) == H2O_ERR_INVALID_ARG);
  EXPECT(h2o_column_scores(nullptr, nullptr, nullptr, 4, nullptr, nullptr) == H2O_ERR_INVALID_ARG);
  EXPECT(h2o_cache_set_pattern(nullptr, 1, 4, 1) == H2O_ERR_INVALID_ARG);
  EXPECT(h2o_prefill_scored(nullptr, nullptr, nullptr, 4, 4, nullptr, nullptr) == H2O_ERR_INVALID_ARG);
  EXPECT(h2o_decode_step_scored(nullptr, nullptr, nullptr, nullptr, nullptr, 1, nullptr, nullptr, nullptr) ==
         H2O_ERR_INVALID_ARG);
  EXPECT(h2o_column_scores_noalloc(nullptr, nullptr, nullptr, 4, nullptr, nullptr) == H2O_ERR_INVALID_ARG);
  p = base(); p.rope_base = 1.f;
  EXPECT(h2o_column_scores_noalloc(&p, nullptr, nullptr, 4, nullptr, nullptr) == H2O_ERR_UNSUPPORTED);
  p = base();
  EXPECT(h2o_column_scores_noalloc(&p, nullptr, nullptr, -1, nullptr, nullptr) == H2O_ERR_INVALID_ARG);
  EXPECT(h2o_column_scores_noalloc(&p, nullptr, nullptr, 0, nullptr, nullptr) == H2O_OK);
  EXPECT(h2o_probe_read(nullptr, 16, nullptr, nullptr) == H2O_ERR_INVALID_ARG);

  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev == 0) {
    std::printf("abi checks ok (%s)\n", g_fail ? "with failures" : "no GPU: argument checks only");
    return g_fail ? 1 : 0;
  }

  // with a GPU: one small cache end to end, plus the state checks that need a cache
  p = base();
  const size_t units = 6, L = 40, d = 128, T = 30;
  EXPECT(h2o_cache_create(&p, -1, &c) == H2O_OK && c != nullptr);
  void *q = nullptr, *k = nullptr, *v = nullptr, *qs = nullptr, *out = nullptr, *ev = nullptr;
  EXPECT(hipMalloc(&q, units * L * d * 2) == hipSuccess);
  EXPECT(hipMalloc(&k, units * L * d * 2) == hipSuccess);
  EXPECT(hipMalloc(&v, units * L * d * 2) == hipSuccess);
  EXPECT(hipMalloc(&qs, units * d * 2) == hipSuccess);
  EXPECT(hipMalloc(&out, units * d * 4) == hipSuccess);
  EXPECT(hipMalloc(&ev, units * 4) == hipSuccess);
  std::vector<uint16_t> h(units * L * d);
  for (size_t i = 0; i < h.size(); ++i) h[i] = static_cast<uint16_t>(0x3c00u + (i * 2654435761u >> 25) % 256u);
  EXPECT(hipMemcpy(q, h.data(), h.size() * 2, hipMemcpyHostToDevice) == hipSuccess);
  EXPECT(hipMemcpy(k, h.data(), h.size() * 2, hipMemcpyHostToDevice) == hipSuccess);
  EXPECT(hipMemcpy(v, h.data(), h.size() * 2, hipMemcpyHostToDevice) == hipSuccess);
  EXPECT(hipMemcpy(qs, h.data(), units * d * 2, hipMemcpyHostToDevice) == hipSuccess);
  EXPECT(h2o_decode_step(c, qs, qs, qs, static_cast<float*>(out), nullptr, nullptr) == H2O_ERR_STATE);
  EXPECT(h2o_prefill_stats_read(c, nullptr, nullptr, nullptr) == H2O_ERR_STATE);
  EXPECT(h2o_prefill(c, q, k, v, 65, nullptr, nullptr) == H2O_ERR_INVALID_ARG);  // above max_prompt
  EXPECT(h2o_prefill(c, static_cast<char*>(q) + 2, k, v, 8, nullptr, nullptr) == H2O_ERR_INVALID_ARG);
  EXPECT(h2o_prefill(c, q, k, v, static_cast<int32_t>(L), nullptr, nullptr) == H2O_OK);
  for (size_t t = 0; t < T / 2; ++t)
    EXPECT(h2o_decode_step(c, qs, qs, qs, static_cast<float*>(out), static_cast<int32_t*>(ev), nullptr) == H2O_OK);
  EXPECT(h2o_decode_steps(c, q, k, v, -1, static_cast<float*>(out), 0, nullptr, nullptr) == H2O_ERR_INVALID_ARG);
  EXPECT(h2o_decode_steps(c, q, k, v, static_cast<int32_t>(T - T / 2), static_cast<float*>(out), 0, nullptr,
                          nullptr) == H2O_OK);
  std::vector<int32_t> pos(units * 16), meta(2);
  std::vector<float> score(units * 16), lse(units * L), cs(units * L);
  std::vector<uint16_t> ks(units * 16 * d), vs(units * 16 * d);
  EXPECT(h2o_cache_read(c, pos.data(), score.data(), ks.data(), vs.data(), meta.data(), nullptr) == H2O_OK);
  EXPECT(meta[0] == 16 && meta[1] == static_cast<int32_t>(L + T));
  EXPECT(h2o_prefill_stats_read(c, lse.data(), cs.data(), nullptr) == H2O_OK);
  int32_t cnt = 0, nxt = 0, pl = 0;
  EXPECT(h2o_cache_info(c, &cnt, &nxt, &pl) == H2O_OK && cnt == 16 && pl == static_cast<int32_t>(L));
  EXPECT(h2o_cache_set_pattern(c, H2O_PATTERN_FIXED, 4, 5) == H2O_ERR_INVALID_ARG);
  EXPECT(h2o_cache_destroy(c) == H2O_OK);
  for (void* ptr : {q, k, v, qs, out, ev}) EXPECT(hipFree(ptr) == hipSuccess);
  std::printf("abi checks ok (%s)\n", g_fail ? "with failures" : "GPU: argument, state and end-to-end checks");
  return g_fail ? 1 : 0;
}
