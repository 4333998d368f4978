// The cache object behind the C ABI declared in include/h2o.h: parameter and
// state validation, up-front device allocation, host-side step counters, and
// launch orchestration.  Every check runs before any GPU call, so a rejected
// call leaves the cache unchanged.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "h2o.h"
#include "launch.h"

struct h2o_cache {
  h2o_params p;
  int device;
  int32_t d, k, units, esize;
  int32_t kstride;  // per-unit stride of score/comp/pos: k rounded up to 32 entries
  float scale, c2;
  // host-side state
  int32_t count;       // entries cached per unit
  int32_t next_pos;    // position of the next token
  int32_t prompt_len;  // last prompt length, -1 before the first prefill
  int32_t lpad_cap;    // row capacity of the prefill scratch (multiple of 32)
  int32_t lpad_last;   // row stride of the last prefill's statistics
  bool stats_valid;    // the prefill scratch holds the last h2o_prefill's statistics
  int32_t pat_kind, pat_period, pat_width;  // sparse pattern kept before heavy hitters
  // device memory
  void* kslots;
  void* vslots;
  float* score;
  float* comp;
  int32_t* pos;
  float* part;
  float* logits;
  // split path, several steps per call: the other buffer of each (one launch
  // per step finishes the previous step into it)
  float* score2;
  float* comp2;
  int32_t* pos2;
  float* part2;
  float* logits2;
  int32_t max_split;
  float* row_lse2;
  float* col_sum;
  // position rolling (rope_base > 0), else null
  int32_t* rank;   // [units, kstride] position of each slot among the cached entries
  int32_t* rank2;  // its second buffer (multi-step calls on the split path with position rolling)
  int32_t rope_units;  // units whose prompt is rotated and scored per pass
  void* rope_ops;  // the rotated prompt of rope_units units: fp32 q, k [rope_units, lpad_cap, d] each;
                   // bf16 q hi, q lo, k hi, k lo [rope_units, lpad_cap, d] each
  float* rope_cs;  // [lpad_cap, d/2] (cos, sin) of position p * theta_m
  float* rope_th;  // [d/2] (hi, lo): theta_m / (2 pi) split so that n * hi is exact
};

namespace {

// Largest budget the kernels take: per-unit LDS holds k+1 logits (decode) and
// k kept positions (prefill select).
constexpr int64_t kMaxK = 12288;
// Units at or above this count run one block per unit in decode; fewer units
// split each unit's slots across blocks.
constexpr int32_t kSplitUnits = 512;
constexpr int32_t kMaxSplit = 64;
constexpr int32_t kMinSlotsPerSplit = 64;
constexpr float kLog2e = 1.4426950408889634f;
// Position rolling rotates the prompt into scratch chunk by chunk of units; the
// chunk is sized so the scratch stays under this many bytes (and at least 8
// units: one per XCD).
constexpr size_t kRopeScratchBytes = size_t{512} << 20;

thread_local std::string g_err;

h2o_status fail(h2o_status s, const std::string& msg) {
  g_err = msg;
  return s;
}

h2o_status hip_fail(hipError_t e, const char* what) {
  g_err = std::string(what) + ": " + hipGetErrorString(e);
  return e == hipErrorOutOfMemory ? H2O_ERR_OOM : H2O_ERR_HIP;
}

// Makes the cache's device current for one call and restores the caller's on
// exit; ok() is false when the device could not be made current, and the call
// then fails before touching any memory.
class DeviceGuard {
 public:
  explicit DeviceGuard(int dev) {
    ok_ = hipGetDevice(&prev_) == hipSuccess;
    if (ok_ && prev_ != dev) {
      ok_ = hipSetDevice(dev) == hipSuccess;
      changed_ = ok_;
    }
  }
  ~DeviceGuard() {
    if (changed_) (void)hipSetDevice(prev_);
  }
  bool ok() const { return ok_; }

 private:
  int prev_ = -1;
  bool ok_ = false;
  bool changed_ = false;
};

h2o_status device_fail() { return fail(H2O_ERR_HIP, "could not make the cache's device current"); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int32_t round32(int32_t n) { return (n + 31) / 32 * 32; }

struct Sizes {
  size_t kv, meta, split, prefill, rope, total;
  int32_t max_split, lpad, rope_units;
};

h2o_status check_params(const h2o_params* p, Sizes* sz) {
  if (p == nullptr) return fail(H2O_ERR_INVALID_ARG, "params is NULL");
  if (p->batch < 1 || p->heads < 1) return fail(H2O_ERR_INVALID_ARG, "batch and heads must be >= 1");
  if (p->head_dim < 1) return fail(H2O_ERR_INVALID_ARG, "head_dim must be >= 1");
  if (p->head_dim != 64 && p->head_dim != 128) return fail(H2O_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (p->heavy_budget < 0 || p->recent_budget < 0) return fail(H2O_ERR_INVALID_ARG, "budgets must be >= 0");
  const int64_t k = static_cast<int64_t>(p->heavy_budget) + p->recent_budget;
  if (k < 1) return fail(H2O_ERR_INVALID_ARG, "heavy_budget + recent_budget must be >= 1");
  if (k > kMaxK) return fail(H2O_ERR_UNSUPPORTED, "heavy_budget + recent_budget exceeds 12288");
  if (p->dtype != H2O_F32 && p->dtype != H2O_BF16) return fail(H2O_ERR_INVALID_ARG, "unknown dtype");
  if (!std::isfinite(p->scale)) return fail(H2O_ERR_INVALID_ARG, "scale must be finite");
  if (p->max_prompt < 0) return fail(H2O_ERR_INVALID_ARG, "max_prompt must be >= 0");
  if (!std::isfinite(p->rope_base) || p->rope_base < 0.f) return fail(H2O_ERR_INVALID_ARG, "rope_base must be >= 0");
  const int64_t units = static_cast<int64_t>(p->batch) * p->heads;
  const int64_t rows = std::max<int64_t>(k, round32(std::min<int32_t>(p->max_prompt, INT32_MAX - 31)));
  if (units * rows >= (int64_t{1} << 31) || units * kMaxSplit >= (int64_t{1} << 31))
    return fail(H2O_ERR_INVALID_ARG, "batch * heads * max(k, max_prompt) must stay below 2^31");
  // the prefill kernels address one unit's [L, d] matrix through a 32-bit byte range
  const int64_t esize = p->dtype == H2O_F32 ? 4 : 2;
  if (static_cast<int64_t>(round32(std::min<int32_t>(p->max_prompt, INT32_MAX - 31))) * p->head_dim * esize >=
      (int64_t{1} << 32))
    return fail(H2O_ERR_INVALID_ARG, "max_prompt * head_dim * element size must stay below 2^32 bytes");
  if (sz != nullptr) {
    const size_t es = p->dtype == H2O_F32 ? 4 : 2;
    const size_t u = static_cast<size_t>(units), kk = static_cast<size_t>(k), d = p->head_dim;
    sz->kv = 2 * u * kk * d * es;
    sz->meta = u * static_cast<size_t>(round32(static_cast<int32_t>(k))) * 12;
    sz->max_split = units < kSplitUnits ? kMaxSplit : 1;
    // split path: partials and logits, and a second buffer of them and of the
    // per-slot score, compensation and position (multi-step calls)
    sz->split = sz->max_split > 1
                    ? 2 * (u * sz->max_split * (2 + d) * 4 + u * (kk + 1) * 4) +
                          u * static_cast<size_t>(round32(static_cast<int32_t>(k))) * 12
                    : 0;
    sz->lpad = round32(p->max_prompt);
    sz->prefill = 2 * u * static_cast<size_t>(sz->lpad) * 4;
    // position rolling: slot ranks (two buffers on the split path), the rotated prompt of a chunk of units (8
    // bytes per element: fp32 q and k, or bf16 hi and lo of each), cos/sin per
    // prompt position and pair, per-pair frequencies (two floats)
    const size_t per_unit = static_cast<size_t>(sz->lpad) * d * 8;
    sz->rope_units = per_unit == 0 ? static_cast<int32_t>(units)
                                   : static_cast<int32_t>(std::min<size_t>(
                                         u, std::max<size_t>(8, kRopeScratchBytes / per_unit)));
    sz->rope = p->rope_base > 0.f ? u * static_cast<size_t>(round32(static_cast<int32_t>(k))) * 4 *
                                            (sz->max_split > 1 ? 2 : 1) +
                                        static_cast<size_t>(sz->rope_units) * per_unit +
                                        static_cast<size_t>(sz->lpad) * (d / 2) * 8 + (d / 2) * 8
                                  : 0;
    sz->total = sz->kv + sz->meta + sz->split + sz->prefill + sz->rope;
  }
  return H2O_OK;
}

void free_all(h2o_cache* c) {
  void* ptrs[] = {c->kslots, c->vslots, c->score, c->comp, c->pos, c->part, c->logits, c->score2, c->comp2,
                  c->pos2, c->part2, c->logits2, c->row_lse2, c->col_sum, c->rank, c->rank2, c->rope_ops,
                  c->rope_cs, c->rope_th};
  for (void* q : ptrs)
    if (q != nullptr) (void)hipFree(q);
}

// Rotary tables, in double precision on the host: (cos, sin) of p * theta_m for
// every prompt position p and pair m (rounded to float), and theta_m / (2 pi)
// split as hi + lo with hi holding 10 significant bits, so that n * hi is exact
// in float for |n| < 2^14 (any rank gap) and the decode angle n * theta keeps its
// fraction of a turn to about 1e-7.
hipError_t upload_rope_tables(h2o_cache* c, float base) {
  const int h = c->d / 2;
  std::vector<float> cs(static_cast<size_t>(c->lpad_cap) * h * 2), th(static_cast<size_t>(h) * 2);
  for (int m = 0; m < h; ++m) {
    const double theta = std::pow(static_cast<double>(base), -2.0 * m / c->d);
    for (int p = 0; p < c->lpad_cap; ++p) {
      cs[(static_cast<size_t>(p) * h + m) * 2] = static_cast<float>(std::cos(p * theta));
      cs[(static_cast<size_t>(p) * h + m) * 2 + 1] = static_cast<float>(std::sin(p * theta));
    }
    const double rev = theta / (2.0 * 3.14159265358979323846);
    int ex = 0;
    std::frexp(rev, &ex);
    const double hi = std::ldexp(std::nearbyint(std::ldexp(rev, 10 - ex)), ex - 10);
    th[static_cast<size_t>(m) * 2] = static_cast<float>(hi);
    th[static_cast<size_t>(m) * 2 + 1] = static_cast<float>(rev - hi);
  }
  hipError_t e = hipSuccess;
  if (!cs.empty()) e = hipMemcpy(c->rope_cs, cs.data(), cs.size() * 4, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(c->rope_th, th.data(), th.size() * 4, hipMemcpyHostToDevice);
  return e;
}

// The prompt's score passes (row normalisers, column sums and, when a.out is
// set, the prompt's own output) over rows 0..a.L-1 of q and k.  With position
// rolling the prompt is first rotated to positions 0..L-1, a chunk of units at a
// time, into the cache's scratch (bf16: as hi and lo parts), and each chunk is
// scored from there.
hipError_t score_prompt(h2o_cache* c, h2o::PrefillArgs a, hipStream_t s) {
  a.stages = h2o::kStageScores;
  if (c->rank == nullptr) return h2o::launch_prefill(c->p.dtype, c->d, a, c->units, s);
  const size_t elems = static_cast<size_t>(a.L) * c->d;  // elements per unit of q, k, v and out
  const size_t cap = static_cast<size_t>(c->rope_units) * c->lpad_cap * c->d;  // elements per scratch array
  char* ops = static_cast<char*>(c->rope_ops);
  const bool bf16 = c->p.dtype == H2O_BF16;
  // bf16: q hi, q lo, k hi, k lo; fp32: q, k
  void* qh = ops;
  void* ql = bf16 ? ops + cap * 2 : nullptr;
  void* kh = ops + cap * 4;
  void* kl = bf16 ? ops + cap * 6 : nullptr;
  const char* q = static_cast<const char*>(a.q);
  const char* k = static_cast<const char*>(a.k);
  for (int32_t u0 = 0; u0 < c->units; u0 += c->rope_units) {
    const int32_t nu = std::min(c->rope_units, c->units - u0);
    const size_t off = static_cast<size_t>(u0) * elems;
    hipError_t e = h2o::launch_rope_prompt(c->p.dtype, c->d, q + off * c->esize, qh, ql, a.L, nu, c->rope_cs, s);
    if (e == hipSuccess)
      e = h2o::launch_rope_prompt(c->p.dtype, c->d, k + off * c->esize, kh, kl, a.L, nu, c->rope_cs, s);
    if (e != hipSuccess) return e;
    h2o::PrefillArgs b = a;
    b.q = qh;
    b.k = kh;
    b.q_lo = ql;
    b.k_lo = kl;
    b.v = a.v != nullptr ? static_cast<const char*>(a.v) + off * c->esize : nullptr;
    b.out = a.out != nullptr ? a.out + off : nullptr;
    b.row_lse2 = a.row_lse2 + static_cast<size_t>(u0) * a.Lpad;
    b.col_sum = a.col_sum + static_cast<size_t>(u0) * a.Lpad;
    e = h2o::launch_prefill(c->p.dtype, c->d, b, nu, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

int choose_nsplit(const h2o_cache* c, int32_t count, int32_t* split_len) {
  int ns = 1;
  if (c->max_split > 1 && count >= 2 * kMinSlotsPerSplit) {
    const int want = (1024 + c->units - 1) / c->units;
    ns = std::max(1, std::min({want, count / kMinSlotsPerSplit, static_cast<int>(c->max_split)}));
  }
  if (ns == 1) {
    *split_len = std::max(count, 1);
    return 1;
  }
  *split_len = (count + ns - 1) / ns;
  return (count + *split_len - 1) / *split_len;  // every split holds >= 1 slot
}

// Scratch of h2o_column_scores_noalloc: a file-scope device array instead of
// an allocation (the prompt's row normalisers and column sums, [units, Lpad]
// float32 each).  Every GPU that loads the library holds its own copy until
// the process ends; host code reaches it only through the address
// hipGetSymbolAddress returns on that device.
constexpr size_t kStaticScratchBytes = size_t{16} << 20;
__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// This device's copy of `scratch` (looked up on the first call per device,
// with the device current).
hipError_t static_scratch(int dev, void** ptr) {
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

const char* h2o_status_str(h2o_status s) {
  switch (s) {
    case H2O_OK: return "ok";
    case H2O_ERR_INVALID_ARG: return "invalid argument";
    case H2O_ERR_STATE: return "invalid state";
    case H2O_ERR_OOM: return "out of device memory";
    case H2O_ERR_HIP: return "HIP runtime error";
    case H2O_ERR_UNSUPPORTED: return "unsupported";
  }
  return "unknown status";
}

const char* h2o_last_error(void) { return g_err.c_str(); }

h2o_status h2o_cache_bytes(const h2o_params* params, size_t* kv_bytes, size_t* total_bytes) {
  Sizes sz{};
  const h2o_status st = check_params(params, &sz);
  if (st != H2O_OK) return st;
  if (kv_bytes != nullptr) *kv_bytes = sz.kv;
  if (total_bytes != nullptr) *total_bytes = sz.total;
  return H2O_OK;
}

h2o_status h2o_cache_create(const h2o_params* params, int device, h2o_cache** out) {
  if (out == nullptr) return fail(H2O_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  Sizes sz{};
  h2o_status st = check_params(params, &sz);
  if (st != H2O_OK) return st;
  if (device < -1) return fail(H2O_ERR_INVALID_ARG, "device must be >= -1");
  int dev = device;
  if (dev == -1) {
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  } else {
    int n = 0;
    const hipError_t e = hipGetDeviceCount(&n);
    if (e != hipSuccess) return hip_fail(e, "hipGetDeviceCount");
    if (dev >= n) return fail(H2O_ERR_INVALID_ARG, "device index out of range");
  }
  DeviceGuard guard(dev);
  if (!guard.ok()) return device_fail();
  h2o_cache* c = new (std::nothrow) h2o_cache{};
  if (c == nullptr) return fail(H2O_ERR_OOM, "host allocation failed");
  c->p = *params;
  c->device = dev;
  c->d = params->head_dim;
  c->k = params->heavy_budget + params->recent_budget;
  c->kstride = round32(c->k);
  c->units = params->batch * params->heads;
  c->pat_kind = H2O_PATTERN_NONE;
  c->pat_period = 1;
  c->pat_width = 1;
  c->esize = params->dtype == H2O_F32 ? 4 : 2;
  c->scale = params->scale > 0.f ? params->scale : 1.f / std::sqrt(static_cast<float>(c->d));
  c->c2 = c->scale * kLog2e;
  c->count = 0;
  c->next_pos = 0;
  c->prompt_len = -1;
  c->lpad_cap = sz.lpad;
  c->lpad_last = 0;
  c->max_split = sz.max_split;
  c->rope_units = sz.rope_units;

  const size_t u = c->units, kk = c->k, d = c->d;
  const bool rope = params->rope_base > 0.f;
  struct Alloc {
    void** p;
    size_t bytes;
  } allocs[] = {
      {&c->kslots, u * kk * d * c->esize},
      {&c->vslots, u * kk * d * c->esize},
      {reinterpret_cast<void**>(&c->score), u * c->kstride * 4},
      {reinterpret_cast<void**>(&c->comp), u * c->kstride * 4},
      {reinterpret_cast<void**>(&c->pos), u * c->kstride * 4},
      {reinterpret_cast<void**>(&c->part), c->max_split > 1 ? u * c->max_split * (2 + d) * 4 : 0},
      {reinterpret_cast<void**>(&c->logits), c->max_split > 1 ? u * (kk + 1) * 4 : 0},
      {reinterpret_cast<void**>(&c->score2), c->max_split > 1 ? u * c->kstride * 4 : 0},
      {reinterpret_cast<void**>(&c->comp2), c->max_split > 1 ? u * c->kstride * 4 : 0},
      {reinterpret_cast<void**>(&c->pos2), c->max_split > 1 ? u * c->kstride * 4 : 0},
      {reinterpret_cast<void**>(&c->part2), c->max_split > 1 ? u * c->max_split * (2 + d) * 4 : 0},
      {reinterpret_cast<void**>(&c->logits2), c->max_split > 1 ? u * (kk + 1) * 4 : 0},
      {reinterpret_cast<void**>(&c->row_lse2), u * c->lpad_cap * 4},
      {reinterpret_cast<void**>(&c->col_sum), u * c->lpad_cap * 4},
      {reinterpret_cast<void**>(&c->rank), rope ? u * c->kstride * 4 : 0},
      {reinterpret_cast<void**>(&c->rank2), rope && c->max_split > 1 ? u * c->kstride * 4 : 0},
      {&c->rope_ops, rope ? static_cast<size_t>(c->rope_units) * c->lpad_cap * d * 8 : 0},
      {reinterpret_cast<void**>(&c->rope_cs), rope ? static_cast<size_t>(c->lpad_cap) * (d / 2) * 8 : 0},
      {reinterpret_cast<void**>(&c->rope_th), rope ? (d / 2) * 8 : 0},
  };
  for (const Alloc& a : allocs) {
    if (a.bytes == 0) continue;
    const hipError_t e = hipMalloc(a.p, a.bytes);
    if (e != hipSuccess) {
      free_all(c);
      delete c;
      return hip_fail(e, "hipMalloc");
    }
  }
  hipError_t e = h2o::launch_clear(c->pos, c->score, c->comp, u * c->kstride, nullptr);
  if (e == hipSuccess && rope) e = upload_rope_tables(c, params->rope_base);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    free_all(c);
    delete c;
    return hip_fail(e, "cache initialisation");
  }
  *out = c;
  return H2O_OK;
}

h2o_status h2o_cache_destroy(h2o_cache* c) {
  if (c == nullptr) return H2O_OK;
  DeviceGuard guard(c->device);
  const hipError_t e = guard.ok() ? hipDeviceSynchronize() : hipErrorInvalidDevice;
  free_all(c);
  delete c;
  if (e != hipSuccess) return hip_fail(e, "hipDeviceSynchronize before free");
  return H2O_OK;
}

h2o_status h2o_prefill(h2o_cache* c, const void* q, const void* k, const void* v, int32_t L, float* out,
                       void* stream) {
  if (c == nullptr) return fail(H2O_ERR_INVALID_ARG, "cache is NULL");
  if (L < 0) return fail(H2O_ERR_INVALID_ARG, "prompt_len must be >= 0");
  if (L > c->p.max_prompt) return fail(H2O_ERR_INVALID_ARG, "prompt_len exceeds max_prompt");
  if (L > 0) {
    if (q == nullptr || k == nullptr || v == nullptr) return fail(H2O_ERR_INVALID_ARG, "q, k, v must be non-NULL");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v))
      return fail(H2O_ERR_INVALID_ARG, "q, k, v must be 16-byte aligned");
    if (out != nullptr && !aligned16(out)) return fail(H2O_ERR_INVALID_ARG, "out must be 16-byte aligned");
  }
  DeviceGuard guard(c->device);
  if (!guard.ok()) return device_fail();
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (L == 0) {
    const hipError_t e = h2o::launch_clear(c->pos, c->score, c->comp, static_cast<size_t>(c->units) * c->kstride, s);
    if (e != hipSuccess) return hip_fail(e, "clear launch");
  } else {
    h2o::PrefillArgs a{};
    a.stages = h2o::kStageScores | h2o::kStageSelect;
    a.q = q;
    a.k = k;
    a.v = v;
    a.kcache = k;
    a.rank = c->rank;
    a.L = L;
    a.Lpad = round32(L);
    a.row_lse2 = c->row_lse2;
    a.col_sum = c->col_sum;
    a.out = out;
    a.kslots = c->kslots;
    a.vslots = c->vslots;
    a.score = c->score;
    a.comp = c->comp;
    a.pos = c->pos;
    a.heavy = c->p.heavy_budget;
    a.recent = c->p.recent_budget;
    a.kcap = c->k;
    a.kstride = c->kstride;
    a.pat_kind = c->pat_kind;
    a.pat_period = c->pat_period;
    a.pat_width = c->pat_width;
    a.kv_rows = L;
    a.scale = c->scale;
    a.c2 = c->c2;
    hipError_t e;
    if (c->rank != nullptr) {  // position rolling: the prompt is scored on its rotated q/k
      e = score_prompt(c, a, s);
      a.stages = h2o::kStageSelect;
      if (e == hipSuccess) e = h2o::launch_prefill(c->p.dtype, c->d, a, c->units, s);
    } else {
      e = h2o::launch_prefill(c->p.dtype, c->d, a, c->units, s);
    }
    if (e != hipSuccess) return hip_fail(e, "prefill launch");
    c->lpad_last = a.Lpad;
  }
  c->count = std::min(L, c->k);
  c->next_pos = L;
  c->prompt_len = L;
  c->stats_valid = true;
  return H2O_OK;
}

h2o_status h2o_column_scores(h2o_cache* c, const void* q, const void* k, int32_t n, float* scores, void* stream) {
  if (c == nullptr) return fail(H2O_ERR_INVALID_ARG, "cache is NULL");
  if (n < 0) return fail(H2O_ERR_INVALID_ARG, "n must be >= 0");
  if (n > c->p.max_prompt) return fail(H2O_ERR_INVALID_ARG, "n exceeds max_prompt");
  if (n == 0) return H2O_OK;
  if (q == nullptr || k == nullptr || scores == nullptr)
    return fail(H2O_ERR_INVALID_ARG, "q, k and scores must be non-NULL");
  if (!aligned16(q) || !aligned16(k)) return fail(H2O_ERR_INVALID_ARG, "q and k must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(scores) & 3u) != 0)
    return fail(H2O_ERR_INVALID_ARG, "scores must be 4-byte aligned");
  DeviceGuard guard(c->device);
  if (!guard.ok()) return device_fail();
  hipStream_t s = static_cast<hipStream_t>(stream);
  h2o::PrefillArgs a{};
  a.stages = h2o::kStageScores;
  a.q = q;
  a.k = k;
  a.L = n;
  a.Lpad = round32(n);
  a.row_lse2 = c->row_lse2;
  a.col_sum = c->col_sum;
  a.scale = c->scale;
  a.c2 = c->c2;
  a.kcap = c->k;
  a.kstride = c->kstride;
  hipError_t e = score_prompt(c, a, s);  // position rolling: at the sequence's own positions
  if (e != hipSuccess) return hip_fail(e, "column score launch");
  c->stats_valid = false;  // the prefill scratch now holds this sequence's statistics
  e = hipMemcpy2DAsync(scores, static_cast<size_t>(n) * 4, c->col_sum, static_cast<size_t>(a.Lpad) * 4,
                       static_cast<size_t>(n) * 4, c->units, hipMemcpyDeviceToDevice, s);
  if (e != hipSuccess) return hip_fail(e, "copy column scores");
  return H2O_OK;
}

h2o_status h2o_column_scores_noalloc(const h2o_params* p, const void* q, const void* k, int32_t n, float* scores,
                                     void* stream) {
  if (p == nullptr) return fail(H2O_ERR_INVALID_ARG, "params is NULL");
  if (p->batch < 1 || p->heads < 1) return fail(H2O_ERR_INVALID_ARG, "batch and heads must be >= 1");
  if (p->head_dim != 64 && p->head_dim != 128) return fail(H2O_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (p->dtype != H2O_F32 && p->dtype != H2O_BF16) return fail(H2O_ERR_INVALID_ARG, "unknown dtype");
  if (!std::isfinite(p->scale)) return fail(H2O_ERR_INVALID_ARG, "scale must be finite");
  if (p->rope_base != 0.f) return fail(H2O_ERR_UNSUPPORTED, "position rolling needs a cache (h2o_column_scores)");
  if (n < 0) return fail(H2O_ERR_INVALID_ARG, "n must be >= 0");
  if (n == 0) return H2O_OK;
  if (q == nullptr || k == nullptr || scores == nullptr)
    return fail(H2O_ERR_INVALID_ARG, "q, k and scores must be non-NULL");
  if (!aligned16(q) || !aligned16(k)) return fail(H2O_ERR_INVALID_ARG, "q and k must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(scores) & 3u) != 0)
    return fail(H2O_ERR_INVALID_ARG, "scores must be 4-byte aligned");
  const int64_t units = static_cast<int64_t>(p->batch) * p->heads;
  const int64_t lpad = round32(std::min<int32_t>(n, INT32_MAX - 31));
  const int64_t esize = p->dtype == H2O_F32 ? 4 : 2;
  if (lpad * p->head_dim * esize >= (int64_t{1} << 32))
    return fail(H2O_ERR_INVALID_ARG, "n * head_dim * element size must stay below 2^32 bytes");
  if (units * lpad * 8 > static_cast<int64_t>(kStaticScratchBytes))
    return fail(H2O_ERR_INVALID_ARG, "batch * heads * n (rounded up to 32) * 8 bytes exceeds the 16 MiB static scratch");
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  void* base = nullptr;
  e = static_scratch(dev, &base);
  if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const float scale = p->scale > 0.f ? p->scale : 1.f / std::sqrt(static_cast<float>(p->head_dim));
  h2o::PrefillArgs a{};
  a.stages = h2o::kStageScores;
  a.q = q;
  a.k = k;
  a.L = n;
  a.Lpad = static_cast<int32_t>(lpad);
  // every value of the scratch that a pass reads, an earlier pass of this call writes
  a.row_lse2 = static_cast<float*>(base);
  a.col_sum = static_cast<float*>(base) + units * lpad;
  a.scale = scale;
  a.c2 = scale * kLog2e;
  e = h2o::launch_prefill(p->dtype, p->head_dim, a, static_cast<int>(units), s);
  if (e != hipSuccess) return hip_fail(e, "column score launch");
  e = hipMemcpy2DAsync(scores, static_cast<size_t>(n) * 4, a.col_sum, static_cast<size_t>(lpad) * 4,
                       static_cast<size_t>(n) * 4, static_cast<size_t>(units), hipMemcpyDeviceToDevice, s);
  if (e != hipSuccess) return hip_fail(e, "copy column scores");
  return H2O_OK;
}

h2o_status h2o_prefill_scored(h2o_cache* c, const void* k, const void* v, int32_t L, int32_t seq_rows,
                              const float* scores, void* stream) {
  if (c == nullptr) return fail(H2O_ERR_INVALID_ARG, "cache is NULL");
  if (L < 0) return fail(H2O_ERR_INVALID_ARG, "prompt_len must be >= 0");
  if (seq_rows < L) return fail(H2O_ERR_INVALID_ARG, "seq_rows must be >= prompt_len");
  if (L > 0) {
    if (k == nullptr || v == nullptr || scores == nullptr)
      return fail(H2O_ERR_INVALID_ARG, "k, v and scores must be non-NULL");
    if (!aligned16(k) || !aligned16(v)) return fail(H2O_ERR_INVALID_ARG, "k and v must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(scores) & 3u) != 0)
      return fail(H2O_ERR_INVALID_ARG, "scores must be 4-byte aligned");
  }
  DeviceGuard guard(c->device);
  if (!guard.ok()) return device_fail();
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (L == 0) {
    const hipError_t e = h2o::launch_clear(c->pos, c->score, c->comp, static_cast<size_t>(c->units) * c->kstride, s);
    if (e != hipSuccess) return hip_fail(e, "clear launch");
  } else {
    h2o::PrefillArgs a{};
    a.stages = h2o::kStageSelect;
    a.k = k;
    a.kcache = k;
    a.rank = c->rank;
    a.v = v;
    a.L = L;
    a.Lpad = round32(L);
    a.scores_in = scores;
    a.scores_stride = seq_rows;
    a.kv_rows = seq_rows;
    a.kslots = c->kslots;
    a.vslots = c->vslots;
    a.score = c->score;
    a.comp = c->comp;
    a.pos = c->pos;
    a.heavy = c->p.heavy_budget;
    a.recent = c->p.recent_budget;
    a.kcap = c->k;
    a.kstride = c->kstride;
    a.pat_kind = c->pat_kind;
    a.pat_period = c->pat_period;
    a.pat_width = c->pat_width;
    a.scale = c->scale;
    a.c2 = c->c2;
    const hipError_t e = h2o::launch_prefill(c->p.dtype, c->d, a, c->units, s);
    if (e != hipSuccess) return hip_fail(e, "scored prefill launch");
  }
  c->count = std::min(L, c->k);
  c->next_pos = L;
  c->prompt_len = L;
  c->stats_valid = false;
  return H2O_OK;
}

namespace {

// Scores gain one weight per decode step.  The first kPlainSteps steps after a
// prefill add them in plain fp32: a sum of n non-negative fp32 terms is within
// (n - 1) * 2^-24 relative of the exact sum, so a score that started from its
// prompt column sum is within 1024 * 2^-24 = 6.1e-5 after them, inside the
// 1e-4 score tolerance, and the compensation array is neither read nor
// written.  Later steps use Kahan-compensated adds (the 4 M-token stream needs
// them: plain fp32 drifts to ~1e-3 there), starting from a compensation of 0.
constexpr int32_t kPlainSteps = 1024;

// The launch arguments of the cache's next decode step.
h2o::DecodeArgs decode_args(const h2o_cache* c, const void* q, const void* k, const void* v, const float* new_score,
                            int32_t score_stride, float* out, int32_t* evicted) {
  h2o::DecodeArgs a{};
  a.q = q;
  a.knew = k;
  a.vnew = v;
  a.kslots = c->kslots;
  a.vslots = c->vslots;
  a.score = c->score;
  a.comp = c->comp;
  a.pos = c->pos;
  a.out = out;
  a.evicted = evicted;
  a.part = c->part;
  a.logits = c->logits;
  a.k = c->k;
  a.kstride = c->kstride;
  a.count = c->count;
  a.new_pos = c->next_pos;
  a.cand_limit = c->next_pos - c->p.recent_budget;
  a.new_is_candidate = c->p.recent_budget == 0 ? 1 : 0;
  a.plain_until = c->prompt_len > INT32_MAX - kPlainSteps ? INT32_MAX : c->prompt_len + kPlainSteps;
  a.fixed_new = new_score;
  a.fixed_stride = score_stride;
  a.pat_kind = c->pat_kind;
  a.pat_period = c->pat_period;
  a.pat_width = c->pat_width;
  a.rank = c->rank;
  a.rope_th = c->rope_th;
  a.nsplit = choose_nsplit(c, c->count, &a.split_len);
  a.c2 = c->c2;
  return a;
}

// One decode step of every unit: the launch and the host-side step counters.
// The caller has validated the arguments and made the cache's device current.
hipError_t decode_launch(h2o_cache* c, const void* q, const void* k, const void* v, const float* new_score,
                         int32_t score_stride, float* out, int32_t* evicted, hipStream_t stream) {
  const h2o::DecodeArgs a = decode_args(c, q, k, v, new_score, score_stride, out, evicted);
  const hipError_t e = h2o::launch_decode(c->p.dtype, c->d, a, c->units, stream);
  if (e != hipSuccess) return e;
  if (c->count < c->k) ++c->count;
  ++c->next_pos;
  return hipSuccess;
}

// Steps per launch of the shared-memory-resident multi-step decode.
constexpr int32_t kResidentSteps = 65536;

h2o_status decode_common(h2o_cache* c, const void* q, const void* k, const void* v, const float* new_score,
                         int32_t score_stride, float* out, int32_t* evicted, void* stream) {
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr)
    return fail(H2O_ERR_INVALID_ARG, "q, k, v and out must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(H2O_ERR_INVALID_ARG, "q, k, v and out must be 16-byte aligned");
  if (evicted != nullptr && (reinterpret_cast<uintptr_t>(evicted) & 3u) != 0)
    return fail(H2O_ERR_INVALID_ARG, "evicted must be 4-byte aligned");
  if (c->prompt_len < 0) return fail(H2O_ERR_STATE, "decode before prefill");
  if (c->next_pos == INT32_MAX) return fail(H2O_ERR_STATE, "position counter would overflow int32");
  DeviceGuard guard(c->device);
  if (!guard.ok()) return device_fail();
  const hipError_t e = decode_launch(c, q, k, v, new_score, score_stride, out, evicted,
                                     static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return H2O_OK;
}

}  // namespace

h2o_status h2o_decode_step(h2o_cache* c, const void* q, const void* k, const void* v, float* out,
                           int32_t* evicted, void* stream) {
  if (c == nullptr) return fail(H2O_ERR_INVALID_ARG, "cache is NULL");
  return decode_common(c, q, k, v, nullptr, 1, out, evicted, stream);
}

h2o_status h2o_decode_steps(h2o_cache* c, const void* q, const void* k, const void* v, int32_t steps, float* out,
                            int64_t out_step, int32_t* evicted, void* stream) {
  if (c == nullptr) return fail(H2O_ERR_INVALID_ARG, "cache is NULL");
  if (steps < 0) return fail(H2O_ERR_INVALID_ARG, "steps must be >= 0");
  if (out_step < 0 || (out_step & 3) != 0) return fail(H2O_ERR_INVALID_ARG, "out_step must be >= 0 and a multiple of 4");
  if (steps == 0) return H2O_OK;
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr)
    return fail(H2O_ERR_INVALID_ARG, "q, k, v and out must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(H2O_ERR_INVALID_ARG, "q, k, v and out must be 16-byte aligned");
  if (evicted != nullptr && (reinterpret_cast<uintptr_t>(evicted) & 3u) != 0)
    return fail(H2O_ERR_INVALID_ARG, "evicted must be 4-byte aligned");
  if (c->prompt_len < 0) return fail(H2O_ERR_STATE, "decode before prefill");
  if (static_cast<int64_t>(c->next_pos) + steps > INT32_MAX)
    return fail(H2O_ERR_STATE, "position counter would overflow int32");
  DeviceGuard guard(c->device);
  if (!guard.ok()) return device_fail();
  const size_t tok = static_cast<size_t>(c->units) * c->d * c->esize;  // bytes of one step's q, k or v
  const size_t units = static_cast<size_t>(c->units);
  hipStream_t s = static_cast<hipStream_t>(stream);
  // Caches on the single-block path for every one of these steps whose rows fit
  // in a block's shared memory run several steps per launch with the rows held
  // there (bit-identical to one launch per step).
  const int64_t last_count = std::min<int64_t>(c->k, static_cast<int64_t>(c->count) + steps - 1);
  const bool resident = c->rank == nullptr && (c->max_split == 1 || last_count < 2 * kMinSlotsPerSplit) &&
                        h2o::decode_resident_fits(c->p.dtype, c->d, c->units, c->k);
  if (resident) {
    for (int32_t t0 = 0; t0 < steps; t0 += kResidentSteps) {
      const int32_t n = std::min(kResidentSteps, steps - t0);
      const size_t off = static_cast<size_t>(t0) * tok;
      const h2o::DecodeArgs a =
          decode_args(c, static_cast<const char*>(q) + off, static_cast<const char*>(k) + off,
                      static_cast<const char*>(v) + off, nullptr, 1, out + t0 * out_step,
                      evicted != nullptr ? evicted + t0 * units : nullptr);
      const hipError_t e = h2o::launch_decode_resident(c->p.dtype, c->d, a, c->units, n,
                                                       static_cast<int64_t>(tok), out_step, s);
      if (e != hipSuccess) return hip_fail(e, "decode launch");
      c->count = static_cast<int32_t>(std::min<int64_t>(c->k, static_cast<int64_t>(c->count) + n));
      c->next_pos += n;
    }
    return H2O_OK;
  }
  // Steps on the split path (which, once reached, lasts: the count only grows)
  // run one launch each: launch i finishes step i-1 and runs step i's slices,
  // alternating two buffers of scores/compensations/positions (and places, with
  // position rolling) and of partials/logits; a finish launch closes the run
  // (bit-identical to a split launch and a finish launch per step).
  const bool fuse = c->max_split > 1;
  int32_t t = 0;
  for (; t < steps; ++t) {
    int32_t unused = 0;
    if (fuse && choose_nsplit(c, c->count, &unused) > 1) break;
    const size_t off = static_cast<size_t>(t) * tok;
    const hipError_t e = decode_launch(c, static_cast<const char*>(q) + off, static_cast<const char*>(k) + off,
                                       static_cast<const char*>(v) + off, nullptr, 1, out + t * out_step,
                                       evicted != nullptr ? evicted + t * units : nullptr, s);
    if (e != hipSuccess) return hip_fail(e, "decode launch");
  }
  if (t == steps) return H2O_OK;
  // the rest on the split path, one launch per step
  struct Buffers {
    float* score;
    float* comp;
    int32_t* pos;
    float* part;
    float* logits;
    int32_t* rank;
  } buf[2] = {{c->score, c->comp, c->pos, c->part, c->logits, c->rank},
              {c->score2, c->comp2, c->pos2, c->part2, c->logits2, c->rank2}};
  auto step_args = [&](int32_t i, int which) {
    const size_t off = static_cast<size_t>(i) * tok;
    h2o::DecodeArgs a = decode_args(c, static_cast<const char*>(q) + off, static_cast<const char*>(k) + off,
                                    static_cast<const char*>(v) + off, nullptr, 1, out + i * out_step,
                                    evicted != nullptr ? evicted + i * units : nullptr);
    a.score = buf[which].score;
    a.comp = buf[which].comp;
    a.pos = buf[which].pos;
    a.part = buf[which].part;
    a.logits = buf[which].logits;
    a.rank = buf[which].rank;  // nullptr without position rolling
    return a;
  };
  auto advance = [&]() {
    if (c->count < c->k) ++c->count;
    ++c->next_pos;
  };
  int which = 0;  // buffer holding step `prev`'s scores and its partials
  h2o::DecodeArgs prev = step_args(t, which);
  hipError_t e =
      h2o::launch_decode_split(c->p.dtype, c->d, nullptr, prev, nullptr, nullptr, nullptr, nullptr, c->units, s);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  advance();
  for (++t; t < steps; ++t) {
    h2o::DecodeArgs cur = step_args(t, which ^ 1);
    e = h2o::launch_decode_split(c->p.dtype, c->d, &prev, cur, buf[which ^ 1].score, buf[which ^ 1].comp,
                                 buf[which ^ 1].pos, buf[which ^ 1].rank, c->units, s);
    if (e != hipSuccess) return hip_fail(e, "decode launch");
    advance();
    which ^= 1;
    prev = cur;
  }
  e = h2o::launch_decode_finish(c->p.dtype, c->d, prev, c->units, s);  // the last step's finish, in place
  if (e == hipSuccess && which == 1) {  // the cache's own arrays receive the final state (occupied slots)
    const size_t pitch = static_cast<size_t>(c->kstride) * 4, width = static_cast<size_t>(c->count) * 4;
    const size_t rows = static_cast<size_t>(c->units);
    e = hipMemcpy2DAsync(c->score, pitch, c->score2, pitch, width, rows, hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess) e = hipMemcpy2DAsync(c->comp, pitch, c->comp2, pitch, width, rows, hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess) e = hipMemcpy2DAsync(c->pos, pitch, c->pos2, pitch, width, rows, hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess && c->rank != nullptr)
      e = hipMemcpy2DAsync(c->rank, pitch, c->rank2, pitch, width, rows, hipMemcpyDeviceToDevice, s);
  }
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return H2O_OK;
}

h2o_status h2o_decode_step_scored(h2o_cache* c, const void* q, const void* k, const void* v,
                                  const float* new_score, int32_t score_stride, float* out, int32_t* evicted,
                                  void* stream) {
  if (c == nullptr) return fail(H2O_ERR_INVALID_ARG, "cache is NULL");
  if (new_score == nullptr) return fail(H2O_ERR_INVALID_ARG, "new_score must be non-NULL");
  if ((reinterpret_cast<uintptr_t>(new_score) & 3u) != 0)
    return fail(H2O_ERR_INVALID_ARG, "new_score must be 4-byte aligned");
  if (score_stride < 1) return fail(H2O_ERR_INVALID_ARG, "score_stride must be >= 1");
  return decode_common(c, q, k, v, new_score, score_stride, out, evicted, stream);
}

h2o_status h2o_cache_read(h2o_cache* c, int32_t* pos, float* score, void* k_slots, void* v_slots, int32_t* meta,
                          void* stream) {
  if (c == nullptr) return fail(H2O_ERR_INVALID_ARG, "cache is NULL");
  DeviceGuard guard(c->device);
  if (!guard.ok()) return device_fail();
  hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  const size_t n = static_cast<size_t>(c->units) * c->k;
  const size_t row = static_cast<size_t>(c->k) * 4, pitch = static_cast<size_t>(c->kstride) * 4;
  if (pos != nullptr &&
      (e = hipMemcpy2D(pos, row, c->pos, pitch, row, c->units, hipMemcpyDeviceToHost)) != hipSuccess)
    return hip_fail(e, "copy pos");
  if (score != nullptr) {
    // the Kahan pair (running sum s, compensation c) folded into one value: the
    // sum of the added weights is s - c
    std::vector<float> comp(n);
    if ((e = hipMemcpy2D(score, row, c->score, pitch, row, c->units, hipMemcpyDeviceToHost)) != hipSuccess ||
        (e = hipMemcpy2D(comp.data(), row, c->comp, pitch, row, c->units, hipMemcpyDeviceToHost)) != hipSuccess)
      return hip_fail(e, "copy score");
    for (size_t i = 0; i < n; ++i)
      score[i] = static_cast<float>(static_cast<double>(score[i]) - static_cast<double>(comp[i]));
  }
  const size_t kvb = n * c->d * c->esize;
  if (k_slots != nullptr && (e = hipMemcpy(k_slots, c->kslots, kvb, hipMemcpyDeviceToHost)) != hipSuccess)
    return hip_fail(e, "copy k slots");
  if (v_slots != nullptr && (e = hipMemcpy(v_slots, c->vslots, kvb, hipMemcpyDeviceToHost)) != hipSuccess)
    return hip_fail(e, "copy v slots");
  if (meta != nullptr) {
    meta[0] = c->count;
    meta[1] = c->next_pos;
  }
  return H2O_OK;
}

h2o_status h2o_prefill_stats_read(h2o_cache* c, float* row_lse, float* col_sum, void* stream) {
  if (c == nullptr) return fail(H2O_ERR_INVALID_ARG, "cache is NULL");
  if (c->prompt_len < 0) return fail(H2O_ERR_STATE, "no prefill yet");
  if (!c->stats_valid)
    return fail(H2O_ERR_STATE, "no statistics: the last call was h2o_prefill_scored or h2o_column_scores");
  DeviceGuard guard(c->device);
  if (!guard.ok()) return device_fail();
  hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  const int32_t L = c->prompt_len;
  if (L == 0) return H2O_OK;
  const float* src[2] = {c->row_lse2, c->col_sum};
  float* dst[2] = {row_lse, col_sum};
  for (int t = 0; t < 2; ++t) {
    if (dst[t] == nullptr) continue;
    e = hipMemcpy2D(dst[t], static_cast<size_t>(L) * 4, src[t], static_cast<size_t>(c->lpad_last) * 4,
                    static_cast<size_t>(L) * 4, c->units, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "copy prefill statistics");
  }
  if (row_lse != nullptr) {  // the kernels keep log2 of the normaliser
    const float ln2 = 0.6931471805599453f;
    const size_t n = static_cast<size_t>(L) * c->units;
    for (size_t i = 0; i < n; ++i) row_lse[i] *= ln2;
  }
  return H2O_OK;
}

h2o_status h2o_cache_set_pattern(h2o_cache* c, int32_t kind, int32_t period, int32_t width) {
  if (c == nullptr) return fail(H2O_ERR_INVALID_ARG, "cache is NULL");
  if (kind == H2O_PATTERN_NONE) {
    c->pat_kind = kind;
    c->pat_period = 1;
    c->pat_width = 1;
    return H2O_OK;
  }
  if (kind != H2O_PATTERN_STRIDED && kind != H2O_PATTERN_FIXED) return fail(H2O_ERR_INVALID_ARG, "unknown pattern");
  if (period < 1) return fail(H2O_ERR_INVALID_ARG, "period must be >= 1");
  if (kind == H2O_PATTERN_FIXED && (width < 1 || width > period))
    return fail(H2O_ERR_INVALID_ARG, "width must be in [1, period]");
  c->pat_kind = kind;
  c->pat_period = period;
  c->pat_width = kind == H2O_PATTERN_FIXED ? width : 1;
  return H2O_OK;
}

h2o_status h2o_cache_info(const h2o_cache* c, int32_t* count, int32_t* next_pos, int32_t* prompt_len) {
  if (c == nullptr) return fail(H2O_ERR_INVALID_ARG, "cache is NULL");
  if (count != nullptr) *count = c->count;
  if (next_pos != nullptr) *next_pos = c->next_pos;
  if (prompt_len != nullptr) *prompt_len = c->prompt_len;
  return H2O_OK;
}

}  // extern "C"
