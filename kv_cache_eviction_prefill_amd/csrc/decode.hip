// H2O decode step: attention over the budgeted cache, score accumulation,
// eviction and in-place overwrite, fused into one kernel launch.
//
// Sources: "H2O: Heavy-Hitter Oracle for Efficient Generative Inference of Large
// Language Models -- 深度解读报告", §3.1 (evicted entries leave the softmax
// normaliser), §3.3 (Algorithm 1: add the new token, then evict the entry whose
// removal keeps the most accumulated attention), §3.4 (preallocated cache,
// overwrite in place, recent window plus heavy hitters, one eviction per head);
// the "H2O" paper card (phantomic12): running accumulated-attention score per
// token.
//
// Work mapping (gfx950, wave64, 256 threads per block):
//   * A K/V row of d elements is 16 bytes per lane over LPR lanes (bf16 d=128:
//     16 lanes), so one wave-wide load instruction moves 4 whole rows (1 KiB),
//     fully coalesced.  The block's 16 row groups walk the unit's slots with
//     kUnroll rows in flight per group, K and V of a slot loaded together.
//   * Each group keeps an online softmax (max, sum, o) in registers; groups are
//     merged through LDS.  Logits go to LDS (single-block path) or to a global
//     scratch row (split path), so the score pass needs no second K read.
//   * Score pass: every occupied slot adds its weight with a Kahan-compensated
//     fp32 sum; eviction candidates compete on a 64-bit key (score bits, pos),
//     which orders by score then position exactly; a wave/LDS min picks the
//     victim, whose slot the new token's K/V, position and score overwrite.
//   * Split path (few units): nsplit blocks per unit each stream a slice of the
//     slots and publish (max, sum, o) partials; the last block to arrive merges
//     them and runs the score pass.
#include "h2o_device.h"
#include "launch.h"

namespace h2o {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;
constexpr uint64_t kNoKey = ~0ull;
constexpr int kNewSlot = -2;

template <typename T, int D>
struct Layout {
  static constexpr int EPL = Elem<T>::kPer16B;  // elements per lane
  static constexpr int LPR = D / EPL;           // lanes per K/V row
  static constexpr int NG = kThreads / LPR;     // row groups per block
  static_assert((LPR & (LPR - 1)) == 0 && LPR <= kWave, "row must map to a power-of-two lane group");
};

template <typename T, int D, bool SPLIT>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a) {
  using Lay = Layout<T, D>;
  constexpr int EPL = Lay::EPL, LPR = Lay::LPR, NG = Lay::NG;
  extern __shared__ float s_logit[];  // single-block path: [k + 1], new token at index k
  __shared__ float s_m[NG], s_l[NG], s_w[NG];
  __shared__ float s_o[NG][D];
  __shared__ uint64_t s_key[kThreads / kWave];
  __shared__ int s_slot;
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int g = tid / LPR, r = tid % LPR;
  const int unit = SPLIT ? blockIdx.x / a.nsplit : blockIdx.x;
  const int split = SPLIT ? blockIdx.x % a.nsplit : 0;
  const int s0 = split * a.split_len;
  const int s1 = min(a.count, s0 + a.split_len);

  const T* kb = static_cast<const T*>(a.kslots) + static_cast<size_t>(unit) * a.k * D;
  const T* vb = static_cast<const T*>(a.vslots) + static_cast<size_t>(unit) * a.k * D;
  const T* qn = static_cast<const T*>(a.q) + static_cast<size_t>(unit) * D;
  const T* kn = static_cast<const T*>(a.knew) + static_cast<size_t>(unit) * D;
  const T* vn = static_cast<const T*>(a.vnew) + static_cast<size_t>(unit) * D;
  float* glog = SPLIT ? a.logits + static_cast<size_t>(unit) * (a.k + 1) : nullptr;

  float qf[EPL];
  Elem<T>::unpack(ld16(qn + r * EPL), qf);

  float m = -INFINITY, l = 0.f, o[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) o[e] = 0.f;

  // The new token belongs to the attended set G = S ∪ {i}; group 0 of the first
  // block seeds its running softmax with it.
  if (split == 0 && g == 0) {
    float kf[EPL], vf[EPL];
    Elem<T>::unpack(ld16(kn + r * EPL), kf);
    Elem<T>::unpack(ld16(vn + r * EPL), vf);
    float dot = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) dot = fmaf(qf[e], kf[e], dot);
    const float x = group_sum<LPR>(dot) * a.c2;
    m = x;
    l = 1.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] = vf[e];
    if (r == 0) {
      if (SPLIT) glog[a.k] = x;
      else s_logit[a.k] = x;
    }
  }

  for (int base = s0 + g; base < s1; base += NG * kUnroll) {
    uint4 kr[kUnroll], vr[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int j = min(base + u * NG, s1 - 1);
      kr[u] = ld16_stream(kb + static_cast<size_t>(j) * D + r * EPL);
      vr[u] = ld16_stream(vb + static_cast<size_t>(j) * D + r * EPL);
    }
    float x[kUnroll];
    float mx = m;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      float kf[EPL];
      Elem<T>::unpack(kr[u], kf);
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) dot = fmaf(qf[e], kf[e], dot);
      dot = group_sum<LPR>(dot);
      x[u] = (base + u * NG < s1) ? dot * a.c2 : -INFINITY;
      mx = fmaxf(mx, x[u]);
    }
    if (r == 0) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int j = base + u * NG;
        if (j < s1) {
          if (SPLIT) glog[j] = x[u];
          else s_logit[j] = x[u];
        }
      }
    }
    const float alpha = fast_exp2(m - mx);
    l *= alpha;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] *= alpha;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const float p = fast_exp2(x[u] - mx);
      float vf[EPL];
      Elem<T>::unpack(vr[u], vf);
      l += p;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[e] = fmaf(p, vf[e], o[e]);
    }
    m = mx;
  }

  // ---- merge the row groups of this block
  if (r == 0) {
    s_m[g] = m;
    s_l[g] = l;
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e) s_o[g][r * EPL + e] = o[e];
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int t = 0; t < NG; ++t) M = fmaxf(M, s_m[t]);
  if (tid < NG) s_w[tid] = fast_exp2(s_m[tid] - M);
  __syncthreads();
  float Ls = 0.f;
#pragma unroll
  for (int t = 0; t < NG; ++t) Ls = fmaf(s_l[t], s_w[t], Ls);

  if constexpr (!SPLIT) {
    if (tid < D) {
      float acc = 0.f;
#pragma unroll
      for (int t = 0; t < NG; ++t) acc = fmaf(s_o[t][tid], s_w[t], acc);
      a.out[static_cast<size_t>(unit) * D + tid] = acc / Ls;
    }
  } else {
    float* pp = a.part + (static_cast<size_t>(unit) * a.nsplit + split) * (2 + D);
    if (tid == 0) {
      pp[0] = M;
      pp[1] = Ls;
    }
    if (tid < D) {
      float acc = 0.f;
#pragma unroll
      for (int t = 0; t < NG; ++t) acc = fmaf(s_o[t][tid], s_w[t], acc);
      pp[2 + tid] = acc;
    }
    // Publish the partial and the logits, then count arrivals; the last block
    // of the unit finishes the step.
    __threadfence();
    __syncthreads();
    if (tid == 0) {
      const unsigned prev = atomicAdd(&a.counters[unit], 1u);
      s_last = (prev == static_cast<unsigned>(a.nsplit - 1));
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    const float* pu = a.part + static_cast<size_t>(unit) * a.nsplit * (2 + D);
    float Mg = -INFINITY;
    for (int s = 0; s < a.nsplit; ++s) Mg = fmaxf(Mg, pu[s * (2 + D)]);
    float Lg = 0.f;
    for (int s = 0; s < a.nsplit; ++s) Lg = fmaf(pu[s * (2 + D) + 1], fast_exp2(pu[s * (2 + D)] - Mg), Lg);
    if (tid < D) {
      float acc = 0.f;
      for (int s = 0; s < a.nsplit; ++s)
        acc = fmaf(pu[s * (2 + D) + 2 + tid], fast_exp2(pu[s * (2 + D)] - Mg), acc);
      a.out[static_cast<size_t>(unit) * D + tid] = acc / Lg;
    }
    if (tid == 0) a.counters[unit] = 0u;  // ready for the next step
    M = Mg;
    Ls = Lg;
  }

  // ---- score accumulation over G, then at most one eviction
  const float invL = 1.f / Ls;
  const int cnt = a.count;
  const bool full = (cnt == a.k);
  float* sc = a.score + static_cast<size_t>(unit) * a.k;
  float* cp = a.comp + static_cast<size_t>(unit) * a.k;
  int32_t* ps = a.pos + static_cast<size_t>(unit) * a.k;
  const float* lg = SPLIT ? glog : s_logit;

  uint64_t best = kNoKey;
  int best_slot = -1;
  for (int j = tid; j < cnt; j += kThreads) {
    const float w = fast_exp2(lg[j] - M) * invL;
    float s = sc[j], c = cp[j];
    const float y = w - c;  // Kahan-compensated add of this step's weight
    const float t = s + y;
    c = (t - s) - y;
    s = t;
    sc[j] = s;
    cp[j] = c;
    if (full) {
      const int32_t p = ps[j];
      if (p <= a.cand_limit) {
        const uint64_t key = evict_key(s, p);
        if (key < best) {
          best = key;
          best_slot = j;
        }
      }
    }
  }
  const float w_new = fast_exp2(lg[a.k] - M) * invL;

  int dst = cnt;  // cache not full: the new token takes the next free slot
  int32_t ev = -1;
  if (full) {
    if (a.new_is_candidate && tid == 0) {
      const uint64_t key = evict_key(w_new, a.new_pos);
      if (key < best) {
        best = key;
        best_slot = kNewSlot;
      }
    }
    const uint64_t wm = wave_min_u64(best);
    if ((tid & (kWave - 1)) == 0) s_key[tid / kWave] = wm;
    __syncthreads();
    uint64_t bm = s_key[0];
#pragma unroll
    for (int w = 1; w < kThreads / kWave; ++w) bm = s_key[w] < bm ? s_key[w] : bm;
    if (best == bm) s_slot = best_slot;  // keys are unique: exactly one owner
    __syncthreads();
    ev = static_cast<int32_t>(static_cast<uint32_t>(bm & 0xffffffffu));
    dst = s_slot == kNewSlot ? -1 : s_slot;
  }
  if (dst >= 0) {
    if (tid == dst % kThreads) {  // the thread that last wrote this slot's score
      sc[dst] = w_new;
      cp[dst] = 0.f;
      ps[dst] = a.new_pos;
    }
    if (g == 0) {
      T* kd = static_cast<T*>(a.kslots) + (static_cast<size_t>(unit) * a.k + dst) * D;
      T* vd = static_cast<T*>(a.vslots) + (static_cast<size_t>(unit) * a.k + dst) * D;
      st16(kd + r * EPL, ld16(kn + r * EPL));
      st16(vd + r * EPL, ld16(vn + r * EPL));
    }
  }
  if (tid == 0 && a.evicted != nullptr) a.evicted[unit] = ev;
}

template <typename T, int D>
hipError_t launch_typed(const DecodeArgs& a, int units, hipStream_t s) {
  if (a.nsplit == 1) {
    const size_t shm = static_cast<size_t>(a.k + 1) * sizeof(float);
    hipLaunchKernelGGL((decode_kernel<T, D, false>), dim3(units), dim3(kThreads), shm, s, a);
  } else {
    hipLaunchKernelGGL((decode_kernel<T, D, true>), dim3(units * a.nsplit), dim3(kThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(int dtype, int head_dim, const DecodeArgs& a, int units, hipStream_t s) {
  if (dtype == 0) {
    return head_dim == 64 ? launch_typed<float, 64>(a, units, s) : launch_typed<float, 128>(a, units, s);
  }
  return head_dim == 64 ? launch_typed<bf16_t, 64>(a, units, s) : launch_typed<bf16_t, 128>(a, units, s);
}

}  // namespace h2o
