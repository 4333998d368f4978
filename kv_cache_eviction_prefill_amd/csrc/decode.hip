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
// Work mapping (gfx950, wave64, 256 threads per block; 128 for small budgets
// over many units; one wave per unit for bf16 d=128 at larger budgets over many
// units, two with position rolling):
//   * A K/V row of d elements is 16 bytes per lane over LPR lanes (bf16 d=128:
//     16 lanes), so one wave-wide load instruction moves 4 whole rows (1 KiB),
//     fully coalesced.  The block's 16 row groups walk the unit's slots with
//     2 (4 with few units) rows in flight per group, K and V of a slot loaded
//     together.
//   * bf16 dot products run as packed bf16 dot-product instructions (fp32
//     accumulation), then a 16-lane DPP reduction per row.
//   * Each group keeps an online softmax (max, sum, o) in registers; groups are
//     merged through LDS.  Logits go to LDS (single-block path) or to a global
//     scratch row (split path), so the score pass needs no second K read.
//   * Score pass: every occupied slot adds its weight with a Kahan-compensated
//     fp32 sum; eviction candidates compete on a 64-bit key (score bits, pos),
//     which orders by score then position exactly; a wave/LDS min picks the
//     victim, whose slot the new token's K/V, position and score overwrite.
//   * Split path (few units): nsplit blocks per unit (one- or two-wave blocks
//     for short bf16 d=128 slices) each stream a slice of the slots and write
//     (max, sum, o) partials and their logits; a second launch, one block per
//     unit, merges the partials and runs the score pass.  The launch boundary
//     orders the two: no block waits for another and no device-scope fence is
//     needed (on gfx950 each such fence writes back and invalidates the whole
//     L2 of its XCD).
//   * Several steps per call: a unit whose state fits a block's shared memory
//     keeps it there over all the steps (decode_resident); on the split path
//     each launch repeats the previous step's finish in every block and then
//     attends its own slices (decode_fused), one launch per step; short
//     slices are staged in shared memory, up to four per 512-thread block.
#include <type_traits>

#include "h2o_device.h"
#include "launch.h"

namespace h2o {
namespace {

constexpr int kThreads = 256;
// Small budgets (k <= kSmallK) over many units run 128-thread blocks: the row
// groups of a 256-thread block would each hold only a few slots, and twice as
// many units are in flight per CU (k = 42 over 7,168 units: 40 -> 34 us per
// launch).  With few units the larger blocks stay faster.
constexpr int kSmallThreads = 128;
constexpr int kSmallK = 128;
constexpr int kSmallKUnits = 1024;
constexpr int kUnroll = 2;    // slots in flight per row group (K and V each)
// Fewer than kFewUnits units (one block each, no split) leave most waves of the
// GPU idle; their row groups keep 4 slots in flight instead (512 units, k = 104:
// 9.3 -> 8.8 us per launch; equal or better at every budget measured).
constexpr int kFewUnits = 1024;
constexpr int kUnrollFew = 4;
// bf16 d=128 over many units at budgets above kSmallK runs one wave per unit,
// its 4 row groups with 8 slots in flight each: twice the bytes in flight per
// wave, and the merge and score pass involve no other wave (2048 units: k = 410
// 74 -> 70 us per launch, k = 2048 368 -> 335 us; 7168 units, k = 2048:
// 1310 -> 1276 us).  At k <= kSmallK or with few units it is slower.
constexpr int kWaveThreads = 64;
constexpr int kWaveUnroll = 8;
// The split path's partial blocks for bf16 d=128 are one-wave blocks too when
// each block's slice of slots is short (32 units x 2048 slots, with the finish
// launch, per step: slices of 64 slots 16.0 -> 15.1 us, of 128 16.6 -> 16.4 us;
// with slices of 256 the 256-thread blocks stay faster, 19.4 against 21.1 us).
constexpr int kWaveSplitLen = 128;
// Slices of at most kTwoWaveSplitLen slots are attended by two-wave blocks (the
// staged multi-step launch, 32 units x 2048 slots: 11.3 -> 10.3 us per step
// against one wave).  Multi-step launches attend with the same block shapes as
// one-step launches, so their partials round alike.
constexpr int kTwoWaveSplitLen = 64;
constexpr int kTwoWaveThreads = 128;
// slots in flight per row group of the two-wave blocks (with position rolling
// each also carries a turned query: 4, so the registers hold).  Position
// rolling over many units at budgets above kSmallK runs two-wave blocks too: the
// 256-thread blocks' registers leave only 5 waves per SIMD, less than the grid
// (2048 units, k = 410: 81.3-82.6 -> 76.8-77.6 us per launch).
template <bool ROPE>
constexpr int kTwoWaveUnroll = ROPE ? 4 : kWaveUnroll;
constexpr int kPrefetch = 2;  // score-pass slots per thread whose metadata is loaded up front
constexpr uint64_t kNoKey = ~0ull;
constexpr int kNewSlot = -2;
constexpr int kMaxSplitBlocks = 64;  // most blocks one unit's slots are split over
constexpr int kFinishThreads = 512;  // threads of a finish block (one block per unit)
constexpr int kFinishPrefetch = 4;   // slots per thread whose metadata the finish launch loads first

template <typename T, int D, int NT = kThreads>
struct Layout {
  static constexpr int EPL = Elem<T>::kPer16B;  // elements per lane
  static constexpr int LPR = D / EPL;           // lanes per K/V row
  static constexpr int NG = NT / LPR;           // row groups per block
  static_assert((LPR & (LPR - 1)) == 0 && LPR <= kWave, "row must map to a power-of-two lane group");
  static_assert(LPR >= kUnroll, "one lane per in-flight slot stores its logit");
};

// Where one unit's state lives for a step: its slot rows and per-slot score,
// compensation and position (global memory, or a block's shared-memory copy),
// the new token's q/k/v rows, and (position rolling) the slots' places among
// the cached entries.
template <typename T>
struct UnitRefs {
  T* k;
  T* v;
  float* sc;
  float* cp;
  int32_t* ps;
  const T* qn;
  const T* kn;
  const T* vn;
  const int32_t* rk;
};

// A unit's state in global memory.
template <typename T, int D>
__device__ inline UnitRefs<T> global_refs(const DecodeArgs& a, int unit) {
  const size_t u = static_cast<size_t>(unit);
  return {static_cast<T*>(a.kslots) + u * a.k * D, static_cast<T*>(a.vslots) + u * a.k * D,
          a.score + u * a.kstride, a.comp + u * a.kstride, a.pos + u * a.kstride,
          static_cast<const T*>(a.q) + u * D, static_cast<const T*>(a.knew) + u * D,
          static_cast<const T*>(a.vnew) + u * D, a.rank != nullptr ? a.rank + u * a.kstride : nullptr};
}

// Adds a step's weight w to a slot's score s with compensation c: a Kahan step
// when compensating, a plain fp32 add otherwise (c stays 0).  No product is
// contracted into these additions, so every kernel that scores rounds alike.
__device__ inline void add_weight(float w, float& s, float& c, bool compensate) {
#pragma clang fp contract(off)
  const float y = w - c;
  const float t = s + y;
  c = compensate ? (t - s) - y : 0.f;
  s = t;
}

// Score pass of one unit (whole block): every occupied slot adds its weight
// exp2(x_j - M) / L with a Kahan-compensated fp32 sum (with fixed scores nothing
// is added and the new token's score is given); when the cache is full the
// eviction candidates (pos <= i - K_r, and the new token when K_r = 0) compete on
// the 64-bit key (score bits, pos) through a wave and LDS min, and the new
// token's K/V, position and score overwrite the victim's slot.  pf_*: this
// thread's first NP slots' metadata, loaded early by the caller; lg: the unit's
// logits, the new token's at index k; s_knew/s_vnew: its K/V rows, in LDS.
template <typename T, int D, int NP, bool kPfX, int NT = kThreads>
__device__ inline void score_pass(const DecodeArgs& a, int unit, const UnitRefs<T>& ur, float M, float invL,
                                  const float* lg, float x_new,
                                  const float (&pf_s)[NP], const float (&pf_c)[NP], const int32_t (&pf_p)[NP],
                                  const float (&pf_x)[NP], const uint4* s_knew, const uint4* s_vnew,
                                  uint64_t* s_key, int* s_slot, int* s_vrank) {
  using Lay = Layout<T, D>;
  constexpr int EPL = Lay::EPL, LPR = Lay::LPR;
  const int tid = threadIdx.x, g = tid / LPR, r = tid % LPR;
  float* sc = ur.sc;
  float* cp = ur.cp;
  int32_t* ps = ur.ps;
  T* ku = ur.k;
  T* vu = ur.v;
  const int cnt = a.count;
  const bool full = (cnt == a.k);
  const bool accumulate = a.fixed_new == nullptr;  // else scores are fixed (global comparator)
  const bool compensate = a.new_pos >= a.plain_until;

  uint64_t best = kNoKey;
  int best_slot = -1;
  for (int i = 0, j = tid; j < cnt; ++i, j += NT) {
    float xj, sj, cj;
    int32_t pj;
    if (i < NP) {
      xj = pf_x[0];
      sj = pf_s[0];
      cj = pf_c[0];
      pj = pf_p[0];
#pragma unroll
      for (int t = 1; t < NP; ++t) {
        xj = i == t ? pf_x[t] : xj;
        sj = i == t ? pf_s[t] : sj;
        cj = i == t ? pf_c[t] : cj;
        pj = i == t ? pf_p[t] : pj;
      }
      if (!kPfX) xj = lg[j];
    } else {
      xj = lg[j];
      sj = sc[j];
      cj = compensate ? cp[j] : 0.f;
      pj = ps[j];
    }
    if (accumulate) {
      add_weight(fast_exp2(xj - M) * invL, sj, cj, compensate);
      if (compensate) cp[j] = cj;  // the compensation stays 0 until compensated adds begin
      sc[j] = sj;
    }
    if (full && pj <= a.cand_limit) {
      const uint64_t key = evict_key(sj, pj) | pattern_bit(a.pat_kind, a.pat_period, a.pat_width, pj, a.new_pos);
      if (key < best) {
        best = key;
        best_slot = j;
      }
    }
  }
  const float w_new = accumulate ? fast_exp2(x_new - M) * invL : a.fixed_new[static_cast<size_t>(unit) * a.fixed_stride];

  int dst = cnt;  // cache not full: the new token takes the next free slot
  int32_t ev = -1;
  if (full) {
    if (a.new_is_candidate && tid == 0) {
      const uint64_t key = evict_key(w_new, a.new_pos) |
                           pattern_bit(a.pat_kind, a.pat_period, a.pat_width, a.new_pos, a.new_pos);
      if (key < best) {
        best = key;
        best_slot = kNewSlot;
      }
    }
    const uint64_t wm = wave_min_key(best);
    if ((tid & (kWave - 1)) == 0) s_key[tid / kWave] = wm;
    __syncthreads();
    uint64_t bm = s_key[0];
#pragma unroll
    for (int w = 1; w < NT / kWave; ++w) bm = s_key[w] < bm ? s_key[w] : bm;
    ev = static_cast<int32_t>(static_cast<uint32_t>(bm & 0xffffffffu));
    if (a.rank == nullptr) {
      // the wave holding the minimum writes the new token over the victim (its
      // owner lane last wrote that slot's score): no second block barrier
      const uint64_t own = __ballot(best == bm);
      if (own != 0) {
        const int ol = __ffsll(static_cast<unsigned long long>(own)) - 1;
        const int vs = __builtin_amdgcn_readlane(best_slot, ol);
        if (vs >= 0) {
          const int lane = tid & (kWave - 1);
          if (lane == ol) {
            sc[vs] = w_new;
            cp[vs] = 0.f;
            ps[vs] = a.new_pos;
          }
          if (lane < LPR) {
            T* kd = ku + static_cast<size_t>(vs) * D;
            T* vd = vu + static_cast<size_t>(vs) * D;
            st16(kd + r * EPL, s_knew[r]);
            st16(vd + r * EPL, s_vnew[r]);
          }
        }
      }
      if (tid == 0 && a.evicted != nullptr) a.evicted[unit] = ev;
      return;
    }
    // position rolling: every thread needs the victim's place among the entries
    if (best == bm) {  // keys are unique: exactly one owner
      *s_slot = best_slot;
      if (best_slot >= 0) *s_vrank = a.rank[static_cast<size_t>(unit) * a.kstride + best_slot];
    }
    __syncthreads();
    dst = *s_slot == kNewSlot ? -1 : *s_slot;
  }
  if (dst >= 0) {
    if (tid == dst % NT) {  // the thread that last wrote this slot's score
      sc[dst] = w_new;
      cp[dst] = 0.f;
      ps[dst] = a.new_pos;
    }
    if (g == 0) {  // s_knew/s_vnew were written before an earlier barrier
      T* kd = ku + static_cast<size_t>(dst) * D;
      T* vd = vu + static_cast<size_t>(dst) * D;
      st16(kd + r * EPL, s_knew[r]);
      st16(vd + r * EPL, s_vnew[r]);
    }
  }
  if (a.rank != nullptr) {  // position rolling: keep every slot's place among the cached entries
    int32_t* rk = a.rank + static_cast<size_t>(unit) * a.kstride;
    if (!full) {
      if (tid == 0) rk[cnt] = cnt;  // the new token is the latest entry
    } else if (dst >= 0) {
      const int rv = *s_vrank;  // entries after the victim move down one place
      for (int j = tid; j < cnt; j += NT) {
        if (j == dst) continue;
        const int32_t rj = rk[j];
        if (rj > rv) rk[j] = rj - 1;
      }
      if (tid == 0) rk[dst] = a.k - 1;
    }
  }
  if (tid == 0 && a.evicted != nullptr) a.evicted[unit] = ev;
}

// Rotary embedding at positions inside the cache: a cached entry at place r
// and the new token at place `count` give the logit k . R(-(r - count)) q, so the
// query is turned per slot.  Each lane holds EPL elements of one half of the
// pairs (m, m + d/2); its partner lane (lane ^ LPR/2) holds the other half.
template <typename T, int D>
struct RopeLane {
  static constexpr int EPL = Layout<T, D>::EPL, LPR = Layout<T, D>::LPR;
  // With 16 lanes per row the partner lane (lane ^ 8) sits in the same DPP row:
  // each lane then evaluates the angles of only half of its pairs and takes the
  // other half from its partner, which needs the same (cos, sin) values.
  static constexpr bool kShare = LPR == 16;
  static constexpr int NA = kShare ? EPL / 2 : EPL;  // angles this lane evaluates
  float qp[EPL];       // the partner lane's query elements
  float hi[NA], lo[NA];  // theta_m / (2 pi) of the pairs this lane evaluates, split
  float sgn;           // +1 on the first half of the pairs, -1 on the second
  __device__ void init(const DecodeArgs& a, const float (&qf)[EPL], int r) {
    const bool second = r >= LPR / 2;
#pragma unroll
    for (int e = 0; e < EPL; ++e) qp[e] = __shfl_xor(qf[e], LPR / 2, kWave);
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      // shared: the first-half lane evaluates pairs e < EPL/2, its partner the rest
      const int m = (r % (LPR / 2)) * EPL + (kShare && second ? EPL / 2 : 0) + i;
      hi[i] = a.rope_th[2 * m];
      lo[i] = a.rope_th[2 * m + 1];
    }
    sgn = second ? -1.f : 1.f;
  }
  // q turned by -(rank gap) n: q c + sgn * q' s with (c, s) of the angle n theta_m
  __device__ void turn(const float (&qf)[EPL], int n, float (&qr)[EPL]) const {
    const float dn = static_cast<float>(n);
    float c[NA], s[NA];
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      float t = dn * hi[i];  // exact: hi has at most 11 significant bits, |n| < 2^14
      t -= rintf(t);
      t = fmaf(dn, lo[i], t);
      t -= rintf(t);  // fraction of a turn
      c[i] = __builtin_amdgcn_cosf(t);
      s[i] = __builtin_amdgcn_sinf(t);
    }
    if constexpr (kShare) {
      // pairs e < EPL/2: the first-half lanes' own values, copied into the
      // second-half lanes (banks 2, 3 of the row); pairs e >= EPL/2: the other way
#pragma unroll
      for (int i = 0; i < NA; ++i) {
        const int ci = __float_as_int(c[i]), si = __float_as_int(s[i]);
        const float c_lo = __int_as_float(__builtin_amdgcn_update_dpp(ci, ci, kDppRowRor8, 0xF, 0xC, false));
        const float s_lo = __int_as_float(__builtin_amdgcn_update_dpp(si, si, kDppRowRor8, 0xF, 0xC, false));
        const float c_hi = __int_as_float(__builtin_amdgcn_update_dpp(ci, ci, kDppRowRor8, 0xF, 0x3, false));
        const float s_hi = __int_as_float(__builtin_amdgcn_update_dpp(si, si, kDppRowRor8, 0xF, 0x3, false));
        qr[i] = fmaf(qf[i], c_lo, sgn * qp[i] * s_lo);
        qr[i + NA] = fmaf(qf[i + NA], c_hi, sgn * qp[i + NA] * s_hi);
      }
    } else {
#pragma unroll
      for (int e = 0; e < EPL; ++e) qr[e] = fmaf(qf[e], c[e], sgn * qp[e] * s[e]);
    }
  }
};

// Barrier among a block's NT threads before they read each other's shared
// memory: a one-wave block's lanes issue in order, so ordering the wave's own
// shared-memory traffic is enough (and such a block may run inside a larger
// launch whose other waves have left).
template <int NT>
__device__ inline void block_sync() {
  if constexpr (NT == kWave) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  } else {
    __syncthreads();
  }
}

// The block's shared memory for one decode step (the logits, [k + 1] on the
// single-block path, are dynamic shared memory of the launch).
template <typename T, int D, int NT>
struct StepShared {
  static constexpr int LPR = Layout<T, D, NT>::LPR, NG = Layout<T, D, NT>::NG;
  float m[NG], l[NG];
  float o[NG][D];
  uint64_t key[NT / kWave];
  uint4 knew[LPR], vnew[LPR];
  int slot, vrank;
};

// Dot product of a lane's 8 bf16 key and query elements: four packed bf16
// dot-product-accumulate steps, pairs (0,1), (2,3), (4,5), (6,7) in order.
__device__ inline float dot8_bf16(const uint4& k, const uint4& q) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  float d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, k.x), __builtin_bit_cast(bf16x2, q.x), 0.f,
                                            false);
  d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, k.y), __builtin_bit_cast(bf16x2, q.y), d, false);
  d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, k.z), __builtin_bit_cast(bf16x2, q.z), d, false);
  d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, k.w), __builtin_bit_cast(bf16x2, q.w), d, false);
  return d;
}

// One decode step of one unit (SPLIT: of one slice of its slots).  ku/vu: the
// unit's slot rows, in global memory, or (LDSKV) the block's copy of them in
// shared memory, which the step reads and overwrites in place (a split step:
// the copy of its slice's rows alone, row 0 the slice's first slot).  tid: the
// thread's index among the NT threads that run the step.
template <typename T, int D, bool SPLIT, bool ROPE, int NT, int UN, bool LDSKV>
__device__ __forceinline__ void decode_step(const DecodeArgs& a, int unit, int split, const UnitRefs<T>& ur,
                                            float* s_logit, StepShared<T, D, NT>& sh, int tid) {
  using Lay = Layout<T, D, NT>;
  constexpr int NP = NT >= kThreads ? kPrefetch : 512 / NT;  // score-pass slots prefetched per thread
  constexpr int NC = (D + NT - 1) / NT;                       // output columns per thread in the merge
  static_assert(Lay::LPR >= UN, "one lane per in-flight slot stores its logit");
  constexpr int EPL = Lay::EPL, LPR = Lay::LPR, NG = Lay::NG;
  float* s_m = sh.m;
  float* s_l = sh.l;
  float (*s_o)[D] = sh.o;
  uint64_t* s_key = sh.key;
  uint4* s_knew = sh.knew;
  uint4* s_vnew = sh.vnew;

  const int g = tid / LPR, r = tid % LPR;
  const int s0 = split * a.split_len;
  const int s1 = min(a.count, s0 + a.split_len);

  const T* kb = ur.k;
  const T* vb = ur.v;
  const T* qn = ur.qn;
  const T* kn = ur.kn;
  const T* vn = ur.vn;
  float* glog = SPLIT ? a.logits + static_cast<size_t>(unit) * (a.k + 1) : nullptr;
  const float* sc = ur.sc;
  const float* cp = ur.cp;
  const int32_t* ps = ur.ps;

  float qf[EPL];
  const uint4 q_raw = ld16(qn + r * EPL);
  Elem<T>::unpack(q_raw, qf);
  // packed bf16 dot products, except in the one-wave blocks of the single-block
  // path: those stream at the HBM rate either way, and with them they ran the
  // 7168-unit, k = 2048 launch slower (941 against 918 us)
  constexpr bool kDot2 = std::is_same<T, bf16_t>::value && !ROPE && !(NT == kWaveThreads && !SPLIT);
  RopeLane<T, D> rope;
  const int32_t* rkb = ROPE ? ur.rk : nullptr;
  if constexpr (ROPE) rope.init(a, qf, r);
  // The new token's rows are loaded once: group 0 attends to them and parks them
  // in LDS for the overwrite at the end.
  uint4 kn_raw = make_uint4(0u, 0u, 0u, 0u), vn_raw = make_uint4(0u, 0u, 0u, 0u);
  if (g == 0) {
    kn_raw = ld16(kn + r * EPL);
    vn_raw = ld16(vn + r * EPL);
    s_knew[r] = kn_raw;
    s_vnew[r] = vn_raw;
  }
  // Score-pass metadata of this thread's first slots: loaded now, it arrives
  // under the K/V stream instead of after it.
  float pf_s[NP], pf_c[NP];
  int32_t pf_p[NP];
  if (!SPLIT) {
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int j = tid + i * NT;
      const bool ok = j < a.count;
      pf_s[i] = ok ? sc[j] : 0.f;
      pf_c[i] = ok && a.new_pos >= a.plain_until ? cp[j] : 0.f;
      pf_p[i] = ok ? ps[j] : 0;
    }
  }

  float m = -INFINITY, l = 0.f, o[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) o[e] = 0.f;

  // The new token belongs to the attended set G = S ∪ {i}; group 0 of the first
  // block seeds its running softmax with it.
  if (split == 0 && g == 0) {
    float kf[EPL], vf[EPL];
    Elem<T>::unpack(kn_raw, kf);
    Elem<T>::unpack(vn_raw, vf);
    float dot = 0.f;
    if constexpr (kDot2) {
      dot = dot8_bf16(kn_raw, q_raw);
    } else {
#pragma unroll
      for (int e = 0; e < EPL; ++e) dot = fmaf(qf[e], kf[e], dot);
    }
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

  for (int base = s0 + g; base < s1; base += NG * UN) {
    uint4 kr[UN], vr[UN];
    int32_t rkj[UN];
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const int j = min(base + u * NG, s1 - 1);
      if constexpr (LDSKV) {
        const int jl = SPLIT ? j - s0 : j;  // a split block holds its slice alone
        kr[u] = ld16(kb + static_cast<size_t>(jl) * D + r * EPL);
        vr[u] = ld16(vb + static_cast<size_t>(jl) * D + r * EPL);
      } else {
        kr[u] = ld16_stream(kb + static_cast<size_t>(j) * D + r * EPL);
        vr[u] = ld16_stream(vb + static_cast<size_t>(j) * D + r * EPL);
      }
      if constexpr (ROPE) rkj[u] = rkb[LDSKV && SPLIT ? j - s0 : j];
    }
    float x[UN];
    float mx = m;
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      float dot = 0.f;
      if constexpr (kDot2) {
        dot = dot8_bf16(kr[u], q_raw);
      } else if constexpr (ROPE) {
        float kf[EPL];
        Elem<T>::unpack(kr[u], kf);
        float qr[EPL];
        rope.turn(qf, rkj[u] - a.count, qr);
#pragma unroll
        for (int e = 0; e < EPL; ++e) dot = fmaf(qr[e], kf[e], dot);
      } else {
        float kf[EPL];
        Elem<T>::unpack(kr[u], kf);
#pragma unroll
        for (int e = 0; e < EPL; ++e) dot = fmaf(qf[e], kf[e], dot);
      }
      dot = group_sum<LPR>(dot);
      x[u] = (base + u * NG < s1) ? dot * a.c2 : -INFINITY;
      mx = fmaxf(mx, x[u]);
    }
    // lane u of the group stores the logit of in-flight slot u
    if (r < UN) {
      const int j = base + r * NG;
      float xr = x[0];
#pragma unroll
      for (int u = 1; u < UN; ++u) xr = r == u ? x[u] : xr;
      if (j < s1) {
        if (SPLIT) glog[j] = xr;
        else s_logit[j] = xr;
      }
    }
    const float alpha = fast_exp2(m - mx);
    l *= alpha;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] *= alpha;
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const float p = fast_exp2(x[u] - mx);
      float vf[EPL];
      Elem<T>::unpack(vr[u], vf);
      l += p;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[e] = fmaf(p, vf[e], o[e]);
    }
    m = mx;
  }

  // ---- merge the row groups of this block (every thread derives the weights)
  if (r == 0) {
    s_m[g] = m;
    s_l[g] = l;
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e) s_o[g][r * EPL + e] = o[e];
  block_sync<NT>();
  float M = -INFINITY;
#pragma unroll 8
  for (int t = 0; t < NG; ++t) M = fmaxf(M, s_m[t]);
  float Ls = 0.f, acc[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) acc[c] = 0.f;
#pragma unroll 8
  for (int t = 0; t < NG; ++t) {
    const float wt = fast_exp2(s_m[t] - M);
    Ls = fmaf(s_l[t], wt, Ls);
#pragma unroll
    for (int c = 0; c < NC; ++c)
      if (tid + c * NT < D) acc[c] = fmaf(s_o[t][tid + c * NT], wt, acc[c]);
  }

  if constexpr (SPLIT) {
    float* pp = a.part + (static_cast<size_t>(unit) * a.nsplit + split) * (2 + D);
    if (tid == 0) {
      pp[0] = M;
      pp[1] = Ls;
    }
#pragma unroll
    for (int c = 0; c < NC; ++c)
      if (tid + c * NT < D) pp[2 + tid + c * NT] = acc[c];
  } else {
#pragma unroll
    for (int c = 0; c < NC; ++c)
      if (tid + c * NT < D) a.out[static_cast<size_t>(unit) * D + tid + c * NT] = acc[c] / Ls;
    score_pass<T, D, NP, false, NT>(a, unit, ur, M, 1.f / Ls, s_logit, s_logit[a.k], pf_s, pf_c, pf_p, pf_s,
                                    s_knew, s_vnew, s_key, &sh.slot, &sh.vrank);
  }
}

// 8 waves per SIMD: all blocks of a 2048-unit launch are resident at once.  A
// one-wave block keeps its 8 slots per group in flight with up to 256 registers.
template <typename T, int D, bool SPLIT, bool ROPE, int NT = kThreads, int UN = kUnroll>
__global__ __launch_bounds__(NT, NT == kWaveThreads ? 2 : (ROPE || UN > kUnroll ? 4 : 8)) void decode_kernel(
    DecodeArgs a) {
  extern __shared__ float s_logit[];  // single-block path: [k + 1], new token at index k
  __shared__ StepShared<T, D, NT> sh;
  const int unit = SPLIT ? blockIdx.x / a.nsplit : blockIdx.x;
  const int split = SPLIT ? blockIdx.x % a.nsplit : 0;
  decode_step<T, D, SPLIT, ROPE, NT, UN, false>(a, unit, split, global_refs<T, D>(a, unit), s_logit, sh,
                                                threadIdx.x);
}

// Butterfly reductions over the wave: at every level the two partner lanes
// combine the same two values, so every lane ends with the same result.
__device__ inline float wave_max_f(float v) {
#pragma unroll
  for (int m = kWave / 2; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}
__device__ inline float wave_sum_f(float v) {
#pragma unroll
  for (int m = kWave / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// Merge of one unit's split partials (max m_q, sum l_q, numerator o_q), the
// same in every wave: lane q holds partial q's (m_q, l_q) (pm, pl; -inf and 0
// past nsplit), Mg = max_q m_q, the weight w_q = exp2(m_q - Mg) and
// Lg = sum_q l_q w_q.  Returns this lane's w_q (0 past nsplit).
__device__ inline float merge_weights(float pm, float pl, int nsplit, float& Mg, float& Lg) {
#pragma clang fp contract(off)
  const bool ok = static_cast<int>(threadIdx.x & (kWave - 1)) < nsplit;
  Mg = wave_max_f(pm);
  const float w = ok ? fast_exp2(pm - Mg) : 0.f;
  Lg = wave_sum_f(pl * w);
  return w;
}

// One column of the merged numerator, sum_q o_q w_q in order of q: po holds the
// column of every partial (0 past nsplit), w the lanes' partial weights.
template <int NS>
__device__ inline float merge_column(const float (&po)[NS], float w) {
  static_assert(NS <= kWave, "one lane per partial");
  float og = 0.f;
#pragma unroll
  for (int q = 0; q < NS; ++q)
    og = fmaf(po[q], __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), q)), og);
  return og;
}

// Second launch of the split path: one block per unit merges the nsplit
// partials of the first launch into the output and runs the score pass over the
// logits it wrote.
template <typename T, int D>
__global__ __launch_bounds__(kFinishThreads) void decode_finish(DecodeArgs a) {
  using Lay = Layout<T, D>;
  constexpr int EPL = Lay::EPL, LPR = Lay::LPR;
  constexpr int NT = kFinishThreads;
  constexpr int NP = kFinishPrefetch;
  __shared__ uint64_t s_key[NT / kWave];
  __shared__ uint4 s_knew[LPR], s_vnew[LPR];
  __shared__ int s_slot, s_vrank;
  const int tid = threadIdx.x, unit = blockIdx.x;
  const float* sc = a.score + static_cast<size_t>(unit) * a.kstride;
  const float* cp = a.comp + static_cast<size_t>(unit) * a.kstride;
  const int32_t* ps = a.pos + static_cast<size_t>(unit) * a.kstride;
  const float* lg = a.logits + static_cast<size_t>(unit) * (a.k + 1);
  const float* pu = a.part + static_cast<size_t>(unit) * a.nsplit * (2 + D);
  // Every load is issued here, before any result is used: the metadata and
  // logits of this thread's first NP slots, its output column of every partial,
  // the partials' (max, sum) and the new token's rows.
  float pf_s[NP], pf_c[NP], pf_x[NP];
  int32_t pf_p[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int j = tid + i * NT;
    const bool ok = j < a.count;
    pf_x[i] = ok ? lg[j] : 0.f;
    pf_s[i] = ok ? sc[j] : 0.f;
    pf_c[i] = ok && a.new_pos >= a.plain_until ? cp[j] : 0.f;
    pf_p[i] = ok ? ps[j] : 0;
  }
  const float x_new = lg[a.k];
  float po[kMaxSplitBlocks];
#pragma unroll
  for (int s = 0; s < kMaxSplitBlocks; ++s)
    po[s] = (tid < D && s < a.nsplit) ? pu[s * (2 + D) + 2 + tid] : 0.f;
  const int lane = tid & (kWave - 1);
  const float pm = lane < a.nsplit ? pu[lane * (2 + D)] : -INFINITY;
  const float pl = lane < a.nsplit ? pu[lane * (2 + D) + 1] : 0.f;
  if (tid < LPR) {
    s_knew[tid] = ld16(static_cast<const T*>(a.knew) + static_cast<size_t>(unit) * D + tid * EPL);
    s_vnew[tid] = ld16(static_cast<const T*>(a.vnew) + static_cast<size_t>(unit) * D + tid * EPL);
  }
  __syncthreads();
  float Mg, Lg;
  const float ws = merge_weights(pm, pl, a.nsplit, Mg, Lg);
  if (tid < D) a.out[static_cast<size_t>(unit) * D + tid] = merge_column(po, ws) / Lg;
  score_pass<T, D, NP, true, NT>(a, unit, global_refs<T, D>(a, unit), Mg, 1.f / Lg, lg, x_new, pf_s, pf_c, pf_p,
                                 pf_x, s_knew, s_vnew, s_key, &s_slot, &s_vrank);
}

// Split-path steps of a multi-step call, one launch per step instead of two.
// Launch t finishes step t-1 and runs step t's slices: every block of a unit
// repeats step t-1's finish (merge the unit's partials, add each weight to every
// score, find the victim over all candidates) with the finish launch's
// arithmetic, writes the updated score, compensation and position of the slots
// in its own step-t slices to the other buffer of each (`ny`; nothing another
// block still reads is overwritten), puts token t-1 into the victim's slot when
// that slot is in its slices, and then runs step t's slices exactly as the split
// launch does.  The unit's first block writes step t-1's output and eviction.
// The result equals one split launch and one finish launch per step, bit for bit.
//
// STAGE: the block's step-t slice of K/V rows and step t's q/k/v rows are
// fetched into shared memory at the start (the slice by direct-to-LDS loads,
// which stay in flight through the finish), the victim's row is patched there,
// and the slice is attended from shared memory; every load of the launch is then
// issued before the first result is used.  Without it the slice is read from
// global memory after the finish.
constexpr int kFusedThreads = 256;
constexpr int kFusedPrefetch = 8;  // slots per thread whose metadata is loaded in one batch
constexpr int kStageBytes = 16 * 1024;  // largest staged K (or V) slice
constexpr int kStagePartials = 32;  // most partials per unit of the staged launch
// Staged launches over at least this many slices run two slices per block, each
// attended by its own two waves, so half as many blocks repeat the finish
// (32 units x 2048 slots: 10.4 -> 9.1 us per step).
constexpr int kPairedSlices = 512;
// Over at least this many slices a 512-thread block holds four slices (one
// block per CU, 128 KB of staged rows): a quarter as many blocks repeat the
// finish, each thread finishing half as many slots (32 units x 2048 slots:
// 9.1-9.3 -> 8.5 us per step).
constexpr int kQuadSlices = 1024;
constexpr int kQuadThreads = 512;

// Blocks are dealt to the 8 XCDs round-robin.  With a grid that divides evenly,
// block b runs as logical block (b mod 8) * grid/8 + b/8, so consecutive logical
// blocks, the slices of one unit, share an XCD: each unit's metadata, logits and
// partials are then fetched into one L2 and shared there by all of its blocks.
constexpr int kXcds = 8;
__device__ inline int xcd_block() {
  const int b = blockIdx.x, g = gridDim.x;
  return g % kXcds == 0 ? (b % kXcds) * (g / kXcds) + b / kXcds : b;
}

// Buffer descriptor over `bytes` bytes from `base`, and 4-byte loads through
// one: an offset at or past the end (kPastEnd always is) reads 0.
constexpr int kPastEnd = 0x7ffffff0;
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
__device__ inline uint32_t ld_u32(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ inline float ld_f32(__amdgpu_buffer_rsrc_t r, int off) { return __uint_as_float(ld_u32(r, off)); }
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ inline u32x4 ld_u32x4(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

// Barrier for shared memory alone: unlike __syncthreads it does not wait for the
// block's global loads still in flight.
__device__ inline void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// NS: step t-1's partials per unit held in registers (>= p.nsplit; the merge
// adds the same terms in the same order for any NS >= nsplit).  SPB: step-t
// slices per block (1, or 2 or 4 when STAGE: one per NTP-thread group; the
// finish is then repeated by a half or a quarter as many blocks).  NT: threads
// per block (256; 512 for four slices).  ROPE: position rolling; each block
// also moves the places of its slices' slots past step t-1's eviction (to
// ny_rank) and attends with them.
template <typename T, int D, int NTP, int UNP, bool STAGE, int NS, int SPB, bool ROPE, int NT = kFusedThreads>
__global__ __launch_bounds__(NT, NT > kFusedThreads ? 2 : 4) void decode_fused(DecodeArgs p, DecodeArgs b,
                                                                           float* ny_score, float* ny_comp,
                                                                           int32_t* ny_pos, int32_t* ny_rank) {
  constexpr int EPL = Layout<T, D>::EPL, LPR = Layout<T, D>::LPR;
  constexpr int NGP = NTP / LPR;  // row groups of one slice's attending threads
  static_assert(NS <= kMaxSplitBlocks, "partials per unit");
  static_assert(!STAGE || 3 * LPR <= kWave, "wave 0 moves step t's q/k/v rows");
  static_assert(SPB == 1 || (STAGE && SPB * NTP <= NT), "several slices per block: staged, one thread group each");
  constexpr int KB = SPB * kStageBytes;  // staged K (or V) bytes
  static_assert(KB % (NT * 16) == 0, "the stage splits into block-wide 16-byte loads");
  __shared__ uint64_t s_key[NT / kWave];
  __shared__ int s_slot, s_vrank;
  __shared__ StepShared<T, D, NTP> sh[SPB];
  __shared__ int32_t s_rank[ROPE && STAGE ? SPB * kStageBytes / (D * sizeof(T)) : 1];  // the slices' places
  __shared__ uint4 s_tok[3][LPR];                            // STAGE: step t's q, k, v rows
  extern __shared__ __align__(16) unsigned char s_stage[];  // STAGE: K rows | V rows of the block's slices
  const int tid = threadIdx.x, lb = xcd_block();
  const int bpu = b.nsplit / SPB;  // blocks per unit (the host makes nsplit a multiple of SPB)
  const int unit = lb / bpu, split0 = (lb % bpu) * SPB;
  // this block's step-t slots: slices split0 .. split0 + SPB - 1
  const int s0 = split0 * b.split_len, s1 = min(b.count, s0 + SPB * b.split_len);
  const size_t uk = static_cast<size_t>(unit) * p.kstride;
  const float* lg = p.logits + static_cast<size_t>(unit) * (p.k + 1);
  const float* pu = p.part + static_cast<size_t>(unit) * p.nsplit * (2 + D);
  const bool compensate = p.new_pos >= p.plain_until;
  const int cnt = p.count;
  const bool full = cnt == p.k;
  // ---- every load first: step t's q/k/v rows, the partials' (max, sum), the
  // metadata of kFusedPrefetch consecutive slots per thread (16-byte loads),
  // token t-1's rows and then the K/V slices, so the block waits out one memory
  // latency, not one per slot; fewer than the 63 loads a wave can have in
  // flight are issued before the slices, so no wait delays them
  const int which = tid / LPR, part = tid % LPR;
  uint4 tok = {};
  if (STAGE && which < 3) {
    const T* src = static_cast<const T*>(which == 0 ? b.q : which == 1 ? b.knew : b.vnew);
    tok = ld16(src + static_cast<size_t>(unit) * D + part * EPL);
  }
  // Through buffer descriptors bounded by the unit's occupied slots (and its
  // partials): bytes past the end read as 0, so no load needs a branch (slots
  // past the occupied count are loaded but never used).
  constexpr int NP = kFusedPrefetch * kFusedThreads / NT;  // one batch covers the same slots at any NT
  static_assert(NP % 4 == 0, "whole 16-byte loads");
  const uint32_t nb = static_cast<uint32_t>(cnt) * 4;
  const __amdgpu_buffer_rsrc_t r_lg = make_rsrc(lg, nb), r_sc = make_rsrc(p.score + uk, nb);
  const __amdgpu_buffer_rsrc_t r_cp = make_rsrc(p.comp + uk, compensate ? nb : 0u);  // plain adds: c = 0
  const __amdgpu_buffer_rsrc_t r_ps = make_rsrc(p.pos + uk, nb);
  const __amdgpu_buffer_rsrc_t r_rk = make_rsrc(ROPE ? p.rank + uk : p.pos + uk, ROPE ? nb : 0u);
  const __amdgpu_buffer_rsrc_t r_pu = make_rsrc(pu, static_cast<uint32_t>(p.nsplit) * (2 + D) * 4);
  const int lane = tid & (kWave - 1);
  float pm = lane < p.nsplit ? ld_f32(r_pu, lane * (2 + D) * 4) : -INFINITY;
  float pl = ld_f32(r_pu, (lane * (2 + D) + 1) * 4);  // 0 past nsplit
  float rx[NP], rs[NP], rc[NP];
  int32_t rp[NP], rr[NP];
  const auto fetch = [&](int base) {  // slots base + tid * NP + i
#pragma unroll
    for (int i = 0; i < NP; i += 4) {
      const int off = (base + tid * NP + i) * 4;
      const u32x4 x = ld_u32x4(r_lg, off), sc = ld_u32x4(r_sc, off), c = ld_u32x4(r_cp, off),
                  ps = ld_u32x4(r_ps, off);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        rx[i + e] = __uint_as_float(x[e]);
        rs[i + e] = __uint_as_float(sc[e]);
        rc[i + e] = __uint_as_float(c[e]);
        rp[i + e] = static_cast<int32_t>(ps[e]);
      }
      if constexpr (ROPE) {
        const u32x4 rk4 = ld_u32x4(r_rk, off);
#pragma unroll
        for (int e = 0; e < 4; ++e) rr[i + e] = static_cast<int32_t>(rk4[e]);
      }
    }
  };
  fetch(0);
  // position rolling, staged: the place of this thread's slot of the block's slices
  const int nmine = s1 - s0;  // staged: at most NT
  const int32_t myrank = ROPE && STAGE && tid < nmine ? static_cast<int32_t>(ld_u32(r_rk, (s0 + tid) * 4)) : 0;
  const bool lead = split0 == 0;  // the unit's first block writes step t-1's output and eviction
  // step t-1's output (the unit's first block): each partial's column of the numerator
  float po[NS];
  if (lead) {
    const int col = tid < D ? (2 + tid) * 4 : kPastEnd;  // other threads read 0
#pragma unroll
    for (int q = 0; q < NS; ++q) po[q] = ld_f32(r_pu, col + q * (2 + D) * 4);
  }
  // every thread holds the 16 bytes of token t-1's rows at its lane's row offset
  const uint4 knew = ld16(static_cast<const T*>(p.knew) + static_cast<size_t>(unit) * D + part * EPL);
  const uint4 vnew = ld16(static_cast<const T*>(p.vnew) + static_cast<size_t>(unit) * D + part * EPL);
  const float x_new = lg[p.k];
  unsigned char* s_k = s_stage;
  unsigned char* s_v = s_stage + KB;
  asm volatile("" ::: "memory");  // the metadata loads go out before the slices'
  if constexpr (STAGE) {
    const size_t row0 = static_cast<size_t>(unit) * b.k + s0;
    const uint32_t bytes = static_cast<uint32_t>(s1 - s0) * D * sizeof(T);  // <= KB (host-checked)
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(static_cast<T*>(b.kslots) + row0 * D, bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(static_cast<T*>(b.vslots) + row0 * D, bytes);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
#pragma unroll
    for (int c = 0; c < KB / (NT * 16); ++c) {  // bytes past the slices read as zero
      const int o = (c * NT + wave * kWave) * 16;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, s_k + o, 16, tid * 16, c * NT * 16, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, s_v + o, 16, tid * 16, c * NT * 16, 0, 0);
    }
  }
  // No result of the loads above is used before all of them are issued (the
  // compiler would otherwise start the merge, and wait for the partials,
  // between the slice loads).
  asm volatile("" : "+v"(pm), "+v"(pl)::"memory");
  // ---- step t-1's finish
  float Mg, Lg;
  const float ws = merge_weights(pm, pl, p.nsplit, Mg, Lg);
  const float invL = 1.f / Lg;
  if (lead && tid < D) p.out[static_cast<size_t>(unit) * D + tid] = merge_column(po, ws) / Lg;
  uint64_t best = kNoKey;
  int best_slot = -1;
  int32_t best_rank = 0;  // position rolling: the place of best_slot
  // Branch-free over each thread's slots (selects, no divergent branches): every
  // slot's updated score, one branch for the threads holding slots of this
  // block's slices, and the candidates' minimum key (the pattern bit only when
  // a pattern is set: the loop exists in both forms).
  const auto finish_slots = [&](auto with_pattern) {
    for (int base = 0; base < cnt; base += NP * NT) {
      if (base > 0) fetch(base);
      const int j0 = base + tid * NP;
      float sn[NP], cn[NP];
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        sn[i] = rs[i];
        cn[i] = rc[i];
        add_weight(fast_exp2(rx[i] - Mg) * invL, sn[i], cn[i], compensate);
      }
      if (j0 < s1 && j0 + NP > s0) {  // this block's slices carry their slots into the next buffer
#pragma unroll
        for (int i = 0; i < NP; ++i) {
          const int j = j0 + i;
          if (j >= s0 && j < s1) {  // s1 <= cnt + 1; slot cnt (the next free one) is written below
            if (j < cnt) {
              ny_score[uk + j] = sn[i];
              ny_comp[uk + j] = cn[i];
              ny_pos[uk + j] = rp[i];
            }
          }
        }
      }
      if (full) {
#pragma unroll
        for (int i = 0; i < NP; ++i) {
          const int j = j0 + i;
          uint64_t key = evict_key(sn[i], rp[i]);
          if constexpr (decltype(with_pattern)::value)
            key |= pattern_bit(p.pat_kind, p.pat_period, p.pat_width, rp[i], p.new_pos);
          key = j < cnt && rp[i] <= p.cand_limit ? key : kNoKey;
          best_slot = key < best ? j : best_slot;
          if constexpr (ROPE) best_rank = key < best ? rr[i] : best_rank;
          best = key < best ? key : best;
        }
      }
    }
  };
  if (p.pat_kind == kPatternNone) finish_slots(std::false_type{});
  else finish_slots(std::true_type{});
  const float w_new = fast_exp2(x_new - Mg) * invL;
  int dst = cnt;  // cache not full: the new token takes the next free slot
  int32_t ev = -1;
  if (full) {
    if (p.new_is_candidate && tid == 0) {
      const uint64_t key =
          evict_key(w_new, p.new_pos) | pattern_bit(p.pat_kind, p.pat_period, p.pat_width, p.new_pos, p.new_pos);
      if (key < best) {
        best = key;
        best_slot = kNewSlot;
      }
    }
    const uint64_t wm = wave_min_key(best);
    if ((tid & (kWave - 1)) == 0) s_key[tid / kWave] = wm;
    lds_barrier();
    uint64_t bm = s_key[0];
#pragma unroll
    for (int w = 1; w < NT / kWave; ++w) bm = s_key[w] < bm ? s_key[w] : bm;
    ev = static_cast<int32_t>(static_cast<uint32_t>(bm & 0xffffffffu));
    if (best == bm) {  // keys are unique: exactly one owner
      s_slot = best_slot;
      if (ROPE) s_vrank = best_rank;
    }
    lds_barrier();
    dst = s_slot == kNewSlot ? -1 : s_slot;
  }
  if (lead && tid == 0 && p.evicted != nullptr) p.evicted[unit] = ev;
  if constexpr (ROPE) {
    // places after step t-1: not full, the new token is the latest entry (place
    // cnt); full, the entries after the victim move down one place and the new
    // token takes the last; the new token itself evicted, nothing moves
    const int rv = full && dst >= 0 ? s_vrank : 0;
    const auto moved = [&](int j, int32_t rk) {
      if (!full) return j == cnt ? cnt : rk;
      if (dst < 0) return rk;
      return j == dst ? p.k - 1 : (rk > rv ? rk - 1 : rk);
    };
    if constexpr (STAGE) {
      if (tid < nmine) {
        const int32_t rk = moved(s0 + tid, myrank);
        ny_rank[uk + s0 + tid] = rk;
        s_rank[tid] = rk;
      }
    } else {
      for (int j = s0 + tid; j < s1; j += NT) ny_rank[uk + j] = moved(j, static_cast<int32_t>(ld_u32(r_rk, j * 4)));
    }
  }
  const bool mine = dst >= s0 && dst < s1;  // token t-1 goes into a slot of this block's slices
  if (mine) {
    if (tid == 0) {
      ny_score[uk + dst] = w_new;
      ny_comp[uk + dst] = 0.f;
      ny_pos[uk + dst] = p.new_pos;
    }
    if (tid < LPR) {
      const size_t row = (static_cast<size_t>(unit) * p.k + dst) * D + tid * EPL;
      st16(static_cast<T*>(p.kslots) + row, knew);
      st16(static_cast<T*>(p.vslots) + row, vnew);
    }
  }
  if constexpr (STAGE) {
    if (which < 3) s_tok[which][part] = tok;
    // the slices have landed in shared memory (each wave waits for its own loads)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();
    const int gi = tid / NTP, gt = tid % NTP;  // slice of this thread group, thread within it
    const int split = split0 + gi;
    if (gi >= SPB || split >= b.nsplit) return;
    const int g0 = split * b.split_len;  // the group's first slot
    if (mine && dst >= g0 && dst < g0 + b.split_len && gt / LPR == (dst - g0) % NGP) {
      // the row group that attends the victim's slot writes token t-1's rows
      // over it, each lane the 16 bytes it reads back
      const int o = ((dst - s0) * D + part * EPL) * static_cast<int>(sizeof(T));
      *reinterpret_cast<uint4*>(s_k + o) = knew;
      *reinterpret_cast<uint4*>(s_v + o) = vnew;
    }
    const T* tk = reinterpret_cast<const T*>(&s_tok[0][0]);
    const size_t gofs = static_cast<size_t>(g0 - s0) * D * sizeof(T);
    const UnitRefs<T> ur{reinterpret_cast<T*>(s_k + gofs), reinterpret_cast<T*>(s_v + gofs), nullptr, nullptr,
                         nullptr, tk, tk + D, tk + 2 * D, ROPE ? s_rank + (g0 - s0) : nullptr};
    decode_step<T, D, true, ROPE, NTP, UNP, true>(b, unit, split, ur, nullptr, sh[gi], gt);
  } else {
    // the slot rows and places written above are read below by this block: wait for them
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid >= NTP) return;
    decode_step<T, D, true, ROPE, NTP, UNP, false>(b, unit, split0, global_refs<T, D>(b, unit), nullptr, sh[0],
                                                   tid);
  }
}

// Several decode steps per launch, one unit per block, with the unit's state
// held in the block's shared memory for the whole launch: its K/V slot rows and
// per-slot score, compensation and position are read once at the start and
// written back once at the end, every step in between attends, scores, evicts
// and overwrites in shared memory, and the next step's q/k/v rows are fetched
// while the current step runs.  Each step is decode_step with the block shape
// the one-step launch would use, so the results are bit-identical to `steps`
// one-step launches; only where the state lives changes.  For caches on the
// single-block path whose state fits in a block's shared memory.
template <typename T, int D, int NT, int UN>
__global__ __launch_bounds__(NT) void decode_resident(DecodeArgs a0, int steps, int64_t tok_bytes,
                                                      int64_t out_step) {
  constexpr int EPL = Layout<T, D, NT>::EPL, LPR = Layout<T, D, NT>::LPR;
  static_assert(3 * LPR <= NT, "one lane per 16 bytes of the next token's q/k/v rows");
  // [k + 1] logits | K rows | V rows | score | comp | pos | 2 x (q, k, v) rows,
  // each part 16-byte aligned (resident_dyn_bytes)
  extern __shared__ __align__(16) float s_dyn[];
  __shared__ StepShared<T, D, NT> sh;
  const int unit = blockIdx.x, k = a0.k, tid = threadIdx.x;
  const int k4 = (k + 3) & ~3;
  float* s_logit = s_dyn;
  T* sk = reinterpret_cast<T*>(s_dyn + k4 + 4);
  T* sv = sk + static_cast<size_t>(k) * D;
  float* ssc = reinterpret_cast<float*>(sv + static_cast<size_t>(k) * D);
  float* scp = ssc + k4;
  int32_t* sps = reinterpret_cast<int32_t*>(scp + k4);
  T* stok = reinterpret_cast<T*>(sps + k4);  // [2][3][D]: q, k, v of the current and the next step
  const UnitRefs<T> g = global_refs<T, D>(a0, unit);
  const int c0 = a0.count;
  for (int i = tid; i < c0 * (D / EPL); i += NT) {
    st16(sk + i * EPL, ld16(g.k + i * EPL));
    st16(sv + i * EPL, ld16(g.v + i * EPL));
  }
  for (int j = tid; j < c0; j += NT) {
    ssc[j] = g.sc[j];
    scp[j] = g.cp[j];
    sps[j] = g.ps[j];
  }
  // lanes 0..3*LPR-1 each move 16 bytes of the next token's q, k or v row
  const int which = tid / LPR, part = tid % LPR;
  const T* src = which == 0 ? g.qn : which == 1 ? g.kn : g.vn;
  if (which < 3) st16(stok + which * D + part * EPL, ld16(src + part * EPL));
  __syncthreads();
  DecodeArgs a = a0;
  for (int t = 0; t < steps; ++t) {
    const int cur = t & 1;
    uint4 nxt = make_uint4(0u, 0u, 0u, 0u);
    if (which < 3 && t + 1 < steps)
      nxt = ld16(reinterpret_cast<const char*>(src) + (t + 1) * tok_bytes + part * 16);
    a.out = a0.out + t * out_step;
    a.evicted = a0.evicted != nullptr ? a0.evicted + static_cast<size_t>(t) * gridDim.x : nullptr;
    a.count = min(k, c0 + t);
    a.split_len = max(a.count, 1);  // one block holds all of the unit's slots
    a.new_pos = a0.new_pos + t;
    a.cand_limit = a0.cand_limit + t;
    const T* tk = stok + cur * 3 * D;
    const UnitRefs<T> ur{sk, sv, ssc, scp, sps, tk, tk + D, tk + 2 * D, nullptr};
    decode_step<T, D, false, false, NT, UN, true>(a, unit, 0, ur, s_logit, sh, tid);
    if (which < 3 && t + 1 < steps) st16(stok + (cur ^ 1) * 3 * D + which * D + part * EPL, nxt);
    __syncthreads();  // this step's writes and the next token's rows before the next step
  }
  const int c1 = min(k, c0 + steps);
  for (int i = tid; i < c1 * (D / EPL); i += NT) {
    st16(g.k + i * EPL, ld16(sk + i * EPL));
    st16(g.v + i * EPL, ld16(sv + i * EPL));
  }
  for (int j = tid; j < c1; j += NT) {
    g.sc[j] = ssc[j];
    g.cp[j] = scp[j];
    g.ps[j] = sps[j];
  }
}

// Block shape of the one-step, single-block launch (launch_typed) for this cache.
struct Shape {
  int nt, un;
};
template <typename T, int D, bool ROPE>
Shape single_block_shape(int units, int k) {
  if constexpr (std::is_same<T, bf16_t>::value && D == 128 && !ROPE)
    if (units >= kFewUnits && k > kSmallK) return {kWaveThreads, kWaveUnroll};
  if (units < kFewUnits) return {kThreads, kUnrollFew};
  if (k <= kSmallK && units >= kSmallKUnits) return {kSmallThreads, kUnroll};
  return {kThreads, kUnroll};
}

// Dynamic shared memory of decode_resident: logits, K and V rows, score,
// compensation and position per slot, two sets of the new token's q/k/v rows.
template <typename T, int D>
size_t resident_dyn_bytes(int k) {
  const size_t k4 = static_cast<size_t>((k + 3) & ~3);
  return (k4 + 4) * 4 + 2 * static_cast<size_t>(k) * D * sizeof(T) + 3 * k4 * 4 + 6 * D * sizeof(T);
}

template <typename T, int D>
size_t resident_lds(int nt, int k) {
  const size_t fixed = nt == kThreads ? sizeof(StepShared<T, D, kThreads>) : sizeof(StepShared<T, D, kSmallThreads>);
  return resident_dyn_bytes<T, D>(k) + fixed;
}

constexpr size_t kResidentLdsMax = 64 * 1024;  // shared memory one block may use

template <typename T, int D>
bool resident_fits(int units, int k) {
  const Shape sh = single_block_shape<T, D, false>(units, k);
  return sh.nt != kWaveThreads && resident_lds<T, D>(sh.nt, k) <= kResidentLdsMax;
}

template <typename T, int D>
hipError_t launch_resident_typed(const DecodeArgs& a, int units, int steps, int64_t tok_bytes, int64_t out_step,
                                 hipStream_t s) {
  const Shape sh = single_block_shape<T, D, false>(units, a.k);
  const size_t dyn = resident_dyn_bytes<T, D>(a.k);
  if (sh.nt == kThreads && sh.un == kUnrollFew)
    hipLaunchKernelGGL((decode_resident<T, D, kThreads, kUnrollFew>), dim3(units), dim3(kThreads), dyn, s, a, steps,
                       tok_bytes, out_step);
  else if (sh.nt == kSmallThreads)
    hipLaunchKernelGGL((decode_resident<T, D, kSmallThreads, kUnroll>), dim3(units), dim3(kSmallThreads), dyn, s, a,
                       steps, tok_bytes, out_step);
  else if (sh.nt == kThreads)
    hipLaunchKernelGGL((decode_resident<T, D, kThreads, kUnroll>), dim3(units), dim3(kThreads), dyn, s, a, steps,
                       tok_bytes, out_step);
  else
    return hipErrorInvalidConfiguration;
  return hipGetLastError();
}

// Block shape of the split path's partial blocks for a slice length.
enum class SplitShape { kTwoWave, kWave, kBlock };
template <typename T, int D, bool ROPE>
SplitShape split_shape(int split_len) {
  if constexpr (std::is_same<T, bf16_t>::value && D == 128) {
    if (split_len <= kTwoWaveSplitLen) return SplitShape::kTwoWave;
    if (!ROPE && split_len <= kWaveSplitLen) return SplitShape::kWave;
  }
  return SplitShape::kBlock;
}

// The split path's partial launch (one block per slice).
template <typename T, int D, bool ROPE>
void launch_partials(const DecodeArgs& a, int units, hipStream_t s) {
  const dim3 grid(units * a.nsplit);
  const SplitShape sh = split_shape<T, D, ROPE>(a.split_len);
  if constexpr (std::is_same<T, bf16_t>::value && D == 128) {
    if (sh == SplitShape::kTwoWave) {
      hipLaunchKernelGGL((decode_kernel<T, D, true, ROPE, kTwoWaveThreads, kTwoWaveUnroll<ROPE>>), grid,
                         dim3(kTwoWaveThreads), 0, s, a);
      return;
    }
  }
  if constexpr (std::is_same<T, bf16_t>::value && D == 128 && !ROPE) {
    if (sh == SplitShape::kWave) {
      hipLaunchKernelGGL((decode_kernel<T, D, true, ROPE, kWaveThreads, kWaveUnroll>), grid, dim3(kWaveThreads), 0,
                         s, a);
      return;
    }
  }
  hipLaunchKernelGGL((decode_kernel<T, D, true, ROPE>), grid, dim3(kThreads), 0, s, a);
}

template <typename T, int D, bool ROPE>
hipError_t launch_typed(const DecodeArgs& a, int units, hipStream_t s) {
  if (a.nsplit == 1) {
    const size_t shm = static_cast<size_t>(a.k + 1) * sizeof(float);
    if constexpr (std::is_same<T, bf16_t>::value && D == 128) {
      if (units >= kFewUnits && a.k > kSmallK) {  // many units, larger budgets
        if constexpr (ROPE)  // two waves per unit, 4 slots in flight per row group (the turned queries' registers)
          hipLaunchKernelGGL((decode_kernel<T, D, false, ROPE, kTwoWaveThreads, kTwoWaveUnroll<ROPE>>), dim3(units),
                             dim3(kTwoWaveThreads), shm, s, a);
        else  // one wave per unit
          hipLaunchKernelGGL((decode_kernel<T, D, false, ROPE, kWaveThreads, kWaveUnroll>), dim3(units),
                             dim3(kWaveThreads), shm, s, a);
        return hipGetLastError();
      }
    }
    if (units < kFewUnits)  // few units: 4 slots in flight per row group
      hipLaunchKernelGGL((decode_kernel<T, D, false, ROPE, kThreads, kUnrollFew>), dim3(units), dim3(kThreads), shm,
                         s, a);
    else if (a.k <= kSmallK && units >= kSmallKUnits)  // small budgets: more units in flight per CU
      hipLaunchKernelGGL((decode_kernel<T, D, false, ROPE, kSmallThreads>), dim3(units), dim3(kSmallThreads), shm, s,
                         a);
    else
      hipLaunchKernelGGL((decode_kernel<T, D, false, ROPE>), dim3(units), dim3(kThreads), shm, s, a);
  } else {
    launch_partials<T, D, ROPE>(a, units, s);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_finish<T, D>), dim3(units), dim3(kFinishThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace

template <typename T, int D, bool ROPE>
hipError_t launch_split_typed(const DecodeArgs* p, const DecodeArgs& b, float* ny_score, float* ny_comp,
                              int32_t* ny_pos, int32_t* ny_rank, int units, hipStream_t s) {
  const dim3 grid(units * b.nsplit);
  const SplitShape sh = split_shape<T, D, ROPE>(b.split_len);
  if (p == nullptr) {  // the first step's slices alone
    launch_partials<T, D, ROPE>(b, units, s);
    return hipGetLastError();
  }
  if constexpr (std::is_same<T, bf16_t>::value && D == 128) {
    static_assert(kTwoWaveSplitLen * D * sizeof(T) <= kStageBytes, "a two-wave slice fits the stage");
    const bool stage = static_cast<size_t>(b.split_len) * D * sizeof(T) <= kStageBytes &&
                       p->nsplit <= kStagePartials;  // the slice fits the stage, the partials 32 registers
    constexpr int UN2 = kTwoWaveUnroll<ROPE>;
    if (sh == SplitShape::kTwoWave && stage) {
      if (b.nsplit % 4 == 0 && units * b.nsplit >= kQuadSlices) {  // four slices per block
        hipLaunchKernelGGL((decode_fused<T, D, kTwoWaveThreads, UN2, true, kStagePartials, 4, ROPE, kQuadThreads>),
                           dim3(units * b.nsplit / 4), dim3(kQuadThreads), 8 * kStageBytes, s, *p, b, ny_score,
                           ny_comp, ny_pos, ny_rank);
      } else if (b.nsplit % 2 == 0 && units * b.nsplit >= kPairedSlices) {  // two slices per block
        hipLaunchKernelGGL((decode_fused<T, D, kTwoWaveThreads, UN2, true, kStagePartials, 2, ROPE>),
                           dim3(units * b.nsplit / 2), dim3(kFusedThreads), 4 * kStageBytes, s, *p, b, ny_score,
                           ny_comp, ny_pos, ny_rank);
      } else {
        hipLaunchKernelGGL((decode_fused<T, D, kTwoWaveThreads, UN2, true, kStagePartials, 1, ROPE>), grid,
                           dim3(kFusedThreads), 2 * kStageBytes, s, *p, b, ny_score, ny_comp, ny_pos, ny_rank);
      }
    } else if (sh == SplitShape::kTwoWave) {
      hipLaunchKernelGGL((decode_fused<T, D, kTwoWaveThreads, UN2, false, kMaxSplitBlocks, 1, ROPE>), grid,
                         dim3(kFusedThreads), 0, s, *p, b, ny_score, ny_comp, ny_pos, ny_rank);
    } else if (sh == SplitShape::kWave) {
      if constexpr (!ROPE)
        hipLaunchKernelGGL((decode_fused<T, D, kWaveThreads, kWaveUnroll, false, kMaxSplitBlocks, 1, false>), grid,
                           dim3(kFusedThreads), 0, s, *p, b, ny_score, ny_comp, ny_pos, ny_rank);
    }
    if (sh != SplitShape::kBlock) return hipGetLastError();
  }
  if (ROPE && p->nsplit <= kStagePartials)  // position rolling: fewer partial registers leave room for the rotation
    hipLaunchKernelGGL((decode_fused<T, D, kThreads, kUnroll, false, kStagePartials, 1, ROPE>), grid,
                       dim3(kFusedThreads), 0, s, *p, b, ny_score, ny_comp, ny_pos, ny_rank);
  else
    hipLaunchKernelGGL((decode_fused<T, D, kThreads, kUnroll, false, kMaxSplitBlocks, 1, ROPE>), grid,
                       dim3(kFusedThreads), 0, s, *p, b, ny_score, ny_comp, ny_pos, ny_rank);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_split_any(const DecodeArgs* p, const DecodeArgs& b, float* ny_score, float* ny_comp,
                            int32_t* ny_pos, int32_t* ny_rank, int units, hipStream_t s) {
  if (b.rank != nullptr) return launch_split_typed<T, D, true>(p, b, ny_score, ny_comp, ny_pos, ny_rank, units, s);
  return launch_split_typed<T, D, false>(p, b, ny_score, ny_comp, ny_pos, ny_rank, units, s);
}

template <typename T, int D>
hipError_t launch_finish_typed(const DecodeArgs& a, int units, hipStream_t s) {
  hipLaunchKernelGGL((decode_finish<T, D>), dim3(units), dim3(kFinishThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_decode_split(int dtype, int head_dim, const DecodeArgs* prev, const DecodeArgs& cur,
                               float* ny_score, float* ny_comp, int32_t* ny_pos, int32_t* ny_rank, int units,
                               hipStream_t s) {
  const bool rope = cur.rank != nullptr;
  if (cur.fixed_new != nullptr || cur.nsplit < 2 ||
      (prev != nullptr && (prev->nsplit < 2 || prev->nsplit > kMaxSplitBlocks || (prev->rank != nullptr) != rope ||
                           (rope && ny_rank == nullptr))))
    return hipErrorInvalidConfiguration;
  if (dtype == 0)
    return head_dim == 64 ? launch_split_any<float, 64>(prev, cur, ny_score, ny_comp, ny_pos, ny_rank, units, s)
                          : launch_split_any<float, 128>(prev, cur, ny_score, ny_comp, ny_pos, ny_rank, units, s);
  return head_dim == 64 ? launch_split_any<bf16_t, 64>(prev, cur, ny_score, ny_comp, ny_pos, ny_rank, units, s)
                        : launch_split_any<bf16_t, 128>(prev, cur, ny_score, ny_comp, ny_pos, ny_rank, units, s);
}

hipError_t launch_decode_finish(int dtype, int head_dim, const DecodeArgs& a, int units, hipStream_t s) {
  if (dtype == 0)
    return head_dim == 64 ? launch_finish_typed<float, 64>(a, units, s) : launch_finish_typed<float, 128>(a, units, s);
  return head_dim == 64 ? launch_finish_typed<bf16_t, 64>(a, units, s) : launch_finish_typed<bf16_t, 128>(a, units, s);
}

bool decode_resident_fits(int dtype, int head_dim, int units, int k) {
  if (dtype == 0) return head_dim == 64 ? resident_fits<float, 64>(units, k) : resident_fits<float, 128>(units, k);
  return head_dim == 64 ? resident_fits<bf16_t, 64>(units, k) : resident_fits<bf16_t, 128>(units, k);
}

hipError_t launch_decode_resident(int dtype, int head_dim, const DecodeArgs& a, int units, int steps,
                                  int64_t tok_bytes, int64_t out_step, hipStream_t s) {
  if (!decode_resident_fits(dtype, head_dim, units, a.k) || a.rank != nullptr || a.fixed_new != nullptr ||
      a.nsplit != 1)
    return hipErrorInvalidConfiguration;
  if (dtype == 0)
    return head_dim == 64 ? launch_resident_typed<float, 64>(a, units, steps, tok_bytes, out_step, s)
                          : launch_resident_typed<float, 128>(a, units, steps, tok_bytes, out_step, s);
  return head_dim == 64 ? launch_resident_typed<bf16_t, 64>(a, units, steps, tok_bytes, out_step, s)
                        : launch_resident_typed<bf16_t, 128>(a, units, steps, tok_bytes, out_step, s);
}

hipError_t launch_decode(int dtype, int head_dim, const DecodeArgs& a, int units, hipStream_t s) {
  if (a.rank != nullptr) {
    if (dtype == 0)
      return head_dim == 64 ? launch_typed<float, 64, true>(a, units, s) : launch_typed<float, 128, true>(a, units, s);
    return head_dim == 64 ? launch_typed<bf16_t, 64, true>(a, units, s) : launch_typed<bf16_t, 128, true>(a, units, s);
  }
  if (dtype == 0) {
    return head_dim == 64 ? launch_typed<float, 64, false>(a, units, s) : launch_typed<float, 128, false>(a, units, s);
  }
  return head_dim == 64 ? launch_typed<bf16_t, 64, false>(a, units, s) : launch_typed<bf16_t, 128, false>(a, units, s);
}

}  // namespace h2o
