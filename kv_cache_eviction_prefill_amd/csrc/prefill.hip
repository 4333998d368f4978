// H2O prefill: score every prompt token by the attention it receives under the
// prompt's causal softmax, keep the heavy hitters plus the recent window, and
// fill the cache slots.
//
// Sources: "H2O: Heavy-Hitter Oracle for Efficient Generative Inference of Large
// Language Models -- 深度解读报告", §2.3 (heavy hitters found from the attention
// each token has received), §3.4 (prefill rule: a long prompt keeps K heavy
// hitters and the K most recent tokens; a short one keeps everything).
//
// Three launches per prefill:
//   1. rowstats:  per prompt row r, m_r = max_j x_rj and l_r = sum_j exp(x_rj - m_r)
//                 over j <= r (x = scale * q_r . k_j); bf16 inputs use MFMA
//                 32x32x16 tiles of S^T = K Q^T, so one lane holds one query's
//                 logits and the row reductions stay inside the lane.
//   2. colsum:    c_j = sum_{r >= j} exp(x_rj - m_r) / l_r, recomputing the
//                 logits as MFMA tiles of S = Q K^T (one lane per key column);
//                 the causal softmax is row-normalised, so the column sums need
//                 the row normalisers of pass 1 first.
//   3. select_fill: per unit, a radix select on the 64-bit key (score bits,
//                 position) finds the K_h-th best heavy-hitter candidate, a
//                 ballot/popcount compaction assigns slots in position order,
//                 and the kept K/V rows, positions and scores are written.
#include <cmath>

#include "h2o_device.h"
#include "launch.h"

namespace h2o {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 32;              // MFMA tile edge (rows and columns)
constexpr uint64_t kNoKey = ~0ull;

__device__ inline bf16x8 ld_bf16x8(const bf16_t* p) { return __builtin_bit_cast(bf16x8, ld16(p)); }

// Row m of a 32x32 MFMA accumulator tile held in element i of lane `lane`
// (the column is lane % 32).
__device__ inline int acc_row(int i, int lane) { return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3); }

// ------------------------------------------------------------------ bf16 MFMA passes
// Each of a block's 4 waves owns 64 rows (pass 1: queries, pass 2: keys) as two
// 32-row subtiles whose operands stay in registers; the other operand streams
// through LDS in 32-row tiles (double-buffered, rows padded by 16 bytes so the
// fragment reads of 32 consecutive rows spread over the banks), loaded
// cooperatively with 16-byte global loads.  A block handles the row blocks b
// and nblk-1-b of its unit, so every block does the same amount of causal work.
// The blocks of one unit are numbered so they land on the same XCD (blocks are
// dealt to the 8 XCDs round-robin) and walk the streamed tiles in the same order
// (pass 1 upwards from key 0, pass 2 downwards from the last query), so each
// tile is fetched once into that XCD's L2 and shared.
constexpr int kBlockRows = 256;
constexpr int kWaveRows = 64;
constexpr int kXcds = 8;

template <int D>
struct TileCfg {
  static constexpr int kLdw = D + 8;                     // LDS row stride (bf16 elements)
  static constexpr int kChunksPerRow = D * 2 / 16;       // 16-byte chunks per row
  static constexpr int kChunks = kTile * kChunksPerRow;  // per 32-row tile
  static constexpr int kPerThread = kChunks / kThreads;  // 2 (d = 128) or 1 (d = 64)
  static_assert(kChunks % kThreads == 0, "tile must split evenly over the block");
};

// (unit, row block) of this block; false for the padding blocks of the last group.
__device__ inline bool block_coords(int nblk, int units, int* unit, int* blk) {
  const int b = blockIdx.x;
  const int slot = b / kXcds;
  *unit = (slot / nblk) * kXcds + b % kXcds;
  *blk = slot % nblk;
  return *unit < units;
}

template <int D>
__device__ inline void tile_gload(const bf16_t* base, int row0, int L, uint4* pre) {
  using C = TileCfg<D>;
#pragma unroll
  for (int c = 0; c < C::kPerThread; ++c) {
    const int ch = threadIdx.x + kThreads * c;
    const int r = ch / C::kChunksPerRow, cc = ch % C::kChunksPerRow;
    const int row = row0 + r;
    pre[c] = row < L ? ld16(base + static_cast<size_t>(row) * D + cc * 8) : make_uint4(0u, 0u, 0u, 0u);
  }
}

template <int D>
__device__ inline void tile_lstore(bf16_t* tile, const uint4* pre) {
  using C = TileCfg<D>;
#pragma unroll
  for (int c = 0; c < C::kPerThread; ++c) {
    const int ch = threadIdx.x + kThreads * c;
    const int r = ch / C::kChunksPerRow, cc = ch % C::kChunksPerRow;
    st16(tile + r * C::kLdw + cc * 8, pre[c]);
  }
}

// Fragment of a 32-row LDS tile as an MFMA A operand (row = lane % 32).
template <int D>
__device__ inline void tile_frag(const bf16_t* tile, int lane, bf16x8* f) {
  const bf16_t* p = tile + (lane & 31) * TileCfg<D>::kLdw + (lane >> 5) * 8;
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) f[kk] = __builtin_bit_cast(bf16x8, ld16(p + 16 * kk));
}

// Row fragment straight from global memory (an operand that stays in registers).
template <int D>
__device__ inline void row_frag(const bf16_t* base, int row, int L, int lane, bf16x8* f) {
  const bf16_t* p = base + static_cast<size_t>(min(row, L - 1)) * D + (lane >> 5) * 8;
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) f[kk] = ld_bf16x8(p + 16 * kk);
}

// Pass 1: S^T = K Q^T per 32x32 tile, so a lane holds 16 logits of one query and
// the online row max / row sum stay inside the lane.  A block handles the row
// blocks blk and nblk-1-blk of its unit (equal work per block).
template <int D>
__global__ __launch_bounds__(kThreads) void rowstats_bf16(PrefillArgs a, int nblk, int units) {
  __shared__ __align__(16) bf16_t sK[2][kTile * TileCfg<D>::kLdw];
  const int npair = (nblk + 1) / 2;
  int unit, pb;
  if (!block_coords(npair, units, &unit, &pb)) return;
  const int L = a.L;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const bf16_t* Qu = static_cast<const bf16_t*>(a.q) + static_cast<size_t>(unit) * L * D;
  const bf16_t* Ku = static_cast<const bf16_t*>(a.k) + static_cast<size_t>(unit) * L * D;
  for (int h = 0; h < 2; ++h) {
    const int blk = h == 0 ? nblk - 1 - pb : pb;
    if (h == 1 && blk == nblk - 1 - pb) break;  // odd count: the middle block is alone
    const int qb = blk * kBlockRows;
    const int qw = qb + wave * kWaveRows;
    bf16x8 bq[2][D / 16];
#pragma unroll
    for (int s = 0; s < 2; ++s) row_frag<D>(Qu, qw + 32 * s + (lane & 31), L, lane, bq[s]);
    const int ntile = (min(qb + kBlockRows, L) - 1) / kTile + 1;
    float m[2] = {-1e30f, -1e30f}, l[2] = {0.f, 0.f};
    uint4 pre[TileCfg<D>::kPerThread];
    tile_gload<D>(Ku, 0, L, pre);
    tile_lstore<D>(sK[0], pre);
    __syncthreads();
    for (int t = 0; t < ntile; ++t) {
      const int k0 = t * kTile;
      if (t + 1 < ntile) tile_gload<D>(Ku, k0 + kTile, L, pre);
      if (qw < L && k0 <= qw + kWaveRows - 1) {
        bf16x8 ak[D / 16];
        tile_frag<D>(sK[t & 1], lane, ak);
        floatx16 acc[2];
        acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak[0], bq[0][0], floatx16{}, 0, 0, 0);
        acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak[0], bq[1][0], floatx16{}, 0, 0, 0);
#pragma unroll
        for (int kk = 1; kk < D / 16; ++kk) {
          acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak[kk], bq[0][kk], acc[0], 0, 0, 0);
          acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak[kk], bq[1][kk], acc[1], 0, 0, 0);
        }
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const int q = qw + 32 * s + (lane & 31);
          float v[16];
#pragma unroll
          for (int i = 0; i < 16; ++i) v[i] = acc[s][i];
          if (k0 + kTile - 1 > qw + 32 * s) {
            const int rel = q - k0 - 4 * (lane >> 5);
#pragma unroll
            for (int i = 0; i < 16; ++i) v[i] = (8 * (i >> 2) + (i & 3)) <= rel ? v[i] : -INFINITY;
          }
          float tm = fmaxf(v[0], v[1]);
#pragma unroll
          for (int i = 2; i < 16; i += 2) tm = fmaxf(tm, fmaxf(v[i], v[i + 1]));
          const float mn = fmaxf(m[s], tm);
          const float mc = mn * a.c2;
          float sum = 0.f;
#pragma unroll
          for (int i = 0; i < 16; ++i) sum += fast_exp2(fmaf(v[i], a.c2, -mc));
          l[s] = fmaf(l[s], fast_exp2((m[s] - mn) * a.c2), sum);
          m[s] = mn;
        }
      }
      if (t + 1 < ntile) tile_lstore<D>(sK[(t + 1) & 1], pre);
      __syncthreads();
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const float m2 = __shfl_xor(m[s], 32, kWave), l2 = __shfl_xor(l[s], 32, kWave);
      const float mn = fmaxf(m[s], m2);
      const float lt = l[s] * fast_exp2((m[s] - mn) * a.c2) + l2 * fast_exp2((m2 - mn) * a.c2);
      const int q = qw + 32 * s + lane;
      if (lane < 32 && q < L) {
        const size_t o = static_cast<size_t>(unit) * a.Lpad + q;
        a.row_max[o] = mn * a.scale;
        a.row_sum[o] = lt;
        a.row_lse2[o] = fmaf(mn, a.c2, log2f(lt));
      }
    }
  }
}

// Pass 2: S = Q K^T per 32x32 tile, so a lane holds 16 rows of one key column;
// c_j accumulates exp2(S c2 - lse2_r) over the rows r >= j.  Query tiles are
// walked from the last one down, so the blocks of a unit read the same tiles at
// the same time (L2 reuse).  A block handles key blocks blk and nblk-1-blk.
template <int D>
__global__ __launch_bounds__(kThreads) void colsum_bf16(PrefillArgs a, int nblk, int units) {
  __shared__ __align__(16) bf16_t sQ[2][kTile * TileCfg<D>::kLdw];
  __shared__ __align__(16) float sL[2][kTile];
  const int npair = (nblk + 1) / 2;
  int unit, pb;
  if (!block_coords(npair, units, &unit, &pb)) return;
  const int L = a.L;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const bf16_t* Qu = static_cast<const bf16_t*>(a.q) + static_cast<size_t>(unit) * L * D;
  const bf16_t* Ku = static_cast<const bf16_t*>(a.k) + static_cast<size_t>(unit) * L * D;
  const float* lse = a.row_lse2 + static_cast<size_t>(unit) * a.Lpad;
  for (int h = 0; h < 2; ++h) {
    const int blk = h == 0 ? pb : nblk - 1 - pb;
    if (h == 1 && blk == pb) break;
    const int kb = blk * kBlockRows;
    const int kw = kb + wave * kWaveRows;
    bf16x8 bk[2][D / 16];
#pragma unroll
    for (int s = 0; s < 2; ++s) row_frag<D>(Ku, kw + 32 * s + (lane & 31), L, lane, bk[s]);
    const int t0 = kb / kTile, tn = (L - 1) / kTile;
    float cs[2] = {0.f, 0.f};
    uint4 pre[TileCfg<D>::kPerThread];
    float lpre = 0.f;
    auto lse_load = [&](int row0) {
      if (threadIdx.x < kTile) lpre = row0 + static_cast<int>(threadIdx.x) < L ? lse[row0 + threadIdx.x] : 0.f;
    };
    tile_gload<D>(Qu, tn * kTile, L, pre);
    lse_load(tn * kTile);
    tile_lstore<D>(sQ[0], pre);
    if (threadIdx.x < kTile) sL[0][threadIdx.x] = lpre;
    __syncthreads();
    for (int t = tn; t >= t0; --t) {
      const int q0 = t * kTile;
      const int buf = (tn - t) & 1;
      if (t > t0) {
        tile_gload<D>(Qu, q0 - kTile, L, pre);
        lse_load(q0 - kTile);
      }
      if (kw < L && q0 + kTile - 1 >= kw) {
        bf16x8 aq[D / 16];
        tile_frag<D>(sQ[buf], lane, aq);
        floatx16 acc[2];
        acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq[0], bk[0][0], floatx16{}, 0, 0, 0);
        acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq[0], bk[1][0], floatx16{}, 0, 0, 0);
#pragma unroll
        for (int kk = 1; kk < D / 16; ++kk) {
          acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq[kk], bk[0][kk], acc[0], 0, 0, 0);
          acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq[kk], bk[1][kk], acc[1], 0, 0, 0);
        }
        float4 lv[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) lv[g] = *reinterpret_cast<const float4*>(&sL[buf][8 * g + 4 * (lane >> 5)]);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const int key = kw + 32 * s + (lane & 31);
          float p[16];
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float4& f = lv[i >> 2];
            const float ls = (i & 3) == 0 ? f.x : (i & 3) == 1 ? f.y : (i & 3) == 2 ? f.z : f.w;
            p[i] = fast_exp2(fmaf(acc[s][i], a.c2, -ls));
          }
          if (q0 < kw + 32 * s + 32 || q0 + kTile > L) {
            const int lo = key - q0 - 4 * (lane >> 5), hi = L - q0 - 4 * (lane >> 5);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int r = 8 * (i >> 2) + (i & 3);
              p[i] = (r >= lo && r < hi) ? p[i] : 0.f;
            }
          }
          float sum = 0.f;
#pragma unroll
          for (int i = 0; i < 16; ++i) sum += p[i];
          cs[s] += sum;
        }
      }
      if (t > t0) {
        tile_lstore<D>(sQ[buf ^ 1], pre);
        if (threadIdx.x < kTile) sL[buf ^ 1][threadIdx.x] = lpre;
      }
      __syncthreads();
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const float c = cs[s] + __shfl_xor(cs[s], 32, kWave);
      const int key = kw + 32 * s + lane;
      if (lane < 32 && key < L) a.col_sum[static_cast<size_t>(unit) * a.Lpad + key] = c;
    }
  }
}

// ------------------------------------------------------------------ fp32 (VALU) passes
template <int D>
__global__ __launch_bounds__(64) void rowstats_f32(PrefillArgs a) {
  const int nblk = (a.L + 63) / 64;
  const int unit = blockIdx.x / nblk;
  const int r = (blockIdx.x % nblk) * 64 + threadIdx.x;
  if (r >= a.L) return;
  const float* Qu = static_cast<const float*>(a.q) + static_cast<size_t>(unit) * a.L * D;
  const float* Ku = static_cast<const float*>(a.k) + static_cast<size_t>(unit) * a.L * D;
  float q[D];
#pragma unroll
  for (int e = 0; e < D; ++e) q[e] = Qu[static_cast<size_t>(r) * D + e];
  float m = -INFINITY, l = 0.f;
  for (int j = 0; j <= r; ++j) {
    float dot = 0.f;
#pragma unroll
    for (int e = 0; e < D; ++e) dot = fmaf(q[e], Ku[static_cast<size_t>(j) * D + e], dot);
    if (dot > m) {
      l = fmaf(l, fast_exp2((m - dot) * a.c2), 1.f);
      m = dot;
    } else {
      l += fast_exp2((dot - m) * a.c2);
    }
  }
  const size_t o = static_cast<size_t>(unit) * a.Lpad + r;
  a.row_max[o] = m * a.scale;
  a.row_sum[o] = l;
  a.row_lse2[o] = fmaf(m, a.c2, log2f(l));
}

template <int D>
__global__ __launch_bounds__(64) void colsum_f32(PrefillArgs a) {
  const int nblk = (a.L + 63) / 64;
  const int unit = blockIdx.x / nblk;
  const int j = (blockIdx.x % nblk) * 64 + threadIdx.x;
  if (j >= a.L) return;
  const float* Qu = static_cast<const float*>(a.q) + static_cast<size_t>(unit) * a.L * D;
  const float* Ku = static_cast<const float*>(a.k) + static_cast<size_t>(unit) * a.L * D;
  const float* lse = a.row_lse2 + static_cast<size_t>(unit) * a.Lpad;
  float kv[D];
#pragma unroll
  for (int e = 0; e < D; ++e) kv[e] = Ku[static_cast<size_t>(j) * D + e];
  float cs = 0.f;
  for (int r = j; r < a.L; ++r) {
    float dot = 0.f;
#pragma unroll
    for (int e = 0; e < D; ++e) dot = fmaf(Qu[static_cast<size_t>(r) * D + e], kv[e], dot);
    cs += fast_exp2(fmaf(dot, a.c2, -lse[r]));
  }
  a.col_sum[static_cast<size_t>(unit) * a.Lpad + j] = cs;
}

// ------------------------------------------------------------------ select + fill
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void select_fill(PrefillArgs a) {
  constexpr int EPL = Elem<T>::kPer16B;
  constexpr int LPR = D / EPL;
  constexpr int NG = kThreads / LPR;
  extern __shared__ int s_kept[];  // [kcap] kept positions in slot order
  __shared__ unsigned s_hist[256];
  __shared__ uint64_t s_prefix;
  __shared__ int s_need;
  __shared__ int s_wsum[kThreads / kWave];

  const int unit = blockIdx.x;
  const int tid = threadIdx.x;
  const int L = a.L, kc = a.kcap;
  const float* c = a.col_sum + static_cast<size_t>(unit) * a.Lpad;

  int nkept;
  if (L <= kc) {
    for (int j = tid; j < L; j += kThreads) s_kept[j] = j;
    nkept = L;
  } else {
    const int pool = L - a.recent;  // heavy-hitter candidates: [0, L - K_r)
    uint64_t thr = kNoKey;
    if (a.heavy > 0) {
      // MSB-first radix select of the heavy-th largest key among the pool
      uint64_t prefix = 0, mask = 0;
      int need = a.heavy;
      for (int shift = 56; shift >= 0; shift -= 8) {
        for (int t = tid; t < 256; t += kThreads) s_hist[t] = 0u;
        __syncthreads();
        for (int j = tid; j < pool; j += kThreads) {
          const uint64_t key = evict_key(c[j], j);
          if ((key & mask) == prefix) atomicAdd(&s_hist[(key >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (tid == 0) {
          int cum = 0, dsel = 0;
          for (int dd = 255; dd >= 0; --dd) {
            const int h = static_cast<int>(s_hist[dd]);
            if (cum + h >= need) {
              dsel = dd;
              break;
            }
            cum += h;
          }
          s_prefix = prefix | (static_cast<uint64_t>(dsel) << shift);
          s_need = need - cum;
        }
        __syncthreads();
        prefix = s_prefix;
        need = s_need;
        mask |= static_cast<uint64_t>(255u) << shift;
        __syncthreads();
      }
      thr = prefix;  // exactly `heavy` pool keys are >= thr (keys are unique)
    }
    // compaction in position order: heavy hitters first, then the recent window
    int base_slot = 0;
    for (int j0 = 0; j0 < L; j0 += kThreads) {
      const int j = j0 + tid;
      bool f;
      if (j < pool) f = (a.heavy > 0) && (evict_key(c[j], j) >= thr);
      else f = (j < L);
      const uint64_t bal = __ballot(f);
      const int lane = tid & (kWave - 1);
      const int wpre = __popcll(bal & ((1ull << lane) - 1ull));
      if (lane == 0) s_wsum[tid / kWave] = __popcll(bal);
      __syncthreads();
      int off = base_slot, tot = 0;
#pragma unroll
      for (int w = 0; w < kThreads / kWave; ++w) {
        if (w < tid / kWave) off += s_wsum[w];
        tot += s_wsum[w];
      }
      if (f && off + wpre < kc) s_kept[off + wpre] = j;
      __syncthreads();
      base_slot += tot;
    }
    nkept = min(base_slot, kc);
  }
  __syncthreads();

  float* sc = a.score + static_cast<size_t>(unit) * kc;
  float* cp = a.comp + static_cast<size_t>(unit) * kc;
  int32_t* ps = a.pos + static_cast<size_t>(unit) * kc;
  for (int s = tid; s < kc; s += kThreads) {
    if (s < nkept) {
      const int j = s_kept[s];
      ps[s] = j;
      sc[s] = c[j];
    } else {
      ps[s] = -1;
      sc[s] = 0.f;
    }
    cp[s] = 0.f;
  }
  const T* Ku = static_cast<const T*>(a.k) + static_cast<size_t>(unit) * L * D;
  const T* Vu = static_cast<const T*>(a.v) + static_cast<size_t>(unit) * L * D;
  T* kd = static_cast<T*>(a.kslots) + static_cast<size_t>(unit) * kc * D;
  T* vd = static_cast<T*>(a.vslots) + static_cast<size_t>(unit) * kc * D;
  const int g = tid / LPR, r = tid % LPR;
  for (int s = g; s < nkept; s += NG) {
    const int j = s_kept[s];
    st16(kd + static_cast<size_t>(s) * D + r * EPL, ld16(Ku + static_cast<size_t>(j) * D + r * EPL));
    st16(vd + static_cast<size_t>(s) * D + r * EPL, ld16(Vu + static_cast<size_t>(j) * D + r * EPL));
  }
}

__global__ void clear_kernel(int32_t* pos, float* score, float* comp, size_t n) {
  for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * blockDim.x) {
    pos[i] = -1;
    score[i] = 0.f;
    comp[i] = 0.f;
  }
}

template <typename T, int D>
hipError_t launch_select(const PrefillArgs& a, int units, hipStream_t s) {
  hipLaunchKernelGGL((select_fill<T, D>), dim3(units), dim3(kThreads),
                     static_cast<size_t>(a.kcap) * sizeof(int), s, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_bf16(const PrefillArgs& a, int units, hipStream_t s) {
  const int nblk = (a.L + kBlockRows - 1) / kBlockRows;
  const int groups = (units + kXcds - 1) / kXcds;
  const dim3 grid(groups * kXcds * ((nblk + 1) / 2));
  hipLaunchKernelGGL((rowstats_bf16<D>), grid, dim3(kThreads), 0, s, a, nblk, units);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((colsum_bf16<D>), grid, dim3(kThreads), 0, s, a, nblk, units);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_select<bf16_t, D>(a, units, s);
}

template <int D>
hipError_t launch_f32(const PrefillArgs& a, int units, hipStream_t s) {
  const int nblk = (a.L + 63) / 64;
  hipLaunchKernelGGL((rowstats_f32<D>), dim3(units * nblk), dim3(64), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((colsum_f32<D>), dim3(units * nblk), dim3(64), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_select<float, D>(a, units, s);
}

}  // namespace

hipError_t launch_prefill(int dtype, int head_dim, const PrefillArgs& a, int units, hipStream_t s) {
  if (dtype == 0) return head_dim == 64 ? launch_f32<64>(a, units, s) : launch_f32<128>(a, units, s);
  return head_dim == 64 ? launch_bf16<64>(a, units, s) : launch_bf16<128>(a, units, s);
}

hipError_t launch_clear(int32_t* pos, float* score, float* comp, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int blocks = static_cast<int>(std::min<size_t>((n + 255) / 256, 4096));
  hipLaunchKernelGGL(clear_kernel, dim3(blocks), dim3(256), 0, s, pos, score, comp, n);
  return hipGetLastError();
}

}  // namespace h2o
