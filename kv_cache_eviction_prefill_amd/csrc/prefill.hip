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
//   1. rowstats:  per prompt row r, the base-2 log of its softmax normaliser,
//                 lse2_r = log2 sum_{j<=r} exp2(c2 q_r.k_j) with c2 = scale*log2(e);
//                 bf16 inputs use MFMA 32x32x16 tiles of S^T = K Q^T, so one lane
//                 holds one query's logits and the row sum stays inside the lane.
//   2. colsum:    c_j = sum_{r>=j} exp2(c2 q_r.k_j - lse2_r), recomputing the
//                 logits as MFMA tiles of S = Q K^T (one lane per key column);
//                 the causal softmax is row-normalised, so the column sums need
//                 the row normalisers of pass 1 first.
//      (rowout instead, when the caller asks for the prompt's own attention
//                 output o_r = sum_j a_rj v_j: the same normalisers and the output
//                 from one sweep over K and V)
//   3. select_fill: per unit, a radix select finds the K_h-th best heavy-hitter
//                 candidate under the (score, position) order - over the score
//                 bits that differ, then over positions only when the boundary
//                 score is tied - a ballot/popcount compaction assigns slots in
//                 position order, and the kept K/V rows, positions and scores
//                 are written.
//
// Cost model of the MFMA passes on gfx950 (measured): per 32x32 logit tile the
// MFMAs take 8 x 32 cycles, and the exponentials alone (one v_exp per logit, at
// half the VALU rate) take as long, so each logit gets exactly one fma, one exp
// and one add on the common path.  Overlap of the matrix cores with the VALU
// needs several waves per SIMD: registers are kept to 128 (4 waves per SIMD).
#include <cmath>
#include <type_traits>

#include "h2o_device.h"
#include "launch.h"

namespace h2o {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 32;  // MFMA tile edge (rows and columns)
constexpr uint64_t kNoKey = ~0ull;

__device__ inline bf16x8 ld_bf16x8(const bf16_t* p) { return __builtin_bit_cast(bf16x8, ld16(p)); }

// The lane's index within its wave, read afresh (the asm is not hoisted out of
// the branch that uses it).
__device__ inline int lane_id_here() {
  int id;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(id));
  return id;
}

// ------------------------------------------------------------------ bf16 MFMA passes
// Each of a block's 4 waves owns 64 rows (pass 1: queries, pass 2: keys) as two
// 32-row subtiles whose operand stays in registers.  The other operand streams
// through a ring of 32-row LDS tiles, loaded straight from global memory to LDS
// (buffer loads with the LDS flag: no registers, no LDS-store instructions):
// plain operands two tiles per barrier from a ring of four (the next two tiles
// load while these are used), split operands one tile per barrier from a ring
// of three, two tiles ahead.  A block handles
// the row blocks b and nblk-1-b of its unit, so every block does the same amount
// of causal work.  The blocks of one unit are numbered so they land on the same
// XCD (blocks are dealt to the 8 XCDs round-robin) and walk the streamed tiles in
// the same order (pass 1 upwards from key 0, pass 2 downwards from the last
// query), so each tile is fetched once into that XCD's L2 and shared.
constexpr int kXcds = 8;
constexpr int kBufs = 3;

// Operands of the score products.  Plain: the bf16 inputs, two 32-row subtiles
// per wave.  Split (position rolling): a rotated row is no longer a bf16 value,
// so it arrives as two bf16 rows hi = bf16(x), lo = bf16(x - hi) (x to about
// 2^-17 relative) and every logit takes three products hi.hi + hi.lo + lo.hi
// (lo.lo, below 2^-16 of each term, is left out); the wave keeps hi and lo of
// one 32-row subtile in the registers two subtiles take otherwise, and each
// streamed tile carries its hi rows, then its lo rows.
template <bool SPLIT>
struct Pass {
  static constexpr int NS = SPLIT ? 1 : 2;  // 32-row subtiles per wave
  static constexpr int NA = SPLIT ? 2 : 1;  // bf16 arrays per operand (hi, lo)
  static constexpr int kWaveRows = 32 * NS;
  static constexpr int kBlockRows = 4 * kWaveRows;
};

// Tiles per barrier and the LDS ring they stream through.  Plain operands: two
// tiles per barrier from a ring of four (one two-tile step computed while the
// next one loads), halving the barriers a row block waits at.  Split operands,
// whose tiles carry hi and lo rows (twice the bytes, 3 waves per SIMD): one tile
// per barrier from a ring of three, loaded two tiles ahead.
template <bool SPLIT>
struct Ring {
  static constexpr int kStep = SPLIT ? 1 : 2;
  static constexpr int kBufs = SPLIT ? 3 : 4;
};

template <int D>
struct Tile {
  static constexpr int kRowBytes = D * 2;
  static constexpr int kChunks = D / 8;                    // 16-byte chunks per row
  static constexpr int kBytes = kTile * kRowBytes;         // 8 KB (d = 128) or 4 KB
  static constexpr int kLoads = kBytes / (kThreads * 16);  // 16-byte loads per thread per tile
  static constexpr int kSwz = kChunks - 1;
  static_assert(kBytes % (kThreads * 16) == 0, "tile must split evenly over the block");
  static_assert(kBytes % 256 == 0, "tiles must keep 256-byte alignment");
};

// (unit, row-block pair) of this block; false for the padding blocks of the last group.
__device__ inline bool block_coords(int npair, int units, int* unit, int* pair) {
  const int b = blockIdx.x;
  const int slot = b / kXcds;
  *unit = (slot / npair) * kXcds + b % kXcds;
  *pair = slot % npair;
  return *unit < units;
}

template <int N>
__device__ inline void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier without the memory fence of __syncthreads (which would also
// wait for the tiles still in flight).  The tile loads into LDS are tracked with
// explicit vmcnt waits; LDS reads are drained first so a tile can be overwritten
// once every wave has passed the barrier.
__device__ inline void tile_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// LDS placement of a streamed tile: chunk c of tile row r sits at chunk
// c ^ (r & kSwz) of the LDS row, so the 32 rows of one fragment read fall in
// different banks.  Each wave-wide load fills 1 KB of consecutive LDS; a lane's
// source offset inside the tile is the same for every tile (tile_voff).
template <int D>
__device__ inline int tile_voff() {
  using T = Tile<D>;
  const int o = threadIdx.x * 16;  // load c adds c * kThreads * 16 bytes
  const int r = o / T::kRowBytes, p = (o % T::kRowBytes) / 16;
  return r * T::kRowBytes + ((p ^ (r & T::kSwz)) * 16);
}

// Rows row0..row0+31 of a [L, D] matrix into an LDS tile through a buffer
// descriptor over the matrix: rows past L read as zero.
__device__ inline void tile_async(__amdgpu_buffer_rsrc_t rs, int voff, int row0, unsigned char* tile,
                                  int row_bytes, int loads) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
#pragma unroll
  for (int c = 0; c < loads; ++c)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, tile + (c * kThreads + wave * kWave) * 16, 16, voff,
                                             row0 * row_bytes + c * kThreads * 16, 0, 0);
}

// The 32 row normalisers (128 bytes) of the query tile starting at row0, by
// lanes 0..7 of wave 0, whose tile offset `voff` is lane * 16.
__device__ inline void lse_async(__amdgpu_buffer_rsrc_t rl, int voff, int row0, unsigned char* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, dst, 16, voff, row0 * 4, 0, 0);
}

// LDS reads by byte address.  These do not alias any compiler-visible store, so
// the only ordering with the tile loads is the explicit vmcnt wait + barrier.
typedef __attribute__((address_space(3))) const unsigned char lds_u8;
typedef __attribute__((address_space(3))) const uint4 lds_u4;
typedef float f32x4 __attribute__((ext_vector_type(4)));
__device__ inline uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_u8*)p));
}
__device__ inline f32x4 lds_float4(uint32_t addr) {
  return __builtin_bit_cast(f32x4, *(lds_u4*)(static_cast<uintptr_t>(addr)));
}
__device__ inline bf16x8 lds_frag(uint32_t addr) {
  return __builtin_bit_cast(bf16x8, *(lds_u4*)(static_cast<uintptr_t>(addr)));
}

// Lane offset of its MFMA A-operand fragment inside a swizzled tile: row fr =
// lane % 32, k-chunk 2kk + lane/32, with the row's swizzle folded in for kk = 0.
// Tiles are 256-byte aligned and the swizzle only touches bits 4..7 of the
// offset, so the fragment of step kk is at (tile + xo) ^ 32kk.
template <int D>
__device__ inline uint32_t frag_offset(int lane) {
  using T = Tile<D>;
  const int fr = lane & 31;
  return fr * T::kRowBytes + (((((lane >> 5) ^ fr) & 1) << 4) | (((fr & T::kSwz) & ~1) << 4));
}
__device__ inline bf16x8 tile_frag_kk(uint32_t base, int kk) { return lds_frag(base ^ static_cast<uint32_t>(kk * 32)); }

// Row fragment straight from global memory (the operand that stays in registers).
template <int D>
__device__ inline void row_frag(const bf16_t* base, int row, int L, int lane, bf16x8* f) {
  const bf16_t* p = base + static_cast<size_t>(min(row, L - 1)) * D + (lane >> 5) * 8;
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) f[kk] = ld_bf16x8(p + 16 * kk);
}

// Wait here (once per row block) for the register operand, so the compiler leaves
// no wait for it inside the tile loop, where it would also wait for the tiles in
// flight.
template <int D, int NS>
__device__ inline void settle(bf16x8 (&f)[NS][D / 16]) {
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) asm volatile("" : "+v"(f[s][kk]));
}

// S tile pair (two 32-row subtiles of the register operand) against the LDS tile
// at `fb`: 2 x D/16 MFMAs, fragments read two steps ahead.
template <int D>
__device__ inline void tile_mfma(uint32_t fb, const bf16x8 (&b)[2][D / 16], floatx16 (&acc)[2]) {
  bf16x8 f2[2] = {tile_frag_kk(fb, 0), tile_frag_kk(fb, 1)};
  acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f2[0], b[0][0], floatx16{}, 0, 0, 0);
  acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f2[0], b[1][0], floatx16{}, 0, 0, 0);
  f2[0] = tile_frag_kk(fb, 2);
#pragma unroll
  for (int kk = 1; kk < D / 16; ++kk) {
    acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f2[kk & 1], b[0][kk], acc[0], 0, 0, 0);
    acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f2[kk & 1], b[1][kk], acc[1], 0, 0, 0);
    if (kk + 2 < D / 16) f2[kk & 1] = tile_frag_kk(fb, kk + 2);
  }
  __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // 2 LDS reads, then (2 MFMA, 1 LDS read)...
#pragma unroll
  for (int kk = 0; kk < D / 16 - 2; ++kk) {
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
}

// Split operands: the S tile of one 32-row subtile (register hi `bh`, lo `bl`)
// against the LDS tile whose hi rows are at `fb` and lo rows at `fbl`:
// hi.hi in one accumulator, hi.lo + lo.hi in another (3 x D/16 MFMAs).
template <int D>
__device__ inline floatx16 tile_mfma_split(uint32_t fb, uint32_t fbl, const bf16x8 (&bh)[D / 16],
                                           const bf16x8 (&bl)[D / 16]) {
  floatx16 a0 = {}, a1 = {};
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    const bf16x8 th = tile_frag_kk(fb, kk), tl = tile_frag_kk(fbl, kk);
    a0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(th, bh[kk], a0, 0, 0, 0);
    a1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(th, bl[kk], a1, 0, 0, 0);
    a1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tl, bh[kk], a1, 0, 0, 0);
  }
  return a0 + a1;
}

// exp2(v_i * c + b) for the 16 logits of a lane, and their sum as four
// interleaved partial sums (one fixed order, shared by every pass that needs it).
__device__ inline floatx16 exp2_16(const floatx16& v, float c, float b) {
  floatx16 p;
#pragma unroll
  for (int i = 0; i < 16; ++i) p[i] = fast_exp2(fmaf(v[i], c, b));
  return p;
}
__device__ inline float sum16(const floatx16& p) {
  float part[4] = {p[0], p[1], p[2], p[3]};
#pragma unroll
  for (int i = 4; i < 16; ++i) part[i & 3] += p[i];
  return (part[0] + part[1]) + (part[2] + part[3]);
}

// Running base-2 normaliser of one query row over one 32-key S^T tile.  Lanes l
// and l^32 hold the same query over different keys; they keep the same offset m,
// which moves only when a tile would push a term of either lane past 2^64 (the
// first tile always does), and each keeps its own partial sum l.  p receives the
// tile's terms exp2(c2 s - m) against the offset after the update; the return
// value is exp2(m_before - m_after), 1 where the offset did not move, and `moved`
// (wave-uniform) says whether any lane's did.  Any offset at or below the row
// maximum gives the same normaliser and no term can overflow, so the result
// equals the usual max-shifted sum.
// kTerms = false drops p (the pass without the output only needs the sums).
template <bool kTerms>
__device__ inline float row_update(const floatx16& s, float c2, int lane, float& m, float& l, floatx16& p,
                                   bool& moved) {
  float ts;
  if (kTerms) {
    p = exp2_16(s, c2, -m);
    ts = sum16(p);
  } else {
    ts = sum16(exp2_16(s, c2, -m));
  }
  float r = 1.f;
  const uint64_t need = __ballot(!(ts <= 0x1p64f));
  moved = need != 0;
  if (!moved) {  // wave-uniform: the common tile only adds its sum (l * 1 + ts, as below)
    l += ts;
    return r;
  }
  const uint32_t pair = static_cast<uint32_t>(need) | static_cast<uint32_t>(need >> 32);
  if ((pair >> (lane & 31)) & 1u) {
    float tm = fmaxf(s[0], s[1]);
#pragma unroll
    for (int i = 2; i < 16; i += 2) tm = fmaxf(tm, fmaxf(s[i], s[i + 1]));
    tm = fmaxf(tm, __shfl_xor(tm, 32, kWave));
    const float mn = fmaxf(m, tm * c2);
    if (kTerms) {
      p = exp2_16(s, c2, -mn);
      ts = sum16(p);
    } else {
      ts = sum16(exp2_16(s, c2, -mn));
    }
    r = fast_exp2(m - mn);
    m = mn;
  }
  l = fmaf(l, r, ts);
  return r;
}

// Pass 1: S^T = K Q^T per 32x32 tile, so a lane holds 16 logits of one query
// (element i is key row 8(i/4) + 4(lane/32) + i%4 of the tile).  The row sum is
// kept by row_update against a lazily moved offset: the common tile costs one
// fma, one exp and one add per logit.  The pass with the attention output runs
// the same per-query arithmetic, so both give the same normalisers bit for bit.
template <int D, bool SPLIT>
__global__ __launch_bounds__(kThreads, SPLIT ? 3 : 4) void rowstats_bf16(PrefillArgs a, int nblk, int units) {
  using T = Tile<D>;
  using P = Pass<SPLIT>;
  constexpr int NS = P::NS, NA = P::NA;
  constexpr int S = Ring<SPLIT>::kStep, R = Ring<SPLIT>::kBufs;
  __shared__ __align__(256) unsigned char sK[R][NA * T::kBytes];
  const int npair = (nblk + 1) / 2;
  int unit, pb;
  if (!block_coords(npair, units, &unit, &pb)) return;
  const int L = a.L;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
  const int fr = lane & 31;
  const size_t uoff = static_cast<size_t>(unit) * L * D;
  const bf16_t* Qu = static_cast<const bf16_t*>(a.q) + uoff;
  const bf16_t* Ku = static_cast<const bf16_t*>(a.k) + uoff;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(Ku, static_cast<uint32_t>(L) * T::kRowBytes);
  // split operands: the lo rows of q and k (unused otherwise)
  const bf16_t* Ql = SPLIT ? static_cast<const bf16_t*>(a.q_lo) + uoff : Qu;
  const __amdgpu_buffer_rsrc_t rkl =
      SPLIT ? make_rsrc(static_cast<const bf16_t*>(a.k_lo) + uoff, static_cast<uint32_t>(L) * T::kRowBytes) : rk;
  const int voff = tile_voff<D>();
  const uint32_t xo = frag_offset<D>(lane);
  for (int h = 0; h < 2; ++h) {
    const int blk = h == 0 ? nblk - 1 - pb : pb;
    if (h == 1 && blk == nblk - 1 - pb) break;  // odd count: the middle block is alone
    const int qb = blk * P::kBlockRows;
    const int qw = qb + wave * P::kWaveRows;
    const int ntile = (min(qb + P::kBlockRows, L) - 1) / kTile + 1;
    if (h == 1) tile_barrier();  // the first row block's tiles are no longer read
    bf16x8 bq[NS][D / 16], bql[NS][D / 16];
#pragma unroll
    for (int s = 0; s < NS; ++s) row_frag<D>(Qu, qw + 32 * s + fr, L, lane, bq[s]);
    if constexpr (SPLIT) row_frag<D>(Ql, qw + fr, L, lane, bql[0]);
    // the key rows t*32.. (hi, then lo when split) into buffer `buf`
    auto issue = [&](int t, int buf) {
      tile_async(rk, voff, t * kTile, sK[buf], T::kRowBytes, T::kLoads);
      if constexpr (SPLIT) tile_async(rkl, voff, t * kTile, sK[buf] + T::kBytes, T::kRowBytes, T::kLoads);
    };
    issue(0, 0);
    if (ntile > 1) issue(1, 1);
    settle<D, NS>(bq);
    if constexpr (SPLIT) settle<D, NS>(bql);
    float m[NS], l[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      m[s] = -1e30f;
      l[s] = 0.f;
    }
    for (int t0 = 0; t0 < ntile; t0 += S) {
      // this step's tiles landed (one tile per step: the next may be in flight)
      if (S == 1 && t0 + 1 < ntile) wait_vm<NA * T::kLoads>();
      else wait_vm<0>();
      tile_barrier();
      if constexpr (S == 1) {
        if (t0 + 2 < ntile) issue(t0 + 2, (t0 + 2) % R);
      } else {
#pragma unroll
        for (int u = 0; u < S; ++u)
          if (t0 + S + u < ntile) issue(t0 + S + u, (t0 + S + u) % R);
      }
#pragma unroll
      for (int u = 0; u < S; ++u) {
        const int t = t0 + u;
        const int k0 = t * kTile;
        if (t < ntile && qw < L && k0 <= qw + P::kWaveRows - 1) {
          uint32_t fb = lds_addr(sK[t % R]) + xo;
          asm volatile("" : "+v"(fb));  // keep the per-step offsets inside the loop
          floatx16 acc[NS];
          if constexpr (SPLIT) acc[0] = tile_mfma_split<D>(fb, fb + T::kBytes, bq[0], bql[0]);
          else tile_mfma<D>(fb, bq, acc);
#pragma unroll
          for (int s = 0; s < NS; ++s) {
            if (k0 + kTile - 1 > qw + 32 * s) {  // diagonal tile: keys after the query leave the row
              const int ln = lane_id_here();  // re-read here: keeping it live across the loop spills
              const int rel = qw + 32 * s + (ln & 31) - k0 - 4 * (ln >> 5);
#pragma unroll
              for (int i = 0; i < 16; ++i) acc[s][i] = (8 * (i >> 2) + (i & 3)) <= rel ? acc[s][i] : -INFINITY;
            }
            floatx16 p;
            bool moved;
            row_update<false>(acc[s], a.c2, lane, m[s], l[s], p, moved);
          }
        }
      }
    }
    // lanes l and l+32 hold the same queries over different key rows
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const float lt = l[s] + __shfl_xor(l[s], 32, kWave);
      const int q = qw + 32 * s + lane;
      // rows L..Lpad-1 get 0 so pass 2 reads finite normalisers for its masked rows
      if (lane < 32 && q < a.Lpad)
        a.row_lse2[static_cast<size_t>(unit) * a.Lpad + q] = q < L ? m[s] + log2f(lt) : 0.f;
    }
  }
}

// Pass 2: S = Q K^T per 32x32 tile, so a lane holds 16 query rows of one key
// column; c_j accumulates exp2(S c2 - lse2_r) over the rows r >= j.  Query tiles
// are walked from the last one down.  Each tile buffer carries the tile's 32 row
// normalisers after its rows (brought by lanes 0..7 of wave 0).
template <int D, bool SPLIT>
__global__ __launch_bounds__(kThreads, SPLIT ? 3 : 4) void colsum_bf16(PrefillArgs a, int nblk, int units) {
  using T = Tile<D>;
  using P = Pass<SPLIT>;
  constexpr int NS = P::NS, NA = P::NA;
  constexpr int kBufBytes = NA * T::kBytes + 256;  // tile rows, normalisers, padding to 256 bytes
  constexpr int S = Ring<SPLIT>::kStep, R = Ring<SPLIT>::kBufs;
  __shared__ __align__(256) unsigned char sQ[R][kBufBytes];
  const int npair = (nblk + 1) / 2;
  int unit, pb;
  if (!block_coords(npair, units, &unit, &pb)) return;
  const int L = a.L;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
  const int fr = lane & 31;
  const size_t uoff = static_cast<size_t>(unit) * L * D;
  const bf16_t* Qu = static_cast<const bf16_t*>(a.q) + uoff;
  const bf16_t* Ku = static_cast<const bf16_t*>(a.k) + uoff;
  const float* lse = a.row_lse2 + static_cast<size_t>(unit) * a.Lpad;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(Qu, static_cast<uint32_t>(L) * T::kRowBytes);
  const __amdgpu_buffer_rsrc_t rl = make_rsrc(lse, static_cast<uint32_t>(a.Lpad) * 4);
  // split operands: the lo rows of q and k (unused otherwise)
  const bf16_t* Kl = SPLIT ? static_cast<const bf16_t*>(a.k_lo) + uoff : Ku;
  const __amdgpu_buffer_rsrc_t rql =
      SPLIT ? make_rsrc(static_cast<const bf16_t*>(a.q_lo) + uoff, static_cast<uint32_t>(L) * T::kRowBytes) : rq;
  const int voff = tile_voff<D>();  // for lanes 0..7 of wave 0 this is lane * 16
  const uint32_t xo = frag_offset<D>(lane);
  const bool lse_lane = wave == 0 && lane < 8;
  for (int h = 0; h < 2; ++h) {
    const int blk = h == 0 ? pb : nblk - 1 - pb;
    if (h == 1 && blk == pb) break;
    const int kb = blk * P::kBlockRows;
    const int kw = kb + wave * P::kWaveRows;
    const int t0 = kb / kTile, tn = (L - 1) / kTile;
    if (h == 1) tile_barrier();
    bf16x8 bk[NS][D / 16], bkl[NS][D / 16];
#pragma unroll
    for (int s = 0; s < NS; ++s) row_frag<D>(Ku, kw + 32 * s + fr, L, lane, bk[s]);
    if constexpr (SPLIT) row_frag<D>(Kl, kw + fr, L, lane, bkl[0]);
    // the query rows t*32.. (hi, then lo when split) and their normalisers into buffer `buf`
    auto issue = [&](int t, int buf) {
      tile_async(rq, voff, t * kTile, sQ[buf], T::kRowBytes, T::kLoads);
      if constexpr (SPLIT) tile_async(rql, voff, t * kTile, sQ[buf] + T::kBytes, T::kRowBytes, T::kLoads);
      if (lse_lane) lse_async(rl, voff, t * kTile, sQ[buf] + NA * T::kBytes);
    };
    issue(tn, 0);
    if (tn > t0) issue(tn - 1, 1);
    settle<D, NS>(bk);
    if constexpr (SPLIT) settle<D, NS>(bkl);
    float cs[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) cs[s] = 0.f;
    // tile t is the it-th of the walk (it = tn - t) and sits in buffer it % R
    for (int i0 = 0; i0 <= tn - t0; i0 += S) {
      // this step's tiles landed (one tile per step: the next may be in flight)
      if (S > 1 || tn - i0 == t0) wait_vm<0>();
      else if (wave == 0) wait_vm<NA * T::kLoads + 1>();  // wave 0 also brings the normalisers
      else wait_vm<NA * T::kLoads>();
      tile_barrier();
      if constexpr (S == 1) {
        if (tn - i0 - 2 >= t0) issue(tn - i0 - 2, (i0 + 2) % R);
      } else {
#pragma unroll
        for (int u = 0; u < S; ++u)
          if (tn - (i0 + S + u) >= t0) issue(tn - (i0 + S + u), (i0 + S + u) % R);
      }
#pragma unroll
      for (int u = 0; u < S; ++u) {
        const int it = i0 + u, t = tn - it;
        const int q0 = t * kTile;
        if (t >= t0 && kw < L && q0 + kTile - 1 >= kw) {
          const uint32_t tile = lds_addr(sQ[it % R]);
          uint32_t fb = tile + xo;
          asm volatile("" : "+v"(fb));
          floatx16 acc[NS];
          if constexpr (SPLIT) acc[0] = tile_mfma_split<D>(fb, fb + T::kBytes, bk[0], bkl[0]);
          else tile_mfma<D>(fb, bk, acc);
          if (q0 < kw + P::kWaveRows || q0 + kTile > L) {  // diagonal or ragged last tile
            // rows above the key and rows past L leave the column: logit -> -inf
            const int h4 = 4 * (lane >> 5);
#pragma unroll
            for (int s = 0; s < NS; ++s) {
              const int lo = kw + 32 * s + fr - q0 - h4, hi = L - q0 - h4;
#pragma unroll
              for (int i = 0; i < 16; ++i) {
                const int r = 8 * (i >> 2) + (i & 3);
                acc[s][i] = (r >= lo && r < hi) ? acc[s][i] : -INFINITY;
              }
            }
          }
          // the 16 rows of this lane sit in 4 runs of 4 consecutive rows: one float4
          // of normalisers per run
          const uint32_t lrow = tile + NA * T::kBytes + 16 * (lane >> 5);
#pragma unroll
          for (int s = 0; s < NS; ++s) {
            float part[4];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const f32x4 f = lds_float4(lrow + 32 * g);
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const float p = fast_exp2(fmaf(acc[s][4 * g + j], a.c2, -f[j]));
                part[j] = g == 0 ? p : part[j] + p;
              }
            }
            cs[s] += (part[0] + part[1]) + (part[2] + part[3]);
          }
        }
      }
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const float c = cs[s] + __shfl_xor(cs[s], 32, kWave);
      const int key = kw + 32 * s + lane;
      if (lane < 32 && key < L) a.col_sum[static_cast<size_t>(unit) * a.Lpad + key] = c;
    }
  }
}

// ------------------------------------------------------------------ prompt attention output
// Pass 1 with the prompt's own attention output, run instead of pass 1 when the
// caller asks for o_r = sum_{j<=r} a_rj v_j: one sweep over the keys gives both
// the row normaliser and the output (the FlashAttention order).  Each of a
// block's 4 waves keeps 32 query rows in registers; K and V tiles stream through
// two rings of three swizzled LDS tiles (global -> LDS loads).  S^T = K Q^T per
// tile gives each lane one query's logits for 16 keys; row_update turns them
// into terms exp2(c2 s - m) against the running offset, and, rounded to bf16,
// those terms are the B operand of O^T += V^T P^T.  When the offset moves, O is
// rescaled with it; at the end O is divided by the row sum.  The V^T operand
// comes from the transposing LDS read: in each group of 16 lanes, output lane
// 4a+b takes element b of the 8-byte reads of lanes a, a+4, a+8, a+12, so
// pointing those lanes at 4 consecutive d values of 4 different key rows hands
// every lane 4 keys of one d column - in the key order of the S^T accumulator
// (element i of lane l is key 8(i/4) + 4(l/32) + i%4).
constexpr int kOutRows = 128;  // 4 waves x 32 query rows

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
__device__ inline i16x4 lds_tr16(uint32_t addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(static_cast<uintptr_t>(addr)));
}

// V tiles have a placement of their own: chunk c of tile row r sits at chunk
// c ^ v_swz(r).  A transposing read takes, per half-wave, 4 consecutive key
// rows (r = 4j .. 4j+3) times 4 chunks of one 64-byte column block; v_swz sends
// those 4 rows to 4 different 64-byte quarters of the 256 bytes the LDS banks
// serve per cycle (d = 128: a row spans all 256 bytes, the quarter is bits 2-3
// of the chunk; d = 64: a row spans half of them, the quarter is the row's
// parity and bit 2 of the chunk), and the 4 chunks of a row fill its quarter,
// so the read is free of bank conflicts.  The placement repeats every 16 rows,
// so one source offset per lane serves every load of a tile.
template <int D>
__device__ inline int v_swz(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

template <int D>
__device__ inline int tile_voff_v() {
  using T = Tile<D>;
  const int o = threadIdx.x * 16;
  const int r = o / T::kRowBytes, p = (o % T::kRowBytes) / 16;
  return r * T::kRowBytes + ((p ^ v_swz<D>(r)) * 16);
}

// Byte offset, inside a V tile, of 16-bit element `col` of tile row `key`.
template <int D>
__device__ inline uint32_t v_elem_offset(int key, int col) {
  using T = Tile<D>;
  const int byte = 2 * col;
  return key * T::kRowBytes + (((byte >> 4) ^ v_swz<D>(key)) << 4) + (byte & 15);
}

// The terms p >= 0 of a lane's 16 keys as two bf16 B operands each: hi = p with
// its low 16 mantissa bits cleared (a bf16 value), lo = bf16(p - hi) (p - hi is
// exact in fp32), so hi + lo is p to 2^-16 relative.  A single bf16 operand
// would carry 2^-9 of each term into the output (about 3e-3 absolute where a
// few keys hold the row's weight).
__device__ inline void split_terms(const floatx16& p, bf16x8 (&hi)[2], bf16x8 (&lo)[2]) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t hb = __float_as_uint(p[i]) & 0xffff0000u;
    hi[i >> 3][i & 7] = __builtin_bit_cast(__bf16, static_cast<uint16_t>(hb >> 16));
    lo[i >> 3][i & 7] = static_cast<__bf16>(p[i] - __uint_as_float(hb));
  }
}

template <int D, bool SPLIT>
__global__ __launch_bounds__(kThreads, SPLIT ? 2 : 3) void rowout_bf16(PrefillArgs a, int nblk, int units) {
  using T = Tile<D>;
  constexpr int NA = Pass<SPLIT>::NA;
  constexpr int NDB = D / 32;  // 32-wide column blocks of the output
  __shared__ __align__(256) unsigned char sK[kBufs][NA * T::kBytes];
  __shared__ __align__(256) unsigned char sV[kBufs][T::kBytes];
  const int npair = (nblk + 1) / 2;
  int unit, pb;
  if (!block_coords(npair, units, &unit, &pb)) return;
  const int L = a.L;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
  const int fr = lane & 31, hh = lane >> 5;
  const size_t uoff = static_cast<size_t>(unit) * L * D;
  const bf16_t* Qu = static_cast<const bf16_t*>(a.q) + uoff;
  const bf16_t* Ku = static_cast<const bf16_t*>(a.k) + uoff;
  const bf16_t* Vu = static_cast<const bf16_t*>(a.v) + uoff;
  float* out = a.out + uoff;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(Ku, static_cast<uint32_t>(L) * T::kRowBytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vu, static_cast<uint32_t>(L) * T::kRowBytes);
  // split operands: the lo rows of q and k (unused otherwise)
  const bf16_t* Ql = SPLIT ? static_cast<const bf16_t*>(a.q_lo) + uoff : Qu;
  const __amdgpu_buffer_rsrc_t rkl =
      SPLIT ? make_rsrc(static_cast<const bf16_t*>(a.k_lo) + uoff, static_cast<uint32_t>(L) * T::kRowBytes) : rk;
  const int voff = tile_voff<D>(), voffv = tile_voff_v<D>();
  const uint32_t xo = frag_offset<D>(lane);
  // this lane's role as a source of the transposing read: key row 4(g/2) + j
  // (+ 8 for the second read, + 16 for the second 16-key block), d columns
  // 16(g%2) + 4a .. +3 (+ 32 per column block), g = lane / 16, a = lane % 4,
  // j = (lane / 4) % 4
  const int tkey = 4 * (lane >> 5) + ((lane >> 2) & 3);
  const int tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  for (int h = 0; h < 2; ++h) {
    const int blk = h == 0 ? nblk - 1 - pb : pb;
    if (h == 1 && blk == nblk - 1 - pb) break;
    const int qw = blk * kOutRows + wave * 32;
    const int ntile = (min(blk * kOutRows + kOutRows, L) - 1) / kTile + 1;
    if (h == 1) tile_barrier();
    bf16x8 bq[1][D / 16], bql[1][D / 16];
    row_frag<D>(Qu, qw + fr, L, lane, bq[0]);
    if constexpr (SPLIT) row_frag<D>(Ql, qw + fr, L, lane, bql[0]);
    // K rows t*32.. (hi, then lo when split) and V rows t*32.. into buffer `buf`
    auto issue = [&](int t, int buf) {
      tile_async(rk, voff, t * kTile, sK[buf], T::kRowBytes, T::kLoads);
      if constexpr (SPLIT) tile_async(rkl, voff, t * kTile, sK[buf] + T::kBytes, T::kRowBytes, T::kLoads);
      tile_async(rv, voffv, t * kTile, sV[buf], T::kRowBytes, T::kLoads);
    };
    issue(0, 0);
    if (ntile > 1) issue(1, 1);
    settle<D, 1>(bq);
    if constexpr (SPLIT) settle<D, 1>(bql);
    floatx16 o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[db] = floatx16{};
    float m = -1e30f, l = 0.f;
    for (int t = 0; t < ntile; ++t) {
      if (t + 1 < ntile) wait_vm<(NA + 1) * T::kLoads>();  // K and V of this tile landed
      else wait_vm<0>();
      tile_barrier();
      if (t + 2 < ntile) issue(t + 2, (t + 2) % kBufs);
      const int k0 = t * kTile;
      if (qw < L && k0 <= qw + 31) {
        uint32_t fb = lds_addr(sK[t % kBufs]) + xo;
        asm volatile("" : "+v"(fb));
        floatx16 sacc;
        if constexpr (SPLIT) {
          sacc = tile_mfma_split<D>(fb, fb + T::kBytes, bq[0], bql[0]);
        } else {
          sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tile_frag_kk(fb, 0), bq[0][0], floatx16{}, 0, 0, 0);
#pragma unroll
          for (int kk = 1; kk < D / 16; ++kk)
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tile_frag_kk(fb, kk), bq[0][kk], sacc, 0, 0, 0);
        }
        if (k0 + kTile - 1 > qw) {  // diagonal tile: keys after the query get weight 0
          const int rel = qw + fr - k0 - 4 * hh;
#pragma unroll
          for (int i = 0; i < 16; ++i) sacc[i] = (8 * (i >> 2) + (i & 3)) <= rel ? sacc[i] : -INFINITY;
        }
        floatx16 p;
        bool moved;
        const float r = row_update<true>(sacc, a.c2, lane, m, l, p, moved);
        if (moved) {  // the lane's offset moved (r = 1 where it did not)
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[db][i] *= r;
        }
        bf16x8 pw[2], pl[2];  // terms of keys 16kb.. as B operands (hi, lo), kb = 0, 1
        split_terms(p, pw, pl);
        uint32_t vt = lds_addr(sV[t % kBufs]);
        asm volatile("" : "+v"(vt));
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            const i16x4 lo = lds_tr16(vt + v_elem_offset<D>(tkey + 16 * kb, tcol + 32 * db));
            const i16x4 hi = lds_tr16(vt + v_elem_offset<D>(tkey + 16 * kb + 8, tcol + 32 * db));
            const bf16x8 av = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pw[kb], o[db], 0, 0, 0);
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pl[kb], o[db], 0, 0, 0);
          }
        }
      }
    }
    // lanes l and l+32 hold the same query over different keys
    const float lt = l + __shfl_xor(l, 32, kWave);
    const int q = qw + lane;
    // rows L..Lpad-1 get 0 so pass 2 reads finite normalisers for its masked rows
    if (lane < 32 && q < a.Lpad) a.row_lse2[static_cast<size_t>(unit) * a.Lpad + q] = q < L ? m + log2f(lt) : 0.f;
    // o[db] element i of lane (fr, hh) is d = 32 db + 8(i/4) + 4 hh + i%4 of query qw + fr
    if (qw + fr < L) {
      const float inv = 1.f / lt;
      float* orow = out + static_cast<size_t>(qw + fr) * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<float4*>(orow + 32 * db + 8 * g + 4 * hh) =
              make_float4(o[db][4 * g] * inv, o[db][4 * g + 1] * inv, o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv);
    }
  }
}

// fp32 inputs: one thread per prompt row, VALU.
template <int D>
__global__ __launch_bounds__(64) void attnout_f32(PrefillArgs a) {
  const int nblk = (a.L + 63) / 64;
  const int unit = blockIdx.x / nblk;
  const int r = (blockIdx.x % nblk) * 64 + threadIdx.x;
  if (r >= a.L) return;
  const float* Qu = static_cast<const float*>(a.q) + static_cast<size_t>(unit) * a.L * D;
  const float* Ku = static_cast<const float*>(a.k) + static_cast<size_t>(unit) * a.L * D;
  const float* Vu = static_cast<const float*>(a.v) + static_cast<size_t>(unit) * a.L * D;
  const float lq = a.row_lse2[static_cast<size_t>(unit) * a.Lpad + r];
  float q[D], o[D];
#pragma unroll
  for (int e = 0; e < D; ++e) {
    q[e] = Qu[static_cast<size_t>(r) * D + e];
    o[e] = 0.f;
  }
  for (int j = 0; j <= r; ++j) {
    float dot = 0.f;
#pragma unroll
    for (int e = 0; e < D; ++e) dot = fmaf(q[e], Ku[static_cast<size_t>(j) * D + e], dot);
    const float p = fast_exp2(fmaf(dot, a.c2, -lq));
#pragma unroll
    for (int e = 0; e < D; ++e) o[e] = fmaf(p, Vu[static_cast<size_t>(j) * D + e], o[e]);
  }
  float* orow = a.out + (static_cast<size_t>(unit) * a.L + r) * D;
#pragma unroll
  for (int e = 0; e < D; ++e) orow[e] = o[e];
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
  a.row_lse2[static_cast<size_t>(unit) * a.Lpad + r] = fmaf(m, a.c2, log2f(l));
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
// Per unit (one block): when the prompt is longer than the budget, the K_h
// largest keys of the heavy-hitter pool [0, L - K_r) are found by a radix
// select and kept with the recent window, in position order; then the kept K/V
// rows, positions and scores are written into the slots.

// Selection key of prompt position j (score bits, position; the pattern bit on top).
template <bool PAT>
__device__ inline uint64_t key_of(const PrefillArgs& a, const float* c, int j, int L) {
  return PAT ? evict_key(c[j], j) | pattern_bit(a.pat_kind, a.pat_period, a.pat_width, j, L) : evict_key(c[j], j);
}

__device__ inline uint32_t wave_or_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v |= static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), o, kWave));
  return v;
}
__device__ inline uint32_t wave_and_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v &= static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), o, kWave));
  return v;
}

// The bin of a 256-bin histogram (one bin per thread of the 256-thread block)
// that holds the need-th largest element, counting from the top bin: on return
// *digit is that bin, *need the element's rank inside it and *cnt the bin's
// count (the same in every thread).  A block-wide scan of the counts from the top.
__device__ inline void pick_bin(const unsigned* hist, int need_in, int* digit, int* need, int* cnt,
                                uint32_t* s_red, int* s_pick) {
  static_assert(kThreads == 256, "one bin per thread");
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int b = 255 - tid;
  const uint32_t h = hist[b];
  uint32_t x = h;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const uint32_t y = static_cast<uint32_t>(__shfl_up(static_cast<int>(x), o, kWave));
    if (lane >= o) x += y;
  }
  if (lane == kWave - 1) s_red[wave] = x;
  __syncthreads();
  uint32_t base = 0u;
#pragma unroll
  for (int w = 0; w < kThreads / kWave; ++w) base += w < wave ? s_red[w] : 0u;
  const uint32_t incl = base + x, excl = incl - h;
  const uint32_t nd = static_cast<uint32_t>(need_in);
  if (excl < nd && nd <= incl) {
    s_pick[0] = b;
    s_pick[1] = static_cast<int>(nd - excl);
    s_pick[2] = static_cast<int>(h);
  }
  __syncthreads();
  *digit = s_pick[0];
  *need = s_pick[1];
  *cnt = s_pick[2];
  __syncthreads();  // s_red and s_pick are reused
}

// PAT: a sparse pattern is set (its bit joins the key; a template flag, so the
// plain rule pays nothing for it).
template <typename T, int D, bool PAT>
__global__ __launch_bounds__(kThreads) void select_fill(PrefillArgs a) {
  constexpr int EPL = Elem<T>::kPer16B;
  constexpr int LPR = D / EPL;
  constexpr int NG = kThreads / LPR;
  extern __shared__ int s_kept[];  // [kcap] kept positions in slot order
  __shared__ unsigned s_hist[256];
  __shared__ uint32_t s_red[2 * (kThreads / kWave)];
  __shared__ int s_pick[3];
  __shared__ int s_wsum[kThreads / kWave];

  const int unit = blockIdx.x;
  const int tid = threadIdx.x;
  const int L = a.L, kc = a.kcap;
  const float* c = a.scores_in != nullptr ? a.scores_in + static_cast<size_t>(unit) * a.scores_stride
                                          : a.col_sum + static_cast<size_t>(unit) * a.Lpad;

  int nkept;
  if (L <= kc) {
    for (int j = tid; j < L; j += kThreads) s_kept[j] = j;
    nkept = L;
  } else {
    const int pool = L - a.recent;  // heavy-hitter candidates: [0, L - K_r)
    uint64_t thr = kNoKey;
    if (a.heavy > 0) {
      // The heavy-th largest key of the pool, high word (score bits) first: the
      // bits every pool key shares are skipped, the rest is a radix select over
      // 8-bit digits from the top; the low word (position) is only needed when
      // the threshold score is tied across the boundary.
      const int wave = tid / kWave, lane = tid % kWave;
      uint32_t hor = 0u, hand = ~0u;
      for (int j = tid; j < pool; j += kThreads) {
        const uint32_t h = static_cast<uint32_t>(key_of<PAT>(a, c, j, L) >> 32);
        hor |= h;
        hand &= h;
      }
      hor = wave_or_u32(hor);
      hand = wave_and_u32(hand);
      if (lane == 0) {
        s_red[wave] = hor;
        s_red[kThreads / kWave + wave] = hand;
      }
      __syncthreads();
      hor = s_red[0];
      hand = s_red[kThreads / kWave];
#pragma unroll
      for (int w = 1; w < kThreads / kWave; ++w) {
        hor |= s_red[w];
        hand &= s_red[kThreads / kWave + w];
      }
      const uint32_t diff = hor ^ hand;
      int need = a.heavy;
      uint32_t H = hand;  // all pool keys share their high word when diff == 0
      int cnt_eq = pool;
      if (diff != 0u) {
        // bits above `top` are common (2u << 31 wraps to 0: then there are none)
        const int top = 31 - __clz(diff);
        uint32_t above = ~((2u << top) - 1u);
        uint32_t prefix = hand & above;
        for (int hi_bit = top; hi_bit >= 0; hi_bit -= 8) {
          const int lo_bit = max(hi_bit - 7, 0);
          const uint32_t wmask = (2u << (hi_bit - lo_bit)) - 1u;
          s_hist[tid] = 0u;
          __syncthreads();
          for (int j = tid; j < pool; j += kThreads) {
            const uint32_t h = static_cast<uint32_t>(key_of<PAT>(a, c, j, L) >> 32);
            if ((h & above) == prefix) atomicAdd(&s_hist[(h >> lo_bit) & wmask], 1u);
          }
          __syncthreads();
          int digit, cnt;
          pick_bin(s_hist, need, &digit, &need, &cnt, s_red, s_pick);
          prefix |= static_cast<uint32_t>(digit) << lo_bit;
          above |= wmask << lo_bit;
          cnt_eq = cnt;
        }
        H = prefix;
      }
      if (need == cnt_eq) {
        thr = static_cast<uint64_t>(H) << 32;  // every key with this high word is kept
      } else {
        // the need largest positions among the keys whose high word is H
        const int top = 31 - __clz(static_cast<uint32_t>(max(pool - 1, 1)));
        uint32_t prefix = 0u, above = ~((2u << top) - 1u);
        for (int hi_bit = top; hi_bit >= 0; hi_bit -= 8) {
          const int lo_bit = max(hi_bit - 7, 0);
          const uint32_t wmask = (2u << (hi_bit - lo_bit)) - 1u;
          s_hist[tid] = 0u;
          __syncthreads();
          for (int j = tid; j < pool; j += kThreads) {
            const uint32_t h = static_cast<uint32_t>(key_of<PAT>(a, c, j, L) >> 32);
            const uint32_t p = static_cast<uint32_t>(j);
            if (h == H && (p & above) == prefix) atomicAdd(&s_hist[(p >> lo_bit) & wmask], 1u);
          }
          __syncthreads();
          int digit, cnt;
          pick_bin(s_hist, need, &digit, &need, &cnt, s_red, s_pick);
          prefix |= static_cast<uint32_t>(digit) << lo_bit;
          above |= wmask << lo_bit;
        }
        thr = (static_cast<uint64_t>(H) << 32) | prefix;
      }
    }
    // compaction in position order: heavy hitters first, then the recent window
    int base_slot = 0;
    for (int j0 = 0; j0 < L; j0 += kThreads) {
      const int j = j0 + tid;
      bool f;
      if (j < pool)
        f = (a.heavy > 0) && key_of<PAT>(a, c, j, L) >= thr;
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

  float* sc = a.score + static_cast<size_t>(unit) * a.kstride;
  float* cp = a.comp + static_cast<size_t>(unit) * a.kstride;
  int32_t* ps = a.pos + static_cast<size_t>(unit) * a.kstride;
  int32_t* rk = a.rank != nullptr ? a.rank + static_cast<size_t>(unit) * a.kstride : nullptr;
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
    if (rk != nullptr) rk[s] = s < nkept ? s : 0;  // slots are filled in position order
  }
  const T* Ku = static_cast<const T*>(a.kcache) + static_cast<size_t>(unit) * a.kv_rows * D;
  const T* Vu = static_cast<const T*>(a.v) + static_cast<size_t>(unit) * a.kv_rows * D;
  T* kd = static_cast<T*>(a.kslots) + static_cast<size_t>(unit) * kc * D;
  T* vd = static_cast<T*>(a.vslots) + static_cast<size_t>(unit) * kc * D;
  // the kept rows: each row group moves kGather rows of K and V per round, all
  // loads issued before the first store
  constexpr int kGather = 4;
  const int g = tid / LPR, r = tid % LPR;
  for (int s0 = g; s0 < nkept; s0 += NG * kGather) {
    uint4 kr[kGather], vr[kGather];
#pragma unroll
    for (int u = 0; u < kGather; ++u) {
      const int s = min(s0 + u * NG, nkept - 1);
      const int j = s_kept[s];
      kr[u] = ld16_stream(Ku + static_cast<size_t>(j) * D + r * EPL);
      vr[u] = ld16_stream(Vu + static_cast<size_t>(j) * D + r * EPL);
    }
#pragma unroll
    for (int u = 0; u < kGather; ++u) {
      const int s = s0 + u * NG;
      if (s < nkept) {
        st16(kd + static_cast<size_t>(s) * D + r * EPL, kr[u]);
        st16(vd + static_cast<size_t>(s) * D + r * EPL, vr[u]);
      }
    }
  }
}

// ------------------------------------------------------------------ rotary embedding of the prompt
// One thread per (row, run of E pairs): the 16-byte chunk holding x_m .. x_{m+E-1}
// and the one holding x_{m+d/2} ..; each pair (x, y) becomes (x c - y s, x s + y c)
// in fp32, with (c, s) the table's entry for (r, m).  fp32 storage keeps the
// result; bf16 storage writes it as hi = bf16(v) into y and lo = bf16(v - hi)
// into y_lo (the score passes' split operands).
__device__ inline float to_f32(float x) { return x; }
__device__ inline float to_f32(bf16_t x) { return __uint_as_float(static_cast<uint32_t>(x.bits) << 16); }
__device__ inline bf16_t bf16_rne(float x) { return bf16_t{__builtin_bit_cast(uint16_t, static_cast<__bf16>(x))}; }

template <typename T, int D>
__global__ __launch_bounds__(256) void rope_prompt(const T* x, T* y, T* y_lo, int L, size_t runs, const float2* cs) {
  constexpr int H = D / 2, E = 16 / static_cast<int>(sizeof(T)), RPR = H / E;  // pairs per run, runs per row
  constexpr bool kSplit = !std::is_same<T, float>::value;
  const size_t t = blockIdx.x * static_cast<size_t>(256) + threadIdx.x;
  if (t >= runs) return;
  const size_t row = t / RPR;  // unit * L + r
  const int m0 = static_cast<int>(t % RPR) * E, r = static_cast<int>(row % L);
  union Chunk {
    uint4 u;
    T e[E];
  } a, b, oa, ob, la, lb;
  a.u = ld16(x + row * D + m0);
  b.u = ld16(x + row * D + m0 + H);
  const float2* w = cs + static_cast<size_t>(r) * H + m0;
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const float2 cw = w[i];
    const float xa = to_f32(a.e[i]), yb = to_f32(b.e[i]);
    const float va = __fsub_rn(__fmul_rn(xa, cw.x), __fmul_rn(yb, cw.y));
    const float vb = __fadd_rn(__fmul_rn(xa, cw.y), __fmul_rn(yb, cw.x));
    if constexpr (kSplit) {
      oa.e[i] = bf16_rne(va);
      ob.e[i] = bf16_rne(vb);
      la.e[i] = bf16_rne(va - to_f32(oa.e[i]));
      lb.e[i] = bf16_rne(vb - to_f32(ob.e[i]));
    } else {
      oa.e[i] = va;
      ob.e[i] = vb;
    }
  }
  st16(y + row * D + m0, oa.u);
  st16(y + row * D + m0 + H, ob.u);
  if constexpr (kSplit) {
    st16(y_lo + row * D + m0, la.u);
    st16(y_lo + row * D + m0 + H, lb.u);
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
  const size_t shm = static_cast<size_t>(a.kcap) * sizeof(int);
  if (a.pat_kind != kPatternNone)
    hipLaunchKernelGGL((select_fill<T, D, true>), dim3(units), dim3(kThreads), shm, s, a);
  else
    hipLaunchKernelGGL((select_fill<T, D, false>), dim3(units), dim3(kThreads), shm, s, a);
  return hipGetLastError();
}

template <int D, bool SPLIT>
hipError_t launch_bf16_scores(const PrefillArgs& a, int units, hipStream_t s) {
  const int nblk = (a.L + Pass<SPLIT>::kBlockRows - 1) / Pass<SPLIT>::kBlockRows;  // a block takes a pair
  const int groups = (units + kXcds - 1) / kXcds;
  const dim3 grid(groups * kXcds * ((nblk + 1) / 2));
  if (a.out != nullptr) {
    const int nbo = (a.L + kOutRows - 1) / kOutRows;
    const dim3 grid_o(groups * kXcds * ((nbo + 1) / 2));
    hipLaunchKernelGGL((rowout_bf16<D, SPLIT>), grid_o, dim3(kThreads), 0, s, a, nbo, units);
  } else {
    hipLaunchKernelGGL((rowstats_bf16<D, SPLIT>), grid, dim3(kThreads), 0, s, a, nblk, units);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((colsum_bf16<D, SPLIT>), grid, dim3(kThreads), 0, s, a, nblk, units);
  return hipGetLastError();
}

template <int D>
hipError_t launch_bf16(const PrefillArgs& a, int units, hipStream_t s) {
  if (a.stages & kStageScores) {
    const hipError_t e = a.q_lo != nullptr ? launch_bf16_scores<D, true>(a, units, s)
                                           : launch_bf16_scores<D, false>(a, units, s);
    if (e != hipSuccess) return e;
  }
  return (a.stages & kStageSelect) ? launch_select<bf16_t, D>(a, units, s) : hipSuccess;
}

template <int D>
hipError_t launch_f32(const PrefillArgs& a, int units, hipStream_t s) {
  const int nblk = (a.L + 63) / 64;
  if (a.stages & kStageScores) {
    hipLaunchKernelGGL((rowstats_f32<D>), dim3(units * nblk), dim3(64), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((colsum_f32<D>), dim3(units * nblk), dim3(64), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.out != nullptr) {
      hipLaunchKernelGGL((attnout_f32<D>), dim3(units * nblk), dim3(64), 0, s, a);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return (a.stages & kStageSelect) ? launch_select<float, D>(a, units, s) : hipSuccess;
}

}  // namespace

hipError_t launch_prefill(int dtype, int head_dim, const PrefillArgs& a, int units, hipStream_t s) {
  if (dtype == 0) return head_dim == 64 ? launch_f32<64>(a, units, s) : launch_f32<128>(a, units, s);
  return head_dim == 64 ? launch_bf16<64>(a, units, s) : launch_bf16<128>(a, units, s);
}

hipError_t launch_rope_prompt(int dtype, int head_dim, const void* x, void* y, void* y_lo, int32_t L, int units,
                              const float* cs, hipStream_t s) {
  // one thread per 16 bytes of the first half of a row
  const size_t runs = static_cast<size_t>(units) * L * (head_dim / 2) / (dtype == 0 ? 4 : 8);
  if (runs == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((runs + 255) / 256));
  const float2* t = reinterpret_cast<const float2*>(cs);
  if (dtype == 0) {
    if (head_dim == 64)
      hipLaunchKernelGGL((rope_prompt<float, 64>), grid, dim3(256), 0, s, static_cast<const float*>(x),
                         static_cast<float*>(y), nullptr, L, runs, t);
    else
      hipLaunchKernelGGL((rope_prompt<float, 128>), grid, dim3(256), 0, s, static_cast<const float*>(x),
                         static_cast<float*>(y), nullptr, L, runs, t);
  } else {
    if (head_dim == 64)
      hipLaunchKernelGGL((rope_prompt<bf16_t, 64>), grid, dim3(256), 0, s, static_cast<const bf16_t*>(x),
                         static_cast<bf16_t*>(y), static_cast<bf16_t*>(y_lo), L, runs, t);
    else
      hipLaunchKernelGGL((rope_prompt<bf16_t, 128>), grid, dim3(256), 0, s, static_cast<const bf16_t*>(x),
                         static_cast<bf16_t*>(y), static_cast<bf16_t*>(y_lo), L, runs, t);
  }
  return hipGetLastError();
}

hipError_t launch_clear(int32_t* pos, float* score, float* comp, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int blocks = static_cast<int>(std::min<size_t>((n + 255) / 256, 4096));
  hipLaunchKernelGGL(clear_kernel, dim3(blocks), dim3(256), 0, s, pos, score, comp, n);
  return hipGetLastError();
}

}  // namespace h2o
