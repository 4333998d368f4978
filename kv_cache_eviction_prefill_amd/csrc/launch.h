// Internal launch interface between the cache object and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace h2o {

// One decode step over every unit of a cache.
struct DecodeArgs {
  const void* q;     // [units, d] new query
  const void* knew;  // [units, d] new key
  const void* vnew;  // [units, d] new value
  void* kslots;      // [units, k, d]
  void* vslots;      // [units, k, d]
  float* score;      // [units, kstride] running score (Kahan sum)
  float* comp;       // [units, kstride] Kahan compensation
  int32_t* pos;      // [units, kstride] position per slot, -1 when empty
  float* out;        // [units, d]
  int32_t* evicted;  // [units] or nullptr
  float* part;       // split mode: [units, nsplit, 2 + d] partial (max, sum, o)
  float* logits;     // split mode: [units, k + 1] base-2 logits (new token at index k)
  const float* fixed_new;  // the new token's fixed score of unit u at fixed_new[u * fixed_stride]
                           // (scores do not accumulate), or nullptr
  int32_t fixed_stride;
  int32_t k;           // slots per unit
  int32_t kstride;     // per-unit stride of score/comp/pos: k rounded up to 32 (128-byte rows)
  int32_t count;       // occupied slots before this step (slots 0..count-1)
  int32_t new_pos;     // position i of the new token
  int32_t cand_limit;  // positions <= cand_limit are eviction candidates (i - K_r)
  int32_t new_is_candidate;  // K_r == 0: the new token competes for eviction
  int32_t plain_until;  // steps at positions below this add weights to scores in plain fp32 (the
                        // compensation stays 0); from it on, Kahan-compensated
  int32_t pat_kind, pat_period, pat_width;  // sparse pattern kept before heavy hitters
  int32_t* rank;       // position rolling: [units, kstride] slot positions inside the cache, or nullptr
  const float* rope_th;  // [d/2] (hi, lo) theta_m / (2 pi), when rank != nullptr
  int32_t nsplit;      // blocks per unit (1: single-block path)
  int32_t split_len;   // slots per split block
  float c2;            // scale * log2(e)
};

hipError_t launch_decode(int dtype, int head_dim, const DecodeArgs& a, int units, hipStream_t s);

// Several decode steps in one launch with every unit's K/V slot rows held in
// shared memory (single-block path, no position rolling, no fixed scores):
// `a` describes the first step; step t reads its q/k/v at + t * tok_bytes and
// writes out + t * out_step and evicted + t * units.  Results equal `steps`
// launch_decode calls.  decode_resident_fits says whether a cache's rows fit.
bool decode_resident_fits(int dtype, int head_dim, int units, int k);

// Split-path steps of a multi-step call in one launch each.  prev == nullptr:
// step `cur`'s slices alone (the split launch).  Otherwise the launch finishes
// step `prev` (its partials and logits in prev.part / prev.logits; scores,
// compensations, positions and, with position rolling, places read from prev's
// arrays and written, for the slots of each block's step-`cur` slices, to ny_*,
// which are cur's arrays) and then runs step `cur`'s slices.
// launch_decode_finish is the finish launch alone (in place on a's arrays).  No
// fixed scores; every step on the split path.
hipError_t launch_decode_split(int dtype, int head_dim, const DecodeArgs* prev, const DecodeArgs& cur,
                               float* ny_score, float* ny_comp, int32_t* ny_pos, int32_t* ny_rank, int units,
                               hipStream_t s);
hipError_t launch_decode_finish(int dtype, int head_dim, const DecodeArgs& a, int units, hipStream_t s);
hipError_t launch_decode_resident(int dtype, int head_dim, const DecodeArgs& a, int units, int steps,
                                  int64_t tok_bytes, int64_t out_step, hipStream_t s);

// Prefill stages: the two score passes (row normalisers, column sums) and the
// select + fill.
enum PrefillStage : int32_t { kStageScores = 1, kStageSelect = 2 };

// Prefill of every unit of a cache.
struct PrefillArgs {
  int32_t stages;     // PrefillStage bits
  const void* q;  // [units, L, d]
  const void* k;  // [units, L, d]
  const void* v;  // [units, L, d]
  const void* q_lo;  // bf16 position rolling: [units, L, d] lo parts of the rotated q (q holds the hi
  const void* k_lo;  // parts), likewise for k; nullptr otherwise
  int32_t L;
  int32_t Lpad;       // stride of the per-row scratch arrays (multiple of 32, >= L)
  float* row_lse2;    // [units, Lpad] log2 sum_j exp2(c2 q_r.k_j) of each row; 0 past L
  float* col_sum;     // [units, Lpad] attention received by each prompt token
  float* out;         // [units, L, d] prompt attention output, or nullptr
  const float* scores_in;  // [units, scores_stride] scores the select ranks by, or nullptr (col_sum)
  int32_t scores_stride;
  int32_t kv_rows;    // rows per unit of k and v (>= L): the select gathers rows 0..L-1
  const void* kcache;  // [units, kv_rows, d] the key rows the select stores (k unless k holds rotated keys)
  int32_t* rank;       // position rolling: [units, kstride] slot positions inside the cache, or nullptr
  int32_t pat_kind, pat_period, pat_width;  // sparse pattern kept before heavy hitters (query i = L)
  void* kslots;       // [units, k, d]
  void* vslots;       // [units, k, d]
  float* score;       // [units, kstride]
  float* comp;        // [units, kstride]
  int32_t* pos;       // [units, kstride]
  int32_t heavy;
  int32_t recent;
  int32_t kcap;       // k
  int32_t kstride;    // per-unit stride of score/comp/pos
  float scale;
  float c2;           // scale * log2(e)
};

hipError_t launch_prefill(int dtype, int head_dim, const PrefillArgs& a, int units, hipStream_t s);

// Rotary embedding of a prompt: rows r of x [units, L, d] rotated to position r
// into y (same layout), from the (cos, sin) table [>= L, d/2].  bf16: y receives
// bf16(v) and y_lo bf16(v - bf16(v)) of each rotated value v; fp32: y receives v
// and y_lo is unused.
hipError_t launch_rope_prompt(int dtype, int head_dim, const void* x, void* y, void* y_lo, int32_t L, int units,
                              const float* cs, hipStream_t s);

// Mark every slot empty (pos = -1, score = comp = 0).
hipError_t launch_clear(int32_t* pos, float* score, float* comp, size_t n, hipStream_t s);

}  // namespace h2o
