// Measurement aids, not part of the method.
//
// Streaming-read probe: reads a buffer once with 16-byte non-temporal loads, 8
// in flight per lane, each block on contiguous 32 KiB runs, so timing it gives
// the read bandwidth this GPU sustains for a plain stream - the practical
// ceiling for the decode kernel's HBM fraction.
//
// Matrix/vector mix probe: the instruction mix of a prefill scoring pass with
// nothing else - per wave and iteration 16 MFMAs 32x32x16 bf16 (the work of one
// 64 x 32 logit tile at d = 128) and, per lane, 32 times one fma, one exp2 and
// one add (the terms and sums of those 2048 logits) - from registers only: no
// memory traffic, no barriers, and the vector work independent of the matrix
// results, so nothing but the two pipes and the clock bounds it.  Timing the
// matrix part alone, the vector part alone and both together gives the rates
// the passes could reach at best on this GPU.
#include <hip/hip_runtime.h>

#include "h2o.h"
#include "h2o_device.h"

namespace h2o {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeInFlight = 8;  // 16-byte loads in flight per lane
constexpr int kProbeBlocksPerCu = 16;

// Each block reads contiguous 32 KiB runs (8 wave-wide loads of 1 KiB per wave),
// the runs of the grid's blocks side by side, then the next grid-wide stripe.
__global__ __launch_bounds__(kProbeThreads) void read_probe(const uint4* p, size_t n16, uint32_t* sink) {
  constexpr size_t kRun = static_cast<size_t>(kProbeThreads) * kProbeInFlight;  // 16-byte chunks per run
  uint32_t acc = 0u;
  for (size_t base = blockIdx.x * kRun; base < n16; base += static_cast<size_t>(gridDim.x) * kRun) {
    const size_t i = base + threadIdx.x;
    if (base + kRun <= n16) {
      uint4 v[kProbeInFlight];
#pragma unroll
      for (int u = 0; u < kProbeInFlight; ++u) v[u] = ld16_stream(p + i + u * kProbeThreads);
#pragma unroll
      for (int u = 0; u < kProbeInFlight; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    } else {  // the buffer's ragged end
      for (size_t t = i; t < n16; t += kProbeThreads) {
        const uint4 v = ld16_stream(p + t);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
      }
    }
  }
  // the loads feed a value the kernel may store, so none can be dropped; the
  // store itself happens only on one chance in 2^32
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

// Mix probe.  MODE 0: the MFMAs alone; 1: MFMAs and vector work; 2: vector work
// alone.  Four accumulator chains keep the matrix pipe fed from one wave; the
// vector values stay in (0, 1] (x -> exp2(-(x/2 + 1/2))).
constexpr int kMixThreads = 256;
constexpr int kMixBlocksPerCu = 4;  // 4 waves per SIMD, as the scoring passes run

template <int MODE>
__global__ __launch_bounds__(kMixThreads) void mix_probe(int iters, uint32_t* sink) {
  const int lane = threadIdx.x % kWave;
  bf16x8 fa, fb;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    fa[e] = static_cast<__bf16>(static_cast<float>((lane + e) % 7 - 3) * 0.125f);
    fb[e] = static_cast<__bf16>(static_cast<float>((lane * 3 + e) % 5 - 2) * 0.25f);
  }
  floatx16 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = floatx16{};
  floatx16 x[2];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int i = 0; i < 16; ++i) x[s][i] = 0.01f * static_cast<float>(lane % 9 + i + s);
  float part[4] = {0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
    if constexpr (MODE != 2) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fb, acc[j], 0, 0, 0);
    }
    if constexpr (MODE != 0) {
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          x[s][i] = fast_exp2(-fmaf(x[s][i], 0.5f, 0.5f));
          part[i & 3] += x[s][i];
        }
    }
    asm volatile("" : "+v"(fa), "+v"(fb));  // operands the compiler cannot treat as loop-invariant
  }
  float tot = (part[0] + part[1]) + (part[2] + part[3]);
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) tot += acc[j][i];
  // every result feeds a value the kernel may store, so no work can be dropped;
  // the store itself happens only on one chance in 2^32
  if (__float_as_uint(tot) == 0x9e3779b9u) sink[0] = __float_as_uint(tot);
}

}  // namespace
}  // namespace h2o

extern "C" h2o_status h2o_probe_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  if (buf == nullptr || sink == nullptr) return H2O_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(buf) & 15u) != 0 || (bytes & 15u) != 0) return H2O_ERR_INVALID_ARG;
  if (bytes == 0) return H2O_OK;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return H2O_ERR_HIP;
  const size_t n16 = bytes / 16;
  // 16 blocks of 256 threads per compute unit, fewer for small buffers
  const size_t want = static_cast<size_t>(cus) * h2o::kProbeBlocksPerCu;
  const size_t run = static_cast<size_t>(h2o::kProbeThreads) * h2o::kProbeInFlight;
  const size_t need = (n16 + run - 1) / run;
  const unsigned blocks = static_cast<unsigned>(want < need ? want : need);
  hipLaunchKernelGGL(h2o::read_probe, dim3(blocks), dim3(h2o::kProbeThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(buf), n16, sink);
  return hipGetLastError() == hipSuccess ? H2O_OK : H2O_ERR_HIP;
}

extern "C" h2o_status h2o_probe_mix(int32_t mode, int32_t iters, uint32_t* sink, void* stream) {
  if (sink == nullptr || mode < 0 || mode > 2 || iters < 1) return H2O_ERR_INVALID_ARG;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return H2O_ERR_HIP;
  const dim3 grid(static_cast<unsigned>(cus * h2o::kMixBlocksPerCu)), block(h2o::kMixThreads);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (mode == 0) hipLaunchKernelGGL(h2o::mix_probe<0>, grid, block, 0, s, iters, sink);
  else if (mode == 1) hipLaunchKernelGGL(h2o::mix_probe<1>, grid, block, 0, s, iters, sink);
  else hipLaunchKernelGGL(h2o::mix_probe<2>, grid, block, 0, s, iters, sink);
  return hipGetLastError() == hipSuccess ? H2O_OK : H2O_ERR_HIP;
}
