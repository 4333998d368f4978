// Streaming-read probe: a measurement aid, not part of the method.  It reads a
// buffer once with 16-byte non-temporal loads, 8 in flight per lane, each block
// on contiguous 32 KiB runs, so timing it gives the read bandwidth this GPU
// sustains for a plain stream - the practical ceiling for the decode kernel's
// HBM fraction.
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
