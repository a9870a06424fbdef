// Streaming-read reference for the bandwidth roofline: a coalesced 16-byte
// read of a whole device buffer, folded with XOR, nothing else.  Its rate is
// the practical HBM read ceiling of the device, against which the
// compressed-page scan's algorithmic bandwidth is also reported.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/tq.h"

namespace tq {
namespace {

typedef uint32_t u4 __attribute__((ext_vector_type(4)));

constexpr int kProbeThreads = 256;
constexpr int kProbeBlocks = 2048;  // 8 work-groups per CU on 256 CUs (grid-stride)

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u4* __restrict__ x, int64_t n16,
                                                                  uint32_t* sink) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kProbeThreads;
  uint32_t s = 0;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kProbeThreads + threadIdx.x; i < n16; i += stride) {
    const u4 v = __builtin_nontemporal_load(x + i);
    s ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // keeps the loads alive; the store happens only for one fold value in 2^32
  if (s == 0x9E3779B9u) sink[0] = s;
}

}  // namespace
}  // namespace tq

TQ_API int tq_read_probe(const void* buf, int64_t bytes, uint32_t* sink, int reps, double* best_ms, void* stream) {
  if (!buf || !sink || !best_ms || bytes <= 0 || bytes % 16 != 0 || reps < 1 || reps > 1000) return TQ_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(buf) % 16 != 0) return TQ_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipEvent_t a = nullptr, b = nullptr;
  // timing-only events, as for the scan's: no system-scope fence when recorded
  if (hipEventCreateWithFlags(&a, hipEventDisableSystemFence) != hipSuccess ||
      hipEventCreateWithFlags(&b, hipEventDisableSystemFence) != hipSuccess) {
    if (a) (void)hipEventDestroy(a);
    return TQ_ERR_HIP;
  }
  int rc = TQ_OK;
  double best = -1.0;
  for (int r = 0; r < reps && rc == TQ_OK; ++r) {
    float ms = 0.0f;
    if (hipEventRecord(a, s) != hipSuccess) rc = TQ_ERR_HIP;
    if (rc == TQ_OK) {
      hipLaunchKernelGGL(tq::read_probe_kernel, dim3(tq::kProbeBlocks), dim3(tq::kProbeThreads), 0, s,
                         static_cast<const tq::u4*>(buf), bytes / 16, sink);
      if (hipGetLastError() != hipSuccess || hipEventRecord(b, s) != hipSuccess || hipEventSynchronize(b) != hipSuccess ||
          hipEventElapsedTime(&ms, a, b) != hipSuccess)
        rc = TQ_ERR_HIP;
    }
    if (rc == TQ_OK && (best < 0.0 || ms < best)) best = ms;
  }
  if (hipEventDestroy(a) != hipSuccess || hipEventDestroy(b) != hipSuccess) rc = TQ_ERR_HIP;
  if (rc == TQ_OK) *best_ms = best;
  return rc;
}
