// Streaming-read probe: reads a device buffer once with 16-byte loads and
// keeps nothing, giving the read bandwidth the HBM sustains for a plain
// stream on this GPU (the reference the decode's cache-read rate is read
// against). Each thread keeps four loads in flight; the loaded words are
// folded into one value that is stored only if it equals a sentinel, so the
// loads cannot be dropped and almost nothing is written. Eight workgroups
// per compute unit (256 on MI355X).
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kProbeThreads = 256;
constexpr uint32_t kSentinel = 0x9E3779B9u;

__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const u32x4_t* __restrict__ src,
                                                                    size_t n16, u32x4_t* sink) {
  const size_t stride = (size_t)gridDim.x * kProbeThreads;
  size_t i = (size_t)blockIdx.x * kProbeThreads + threadIdx.x;
  u32x4_t acc = {0, 0, 0, 0};
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4_t a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    acc ^= a ^ b ^ c ^ d;
  }
  for (; i < n16; i += stride) acc ^= src[i];
  if ((acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) == kSentinel) sink[0] = acc;
}

}  // namespace

hipError_t launch_stream_read(const void* src, size_t bytes, void* sink, hipStream_t s) {
  const size_t n16 = bytes / 16;
  hipLaunchKernelGGL(stream_read_kernel, dim3(256 * 8), dim3(kProbeThreads), 0, s,
                     (const u32x4_t*)src, n16, (u32x4_t*)sink);
  return hipGetLastError();
}

}  // namespace mla
