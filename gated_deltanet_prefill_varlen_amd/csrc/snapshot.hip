// Checkpoint copy: gathers checkpoint states into caller-owned pool slots
// (device memory or device-mapped pinned host memory).  Pure streaming copy in
// 16-byte vectors with non-temporal hints, so it does not evict the scan's
// working set from the caches it shares while both run.  Into host memory one
// workgroup per item keeps the host link saturated on few CUs (a copy there
// runs about 8x longer than a chat-wave scan, and stalls the scan
// workgroups that share its CUs).
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = 4;  // 16-byte vectors per thread per pass
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(kThreads) snapshot_copy_kernel(const CopyArgs a) {
  const int i = blockIdx.y;
  const int64_t n16 = a.bytes_each / 16;
  const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const char*>(a.src) +
                                                    (size_t)i * a.bytes_each);
  u32x4* dst = reinterpret_cast<u32x4*>(static_cast<char*>(a.dst) + (size_t)a.slot[i] * a.bytes_each);
  const int64_t step = (int64_t)gridDim.x * kThreads * kPerThread;
  for (int64_t base = (int64_t)blockIdx.x * kThreads * kPerThread + threadIdx.x; base < n16;
       base += step) {
    u32x4 v[kPerThread];
#pragma unroll
    for (int u = 0; u < kPerThread; ++u) {
      const int64_t e = base + (int64_t)u * kThreads;
      if (e < n16) v[u] = __builtin_nontemporal_load(src + e);
    }
#pragma unroll
    for (int u = 0; u < kPerThread; ++u) {
      const int64_t e = base + (int64_t)u * kThreads;
      if (e < n16) __builtin_nontemporal_store(v[u], dst + e);
    }
  }
}

}  // namespace

hipError_t launch_snapshot_copy(const CopyArgs& a, hipStream_t st) {
  const int64_t n16 = a.bytes_each / 16;
  const int64_t per_block = (int64_t)kThreads * kPerThread;
  const int gx = a.host_dst ? 1 : (int)std::min<int64_t>((n16 + per_block - 1) / per_block, 1024);
  for (int i0 = 0; i0 < a.n; i0 += 65535) {
    CopyArgs b = a;
    b.src = static_cast<const char*>(a.src) + (size_t)i0 * a.bytes_each;
    b.slot = a.slot + i0;
    b.n = std::min(65535, a.n - i0);
    hipLaunchKernelGGL(snapshot_copy_kernel, dim3(gx, b.n), dim3(kThreads), 0, st, b);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace gdn
