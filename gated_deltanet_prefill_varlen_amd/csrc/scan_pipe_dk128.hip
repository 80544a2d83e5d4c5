// Launcher of the pipelined chunked scan (d_k = d_v = 128, 32-token chunks):
// one workgroup of twelve waves per (prompt, value head); with pre-conv rows
// (ScanArgs::conv_x) the variant whose loader waves apply the short conv.
#include "scan_pipe_kernel.h"

namespace gdn {
namespace chunked {

template <bool CONV>
static hipError_t launch_pipe(const ScanArgs& a, hipStream_t st) {
  using C = PipeCfg<128, 128>;
  auto kern = pipelined_prefill_kernel<128, 128, CONV>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, C::bytes);
  if (e != hipSuccess) return e;
  ScanArgs b = a;
  b.chunk = C::CT;
  hipLaunchKernelGGL(kern, dim3(b.n_seqs, b.Hv), dim3(C::NTH), C::bytes, st, b);
  return hipGetLastError();
}

hipError_t launch_pipe_dk128(const ScanArgs& a, hipStream_t st) {
  return a.conv_x ? launch_pipe<true>(a, st) : launch_pipe<false>(a, st);
}

}  // namespace chunked
}  // namespace gdn
