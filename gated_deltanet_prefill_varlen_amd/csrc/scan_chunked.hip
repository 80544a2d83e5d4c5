// Prefill dispatch: bf16 io runs the chunked MFMA scan (scan_chunked_kernel.h).
// fp32 io runs the token-recurrent fp32 kernel: fp32 inputs are not exact bf16
// MFMA operands, so every product of the chunked form would need split
// operands and twice the LDS staging, for a dtype used only at small sizes.
#include "gdn_internal.h"

namespace gdn {
namespace chunked {
hipError_t launch_dk32(const ScanArgs& a, hipStream_t st);
hipError_t launch_dk64(const ScanArgs& a, hipStream_t st);
hipError_t launch_dk128(const ScanArgs& a, hipStream_t st);
hipError_t launch_pipe_dk128(const ScanArgs& a, hipStream_t st);
}  // namespace chunked

hipError_t launch_prefill(const ScanArgs& a, hipStream_t st) {
  if (!a.bf16) return launch_prefill_recurrent(a, st);
  if (a.dk == 32) return chunked::launch_dk32(a, st);
  if (a.dk == 64) return chunked::launch_dk64(a, st);
  if (a.dk == 128 && a.dv == 128 && a.chunk >= 32) return chunked::launch_pipe_dk128(a, st);
  if (a.dk == 128) return chunked::launch_dk128(a, st);
  return hipErrorInvalidValue;
}

}  // namespace gdn
