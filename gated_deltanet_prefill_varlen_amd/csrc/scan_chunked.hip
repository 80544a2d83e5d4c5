// Prefill dispatch.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

hipError_t launch_prefill(const ScanArgs& a, hipStream_t st) { return launch_prefill_recurrent(a, st); }

}  // namespace gdn
