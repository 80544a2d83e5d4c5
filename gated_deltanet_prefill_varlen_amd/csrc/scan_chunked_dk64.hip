// Chunked prefill kernels for head_k_dim = 64.
#include "scan_chunked_kernel.h"

GDN_CHUNKED_LAUNCHERS(64)
