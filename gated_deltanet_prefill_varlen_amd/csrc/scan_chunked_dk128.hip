// Chunked prefill kernels for head_k_dim = 128.
#include "scan_chunked_kernel.h"

GDN_CHUNKED_LAUNCHERS(128)
