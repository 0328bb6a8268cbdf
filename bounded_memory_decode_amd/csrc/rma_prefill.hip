// Chunked-prefill kernels (placeholder translation unit; the block path
// currently runs the decode kernels token by token, see rma_host.cpp).
#include "rma_kernels.h"
