// The backward kernels for fp32 I/O, one instantiation per head dimension
// (a translation unit of its own, so the library builds in parallel).
#include "run_bwd.h"

using monarch::bf16_t;
using namespace monarch_host;

MONARCH_INSTANTIATE_RUN_BWD(float, 16)
MONARCH_INSTANTIATE_RUN_BWD(float, 32)
MONARCH_INSTANTIATE_RUN_BWD(float, 64)
MONARCH_INSTANTIATE_RUN_BWD(float, 128)
