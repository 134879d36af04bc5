// Instantiates the bf16 backward kernels for dk = 64.
#include "dp_bwd.hpp"

DP_DEFINE_BWD_LAUNCHER(dp::bf16_t, bf16, 64)
