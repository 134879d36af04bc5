// Instantiates the bf16 backward kernels for dk = 16.
#include "dp_bwd.hpp"

DP_DEFINE_BWD_LAUNCHER(dp::bf16_t, bf16, 16)
