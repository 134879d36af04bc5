// Instantiates the bf16 forward and phase-1 kernels for dk = 32.
#include "dp_kernels.hpp"

DP_DEFINE_LAUNCHERS(dp::bf16_t, bf16, 32)
