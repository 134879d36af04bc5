// Instantiates the f32 forward and phase-1 kernels for dk = 16.
#include "dp_kernels.hpp"

DP_DEFINE_LAUNCHERS(float, f32, 16)
