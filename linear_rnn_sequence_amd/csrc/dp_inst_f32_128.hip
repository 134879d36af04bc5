// Instantiates the f32 forward and phase-1 kernels for dk = 128.
#include "dp_kernels.hpp"

DP_DEFINE_LAUNCHERS(float, f32, 128)
