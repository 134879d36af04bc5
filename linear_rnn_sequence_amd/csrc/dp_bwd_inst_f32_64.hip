// Instantiates the f32 backward kernels for dk = 64.
#include "dp_bwd.hpp"

DP_DEFINE_BWD_LAUNCHER(float, f32, 64)
