// Discrete reduce-scatter kernels for fp32 input, bf16 output (every order, average mode,
// K specialisation and tile shape the planner picks among).
#include "zr_rsf_kernel.hpp"

namespace zr {
namespace rsf {
template Fns pick_avg<float, uint16_t>(int, int, int, bool, bool);
}  // namespace rsf
}  // namespace zr
