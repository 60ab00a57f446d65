// Discrete reduce-scatter kernels for bf16 input, fp32 output (every order, average mode,
// K specialisation and tile shape the planner picks among).
#include "zr_rsf_kernel.hpp"

namespace zr {
namespace rsf {
template Fns pick_avg<uint16_t, float>(int, int, int, bool, bool);
}  // namespace rsf
}  // namespace zr
