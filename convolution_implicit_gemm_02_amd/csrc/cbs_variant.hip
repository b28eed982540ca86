// cbs_variant.hip -- one kernel variant of libcbs (fp32 / int8, operand
// gathering, epilogue), selected at compile time with -DCBS_VAR=<n>; the
// build compiles this file once per variant, in parallel.
#include "conv_kernels.h"

#ifndef CBS_VAR
#error "compile with -DCBS_VAR=<variant>"
#endif

namespace cbs {
#define CBS_PASTE2(a, b) a##b
#define CBS_PASTE(a, b) CBS_PASTE2(a, b)
hipError_t CBS_PASTE(launch_var_, CBS_VAR)(int cfg, const ConvParams &p, hipStream_t stream) {
  return launch_variant<CBS_VAR>(cfg, p, stream);
}
#if CBS_VAR != 3 && CBS_VAR != 4 && CBS_VAR != 10 && CBS_VAR != 11  // not the raw-accumulator test hooks
hipError_t CBS_PASTE(launch_group_var_, CBS_VAR)(int cfg, const GroupArgs &g, unsigned grid, hipStream_t stream) {
  return launch_group_variant<CBS_VAR>(cfg, g, grid, stream);
}
#endif
}  // namespace cbs
