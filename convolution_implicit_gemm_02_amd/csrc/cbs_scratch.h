// cbs_scratch.h -- between the host library (cbs_host.cpp) and the
// no-allocation entry point (cbs_noalloc.hip).  Not part of the public C ABI.
#pragma once
#include "../../include/cbs.h"
#include "cbs_internal.h"

namespace cbs {

// Launch parameters of one run of layer L with its current configuration and
// cross-workgroup split-K factor splitk (0: the layer's own), writing the
// partial tiles to ws (ws_cap bytes) and taking tickets in counters
// (counters_cap entries) instead of the layer's own workspace.  *tiles is the
// number of counters the launch uses (0 without a split).  Checks the layer
// and buffers as cbs_run_layer does, that the configuration can run the split,
// that the run fits the given workspace, and that the current device is the
// layer's; sets the thread's last error on failure.
cbs_status scratch_launch(const cbs_layer *L, const void *in, void *out, int32_t splitk, void *ws, size_t ws_cap,
                          unsigned *counters, size_t counters_cap, ConvParams *p, int *variant, int *config,
                          unsigned *tiles);

// Record a failure as the calling thread's last error and return st.
cbs_status report_error(cbs_status st, const char *what, const char *detail);

}  // namespace cbs
