// cbs_noalloc.hip -- cbs_run_layer_noalloc: cbs_run_layer for callers that
// cannot allocate device memory (code under HIP graph capture, serving loops
// that must not call hipMalloc), with the cross-workgroup split-K factor
// chosen per call.
//
// A split-K run needs device memory beyond its input and output: each
// workgroup's partial tile and one arrival ticket per output tile.  Here they
// live in `scratch`, a fixed array of this library on every device, instead
// of the workspace that cbs_layer_set_config allocates for a layer.  This
// entry point therefore allocates nothing, whatever split it is asked for.
//
// `scratch` is a device symbol: in host code its name is not a device
// address.  Its address on a device comes from hipGetSymbolAddress, once per
// device with that device current, and only that address is passed on.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "../../include/cbs.h"
#include "cbs_internal.h"
#include "cbs_scratch.h"

namespace {

constexpr size_t kPartialBytes = CBS_NOALLOC_PARTIAL_BYTES;
constexpr size_t kTickets = CBS_NOALLOC_TICKETS;

// Partial tiles (kPartialBytes), then the arrival tickets (kTickets
// unsigned).  Every run on a device shares that device's copy.
static __device__ __align__(256) unsigned char scratch[kPartialBytes + kTickets * sizeof(unsigned)];

// The tickets a launch uses must start at zero: cleared by a kernel (not a
// memset, so that a captured graph holds only kernel nodes).
__global__ __launch_bounds__(256) void clear_tickets(unsigned *t, unsigned n) {
  const unsigned i = blockIdx.x * 256u + threadIdx.x;
  if (i < n) t[i] = 0u;
}

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch[kMaxDevices] = {};  // the device address of `scratch` on each device, once looked up

// The address of the current device's `scratch`, looked up on the first call
// on that device.
cbs_status scratch_address(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return cbs::report_error(CBS_EDEVICE, "run_layer_noalloc", "no current HIP device");
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_scratch[dev]) {
    void *ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return cbs::report_error(CBS_EDEVICE, "run_layer_noalloc: hipGetSymbolAddress(scratch)",
                               e != hipSuccess ? hipGetErrorString(e) : "null address");
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return CBS_OK;
}

}  // namespace

extern "C" cbs_status cbs_run_layer_noalloc(const cbs_layer *layer, const void *in, void *out, int32_t splitk,
                                            void *stream) {
  void *base = nullptr;
  cbs_status st = scratch_address(&base);
  if (st != CBS_OK) return st;
  unsigned *tickets = (unsigned *)((unsigned char *)base + kPartialBytes);
  cbs::ConvParams p;
  int variant = 0, cfg = 0;
  unsigned tiles = 0;
  st = cbs::scratch_launch(layer, in, out, splitk, base, kPartialBytes, tickets, kTickets, &p, &variant, &cfg, &tiles);
  if (st != CBS_OK) return st;
  const hipStream_t s = (hipStream_t)stream;
  if (tiles > 0) {
    hipLaunchKernelGGL(clear_tickets, dim3((tiles + 255u) / 256u), dim3(256), 0, s, tickets, tiles);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return cbs::report_error(CBS_ELAUNCH, "run_layer_noalloc: ticket clear", hipGetErrorString(e));
  }
  const hipError_t e = cbs::launch_conv(variant, cfg, p, s);
  if (e != hipSuccess) return cbs::report_error(CBS_ELAUNCH, "run_layer_noalloc: conv launch", hipGetErrorString(e));
  return CBS_OK;
}
