// cbs_kernels.hip -- the configuration table, the variant dispatcher and the
// graph-entry NCHW -> NHWC pack / quantise kernels of libcbs.  The conv
// kernels themselves are in conv_kernels.h (one translation unit per variant).
#include "cbs_internal.h"
#include "conv_configs.h"

namespace cbs {

typedef float f32x4 __attribute__((ext_vector_type(4)));

static const KernelConfig kConfigs[] = {
#define X(id, cb, pb, wco, wpx, wk, pf, name) {cb, pb, wco, wpx, wk, 0, 0, 0, name},
    CBS_CONFIG_LIST(X)
#undef X
#define X(id, mb, nb, wm, wn, ks, name) {nb, mb, wn, wm, 1, 1, 0, 0, name},
    CBS_LDS_CONFIG_LIST(X)
#undef X
#define X(id, th, tw, name) {4, th * tw / 64, 1, 4, 1, 2, th, tw, name},
    CBS_HALO_CONFIG_LIST(X)
#undef X
#define X(id, cb, pb, wco, wpx, wk, pf, name) {cb, pb, wco, wpx, wk, 0, 0, 0, name},
    CBS_CONFIG_LIST_EXT(X)
#undef X
#define X(id, mb, nb, wm, wn, ks, name) {nb, mb, wn, wm, 1, 1, 0, 0, name},
    CBS_LDS_CONFIG_LIST_EXT(X)
#undef X
#define X(id, mb, nb, wm, wn, ks, ns, name) {nb, mb, wn, wm, 1, 1, 0, 0, name},
    CBS_LDS_RING_CONFIG_LIST(X)
#undef X
#define X(id, th, tw, name) {1, th * tw / 64, 1, 4, 1, 3, th, tw, name},
    CBS_HALO_PAIR_CONFIG_LIST(X)
#undef X
#define X(id, mb, nb, wm, wn, ks, ns, name) {nb, mb, wn, wm, 1, 1, 0, 0, name},
    CBS_LDS_RING_SWZ_CONFIG_LIST(X)
#undef X
#define X(id, cbw, wco, wpx, occ, name) {cbw, 1, wco, wpx, 1, 4, occ, 0, name},
    CBS_WS_CONFIG_LIST(X)
#undef X
#define X(id, cbw, wpx, occ, name) {cbw, 1, 1, wpx, 1, 5, occ, 0, name},
    CBS_WSG_CONFIG_LIST(X)
#undef X
#define X(id, cbw, wco, wpx, occ, name) {cbw, 1, wco, wpx, 1, 4, occ, 0, name},
    CBS_WS_CONFIG_LIST_EXT(X)
#undef X
};

// A configuration's id is its index in kConfigs (the launch switch and the
// tile table refer to it by number): the lists must stay in id order.
constexpr int kConfigIds[] = {
#define X(id, ...) id,
    CBS_CONFIG_LIST(X) CBS_LDS_CONFIG_LIST(X) CBS_HALO_CONFIG_LIST(X) CBS_CONFIG_LIST_EXT(X) CBS_LDS_CONFIG_LIST_EXT(X)
    CBS_LDS_RING_CONFIG_LIST(X) CBS_HALO_PAIR_CONFIG_LIST(X) CBS_LDS_RING_SWZ_CONFIG_LIST(X) CBS_WS_CONFIG_LIST(X)
    CBS_WSG_CONFIG_LIST(X) CBS_WS_CONFIG_LIST_EXT(X)
#undef X
};
constexpr bool config_ids_in_order() {
  for (int i = 0; i < (int)(sizeof(kConfigIds) / sizeof(kConfigIds[0])); i++)
    if (kConfigIds[i] != i) return false;
  return sizeof(kConfigIds) == sizeof(kConfigs) / sizeof(kConfigs[0]) * sizeof(int);
}
static_assert(config_ids_in_order(), "configuration ids must equal their index in kConfigs");

int num_configs() { return (int)(sizeof(kConfigs) / sizeof(kConfigs[0])); }
const KernelConfig &config(int i) { return kConfigs[i]; }

hipError_t launch_conv(int var, int cfg, const ConvParams &p, hipStream_t stream) {
  switch (var) {
    case 0: return launch_var_0(cfg, p, stream);
    case 1: return launch_var_1(cfg, p, stream);
    case 2: return launch_var_2(cfg, p, stream);
    case 3: return launch_var_3(cfg, p, stream);
    case 4: return launch_var_4(cfg, p, stream);
    case 5: return launch_var_5(cfg, p, stream);
    case 6: return launch_var_6(cfg, p, stream);
    case 7: return launch_var_7(cfg, p, stream);
    case 8: return launch_var_8(cfg, p, stream);
    case 9: return launch_var_9(cfg, p, stream);
    case 10: return launch_var_10(cfg, p, stream);
    case 11: return launch_var_11(cfg, p, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_conv_group(int var, int cfg, const GroupArgs &g, unsigned grid, hipStream_t stream) {
  switch (var) {
    case 0: return launch_group_var_0(cfg, g, grid, stream);
    case 1: return launch_group_var_1(cfg, g, grid, stream);
    case 2: return launch_group_var_2(cfg, g, grid, stream);
    case 5: return launch_group_var_5(cfg, g, grid, stream);
    case 6: return launch_group_var_6(cfg, g, grid, stream);
    case 7: return launch_group_var_7(cfg, g, grid, stream);
    case 8: return launch_group_var_8(cfg, g, grid, stream);
    case 9: return launch_group_var_9(cfg, g, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

// ------------------------------------------------------ graph-entry packs --
// One thread per (pixel, 4-channel group); consecutive threads take
// consecutive pixels so the NCHW plane reads are coalesced.
__global__ __launch_bounds__(256) void pack_nhwc_f32_kernel(const float *__restrict__ x,
                                                            float *__restrict__ y, int n, int c, int hw,
                                                            int c_pad) {
  const long total = (long)n * hw * (c_pad >> 2);
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const long npix = (long)n * hw;
  const int q = (int)(idx / npix);
  const long pix = idx - (long)q * npix;
  const int b = (int)(pix / hw);
  const int i = (int)(pix - (long)b * hw);
  f32x4 v;
#pragma unroll
  for (int e = 0; e < 4; e++) {
    const int ch = 4 * q + e;
    v[e] = ch < c ? x[((long)b * c + ch) * hw + i] : 0.0f;
  }
  *(f32x4 *)(y + pix * c_pad + 4 * q) = v;
}

__global__ __launch_bounds__(256) void quantize_nhwc_i8_kernel(const float *__restrict__ x,
                                                               int8_t *__restrict__ y, float s_x, int n,
                                                               int c, int hw, int c_pad) {
  const long total = (long)n * hw * (c_pad >> 2);
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const long npix = (long)n * hw;
  const int q = (int)(idx / npix);
  const long pix = idx - (long)q * npix;
  const int b = (int)(pix / hw);
  const int i = (int)(pix - (long)b * hw);
  unsigned word = 0;
#pragma unroll
  for (int e = 0; e < 4; e++) {
    const int ch = 4 * q + e;
    int qv = 0;
    if (ch < c) {
      // fp32 division, correctly rounded, then round half to even and clamp
      const float t = __fdiv_rn(x[((long)b * c + ch) * hw + i], s_x);
      float rr = rintf(t);
      rr = fminf(fmaxf(rr, -127.0f), 127.0f);
      qv = (int)rr;
    }
    word |= ((unsigned)(qv & 0xff)) << (8 * e);
  }
  *(unsigned *)(y + pix * c_pad + 4 * q) = word;
}

// Asymmetric uint8: q = clamp(rne(fp32(x / s_x)) + z, 0, 255); padded lanes
// get z, the code of a real zero.
__global__ __launch_bounds__(256) void quantize_nhwc_u8_kernel(const float *__restrict__ x,
                                                               uint8_t *__restrict__ y, float s_x, int z, int n,
                                                               int c, int hw, int c_pad) {
  const long total = (long)n * hw * (c_pad >> 2);
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const long npix = (long)n * hw;
  const int q = (int)(idx / npix);
  const long pix = idx - (long)q * npix;
  const int b = (int)(pix / hw);
  const int i = (int)(pix - (long)b * hw);
  const float zf = (float)z;
  unsigned word = 0;
#pragma unroll
  for (int e = 0; e < 4; e++) {
    const int ch = 4 * q + e;
    int qv = z;
    if (ch < c) {
      // fp32 division, correctly rounded, round half to even, then the zero point and the clamp
      const float t = __fdiv_rn(x[((long)b * c + ch) * hw + i], s_x);
      const float rr = fminf(fmaxf(rintf(t) + zf, 0.0f), 255.0f);
      qv = (int)rr;
    }
    word |= ((unsigned)(qv & 0xff)) << (8 * e);
  }
  *(unsigned *)(y + pix * c_pad + 4 * q) = word;
}

hipError_t launch_pack_nhwc_f32(const float *x, float *y, int n, int c, int hw, int c_pad,
                                hipStream_t stream) {
  const long total = (long)n * hw * (c_pad >> 2);
  if (total == 0) return hipSuccess;
  const unsigned grid = (unsigned)((total + 255) / 256);
  hipLaunchKernelGGL(pack_nhwc_f32_kernel, dim3(grid), dim3(256), 0, stream, x, y, n, c, hw, c_pad);
  return hipGetLastError();
}

hipError_t launch_quantize_nhwc_i8(const float *x, int8_t *y, float s_x, int n, int c, int hw,
                                   int c_pad, hipStream_t stream) {
  const long total = (long)n * hw * (c_pad >> 2);
  if (total == 0) return hipSuccess;
  const unsigned grid = (unsigned)((total + 255) / 256);
  hipLaunchKernelGGL(quantize_nhwc_i8_kernel, dim3(grid), dim3(256), 0, stream, x, y, s_x, n, c, hw,
                     c_pad);
  return hipGetLastError();
}

hipError_t launch_quantize_nhwc_u8(const float *x, uint8_t *y, float s_x, int z, int n, int c, int hw,
                                   int c_pad, hipStream_t stream) {
  const long total = (long)n * hw * (c_pad >> 2);
  if (total == 0) return hipSuccess;
  const unsigned grid = (unsigned)((total + 255) / 256);
  hipLaunchKernelGGL(quantize_nhwc_u8_kernel, dim3(grid), dim3(256), 0, stream, x, y, s_x, z, n, c, hw, c_pad);
  return hipGetLastError();
}

}  // namespace cbs
