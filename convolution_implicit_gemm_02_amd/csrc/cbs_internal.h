// cbs_internal.h -- shared between the host library (cbs_host.cpp) and the
// kernels (cbs_kernels.hip) of libcbs.  Not part of the public C ABI.
#pragma once
#include <cstddef>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cbs {

// Kernel configuration: one wave computes CB x PB blocks of 16 output
// channels x 16 output pixels; a workgroup holds WCO x WPX x WK waves (WK
// waves split K inside the workgroup and are reduced through LDS).
struct KernelConfig {
  int cb, pb, wco, wpx, wk;
  int lds;  // 0: operands straight to registers (conv_igemm); 1: LDS-staged tiles (conv_lds);
            // 2: input halo tile + all weights in LDS (conv_halo, 3x3 with <= 64 output channels);
            // 3: conv_halo on column pairs (3x3 stride 1 with <= 8 output channels; th x tw pairs)
            // 4: conv_ws (fp32 1x1 stride 1: weights held in registers, runs of pixel blocks)
            // 5: conv_ws with the window gather (fp32 3x3, 9 or 18 K steps each within one tap;
            //    wpx waves interleave the run's blocks)
  int th, tw;  // conv_halo: output tile of th x tw pixels; conv_ws: th = workgroups per CU
  const char *name;
};

// conv_ws: deepest K (in 16-channel steps) compiled for waves holding cb
// channel blocks each, so that weights and two blocks of activations fit the
// registers of a wave without spilling.
constexpr int ws_max_steps(int cb) { return cb == 1 ? 24 : cb == 2 ? 16 : 8; }

// Kernel-variant families (dtype x operand gathering x epilogue).
enum Variant {
  VAR_F32 = 0,          // fp32 activations, 4-channel chunks, SiLU epilogue
  VAR_I8_C16 = 1,       // int8, 16-channel chunks (C_in_pad % 16 == 0), dequant+SiLU
  VAR_I8_C4 = 2,        // int8, 4-channel chunks (any C_in_pad % 4 == 0), dequant+SiLU
  VAR_I8_C16_RAW = 3,   // as VAR_I8_C16, stores raw int32 accumulators
  VAR_I8_C4_RAW = 4,    // as VAR_I8_C4, stores raw int32 accumulators
  // the same three with the general epilogue: identity activation, residual,
  // int8 output (runtime, wave-uniform); the plain ones above keep the short
  // SiLU + fp32 store, so the common case executes no extra instructions
  VAR_F32_X = 5,
  VAR_I8_C16_X = 6,
  VAR_I8_C4_X = 7,
  // asymmetric uint8 activations: codes are gathered as q ^ 0x80 = q - 128
  // (signed) and every accumulator starts at the zero-point correction of its
  // pixel's border class; general epilogue, or raw int32 accumulators
  VAR_U8_C16_X = 8,
  VAR_U8_C4_X = 9,
  VAR_U8_C16_RAW = 10,
  VAR_U8_C4_RAW = 11,
  VAR_COUNT = 12
};

// Everything a launch needs; filled at create, passed by value.
// Epilogue activation codes (ConvParams::act).
enum Act { ACT_SILU = 0, ACT_NONE = 1 };

// Division by a run-time constant d >= 1, for numerators below 2^31, with one
// multiply-high, an add and a shift (Granlund and Montgomery, "Division by
// invariant integers using multiplication", PLDI 1994, Figure 4.1): with
// l = ceil(log2 d) and magic = floor(2^32 (2^l - d) / d) + 1,
//   n / d = (mulhi(n, magic) + n) >> l,
// where the sum stays below 2^32 because n < 2^31.  Set up on the host.
struct FastDiv {
  unsigned magic;
  int shift;
};

// Fields are grouped by the kernels that read them (all kernels, then the
// pixel-tiled ones, split-K, the halo kernel, host-only), so the kernels'
// wide scalar loads of the argument block fetch few unused words.
struct ConvParams {
  // ---- every kernel
  const void *x;         // NHWC input, first channel of the layer: pixel i at x + i*x_cs
  const void *wfrag;     // weights in MFMA fragment order [co_blocks][steps][64 lanes][16 bytes]
  const float *bias;     // folded bias [co_blocks*16] (zero beyond C_out)
  const float *dq;       // INT8 dequant factors f[co] [co_blocks*16] (null for fp32)
  void *out;             // NHWC output, first channel of the layer: pixel (n,oh,ow) at
                         // out + ((n*OH + oh)*pitch + ow)*out_cs  (fp32, int8, or int32 for raw)
  const void *res;       // residual, first channel: logical pixel m at res + m*res_cs (null if none)
  const int *corr;       // uint8 input: accumulator start values [64 border classes][co_blocks*16]
  int H, W;
  int x_cs;              // input elements between consecutive pixels (cin_pad when dense)
  int k, stride, pad;
  int chunk_ch;          // channels per chunk (4 or 16)
  int chunks_per_tap;    // cin_pad / chunk_ch
  unsigned cpt_magic;    // chunk / chunks_per_tap == (chunk * cpt_magic) >> 20 for the chunks in use
  int total_chunks;      // k*k*chunks_per_tap
  int steps;             // K steps (each 16 fp32 or 64 int8 channels of K)
  int co_blocks;         // 16-channel output blocks holding real channels
  unsigned x_bytes;      // bytes of the input buffer from x (buffer-load range)
  unsigned w_bytes;      // bytes of the fragment-ordered weights (buffer-load range)
  int OH, OW, cout_pad, pitch;
  int out_cs;            // output elements between consecutive pixels (cout_pad when dense)
  int res_cs;            // residual elements between consecutive pixels (0: no residual)
  unsigned res_bytes;    // bytes of the residual buffer from res (buffer-load range)
  unsigned out_bytes;    // bytes of the output buffer from out (buffer-store range)
  int act;               // Act
  int out_q;             // 1: byte output codes q = clamp(rne(fp32(y / out_scale)) + out_zp, out_lo, out_hi)
  float out_scale;       // s_y for byte output
  float out_rcp;         // RN(1/s_y), the correctly rounded fp32 reciprocal
  float out_zp;          // output zero point (0 for int8 codes)
  float out_lo, out_hi;  // code range: -127, 127 (int8) or 0, 255 (uint8)
  float res_scale;       // scale of byte residual codes
  unsigned res_xor;      // byte residual decode, per byte: value = float(byte ^ res_xor) - res_zp,
  float res_zp;          //   with 0x80808080 and 128 for int8 codes, 0 and the zero point for uint8
  // ---- pixel-tiled kernels (conv_igemm, conv_lds)
  int M;                 // N*OH*OW output pixels
  int inner_tiles;       // tiles along the inner dimension of the workgroup order
  int px_inner;          // 1: pixel tiles inner (channel-major order), 0: channel tiles inner
  FastDiv div_ow, div_oh;    // by OW and OH: pixel index -> (n, oh, ow)
  FastDiv div_inner;         // by inner_tiles: workgroup -> (outer tile, inner tile)
  int run_base, run_rem;     // conv_ws: run t holds 16-pixel blocks [t*run_base + min(t, run_rem), +run_base + (t < run_rem))
  const void *x2;            // conv_ws 1x1: second input, channels c1 .. C_in - 1 (null: none)
  int x2_cs;                 // its elements between consecutive pixels
  unsigned x2_bytes;         // bytes of its buffer (buffer-load range)
  int c1;                    // channels from the first input (a multiple of 16)
  // ---- cross-workgroup split-K (conv_igemm)
  float *ws;             // split-K partial tiles (null when splitk == 1)
  unsigned *counters;    // split-K arrival counters, one per output tile (zero between launches)
  int splitk;            // workgroups per output tile along K
  int steps_per_split;   // K steps per split-K workgroup
  FastDiv div_sk;            // by splitk
  // ---- conv_halo
  int cin_pad;
  int tiles_x, tiles_y;  // output tiles along a row and along the rows of one image
  int halo_bytes;        // LDS bytes of the input halo tile (weights follow)
  int halo_cq;           // 4-channel slots per pixel in LDS (padded, see halo_lds)
  FastDiv div_tx, div_ty;    // by tiles_x and tiles_y
  FastDiv div_hcq, div_hwd;  // by halo_cq and by the halo width in pixels
  // ---- host only
  int N;
  int px_tiles;          // workgroup tiles along pixels
  int co_tiles;          // workgroup tiles along output channels
  int smem_bytes;        // conv_halo: dynamic LDS bytes per workgroup
};

// Arguments of one grouped launch (conv_igemm_group): up to kGroupMax
// independent layers of one kernel variant, run with one register-direct
// configuration.  p must stay the first member: the kernel reads p[i] from the
// start of its argument segment.
constexpr int kGroupMax = 4;
struct GroupArgs {
  ConvParams p[kGroupMax];
  int first[kGroupMax];  // first logical workgroup of each member (first[0] = 0; INT_MAX for unused slots)
};
static_assert(offsetof(GroupArgs, p) == 0, "member parameters must start the argument segment");
static_assert(sizeof(GroupArgs) <= 4096, "kernel arguments above 4 KB");

int num_configs();
const KernelConfig &config(int i);
// Launch variant `var` with configuration `cfg`; returns the hipError_t of the launch.
hipError_t launch_conv(int var, int cfg, const ConvParams &p, hipStream_t stream);
// One per variant (cbs_variant.hip compiled with -DCBS_VAR=n).
hipError_t launch_var_0(int cfg, const ConvParams &p, hipStream_t stream);
hipError_t launch_var_1(int cfg, const ConvParams &p, hipStream_t stream);
hipError_t launch_var_2(int cfg, const ConvParams &p, hipStream_t stream);
hipError_t launch_var_3(int cfg, const ConvParams &p, hipStream_t stream);
hipError_t launch_var_4(int cfg, const ConvParams &p, hipStream_t stream);
hipError_t launch_var_5(int cfg, const ConvParams &p, hipStream_t stream);
hipError_t launch_var_6(int cfg, const ConvParams &p, hipStream_t stream);
hipError_t launch_var_7(int cfg, const ConvParams &p, hipStream_t stream);
hipError_t launch_var_8(int cfg, const ConvParams &p, hipStream_t stream);
hipError_t launch_var_9(int cfg, const ConvParams &p, hipStream_t stream);
hipError_t launch_var_10(int cfg, const ConvParams &p, hipStream_t stream);
hipError_t launch_var_11(int cfg, const ConvParams &p, hipStream_t stream);
// Grouped launch of variant `var` with register-direct configuration `cfg` over
// `grid` workgroups (the members' grids end to end).  RAW variants have none.
hipError_t launch_conv_group(int var, int cfg, const GroupArgs &g, unsigned grid, hipStream_t stream);
hipError_t launch_group_var_0(int cfg, const GroupArgs &g, unsigned grid, hipStream_t stream);
hipError_t launch_group_var_1(int cfg, const GroupArgs &g, unsigned grid, hipStream_t stream);
hipError_t launch_group_var_2(int cfg, const GroupArgs &g, unsigned grid, hipStream_t stream);
hipError_t launch_group_var_5(int cfg, const GroupArgs &g, unsigned grid, hipStream_t stream);
hipError_t launch_group_var_6(int cfg, const GroupArgs &g, unsigned grid, hipStream_t stream);
hipError_t launch_group_var_7(int cfg, const GroupArgs &g, unsigned grid, hipStream_t stream);
hipError_t launch_group_var_8(int cfg, const GroupArgs &g, unsigned grid, hipStream_t stream);
hipError_t launch_group_var_9(int cfg, const GroupArgs &g, unsigned grid, hipStream_t stream);

hipError_t launch_pack_nhwc_f32(const float *x, float *y, int n, int c, int hw, int c_pad,
                                hipStream_t stream);
hipError_t launch_quantize_nhwc_i8(const float *x, int8_t *y, float s_x, int n, int c, int hw,
                                   int c_pad, hipStream_t stream);
hipError_t launch_quantize_nhwc_u8(const float *x, uint8_t *y, float s_x, int z, int n, int c, int hw,
                                   int c_pad, hipStream_t stream);

}  // namespace cbs
