// cbs_host.cpp -- host side of libcbs: descriptor validation, batch-norm
// folding, weight re-layout into MFMA fragment order, per-channel int8 weight
// quantisation, per-shape kernel selection, device memory, launches, layer
// lists and graph capture.  The public contract is include/cbs.h.
//
// Folding and quantisation follow the vision-rs "YOLO26N Inference
// Optimisation" page (section "Baseline benchmark": BN folded into the
// weights at load; section "NHWC migration -- Weight layout": a one-time
// re-layout of the OIHW weights at load so that C_in is contiguous along K)
// and the edge-optimization README ("Highlights", "Design notes": one
// symmetric int8 scale per output channel).  The arithmetic is in double and
// this file is compiled with -ffp-contract=off, so every product and sum is
// rounded exactly as written.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <string>
#include <tuple>
#include <vector>

#include "../../include/cbs.h"
#include "cbs_internal.h"
#include "cbs_scratch.h"

using namespace cbs;

namespace {

thread_local std::string g_last_error;

cbs_status fail(cbs_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

inline int round_up(int v, int m) { return (v + m - 1) / m * m; }
inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

int out_dim(int in, int k, int s, int p) {
  if (in + 2 * p < k) return 0;
  return (in + 2 * p - k) / s + 1;
}

#include "tile_table.inc"

}  // namespace

struct cbs_layer {
  cbs_conv_desc d;
  int oh, ow, pitch, cin_pad, cout_pad, co_blocks, M;
  int in_cs, out_cs, res_cs;  // channel strides of input, output, residual (res_cs 0: none)
  int in2_ch = 0, in2_cs = 0;  // second input: its channels (the last of C_in; 0: none) and pixel stride
  int variant;       // fused-epilogue variant
  int raw_variant;   // raw-accumulator variant (INT8), -1 for fp32
  int chunk_ch, chunks_per_tap, total_chunks, steps;
  unsigned cpt_magic;
  int config, splitk;
  int device;
  int cus = 256;     // compute units of the device (sizes the conv_ws grid)
  int lds_max = 65536;  // LDS bytes a workgroup may use on the device (bounds the halo tiles)
  // device memory
  void *d_wfrag = nullptr;
  float *d_bias = nullptr;
  float *d_dq = nullptr;
  int *d_corr = nullptr;   // uint8 input: accumulator start values [64][co_blocks*16]
  // column-pair halo tiles (3x3 stride 1, <= 8 output channels; see conv_halo):
  // weights over the 3 x 4 window of a pixel pair and a 16-row bias/dequant
  bool pair = false;
  int pair_total_chunks = 0, pair_steps = 0;
  void *d_wfrag_pair = nullptr;
  float *d_bias_pair = nullptr;
  float *d_dq_pair = nullptr;
  // Cross-workgroup split-K partial tiles and arrival counters.  A captured
  // graph holds these addresses in its kernel arguments, so they never move
  // while a graph references the layer (graph_refs > 0): a configuration that
  // needs more than the current capacity is then refused instead of
  // reallocating.  Counters are zero between launches (each tile's last
  // workgroup re-arms its own).
  float *d_ws = nullptr;
  unsigned *d_counters = nullptr;
  size_t ws_bytes = 0, counters_len = 0;  // in use by the current configuration
  size_t ws_cap = 0, counters_cap = 0;    // allocated
  mutable std::atomic<int> graph_refs{0};
  // host copies for the test hooks
  std::vector<float> h_wfold;   // fp32 W' OIHW
  std::vector<float> h_bias;    // fp32 b'
  std::vector<int8_t> h_qw;     // int8 q_w OIHW
  std::vector<double> h_sw;     // s_w
};

// Per candidate group of cbs_graph_create_grouped: what was measured and kept.
struct GraphGroup {
  int id = -1, members = 0, kept = 0, config = -1;
  float us_grouped = 0.f, us_separate = 0.f;
};

struct cbs_graph {
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  std::vector<const cbs_layer *> layers;  // each holds one graph reference (see cbs_layer::graph_refs)
  std::vector<cbs_group *> groups;        // grouped launches owned by the graph
  std::vector<GraphGroup> group_info;
  int launches = 0;
};

// Independent layers run by one grouped launch.  The members are kept in
// grid order (the caller's index of each in `slot`); all share one kernel
// variant and one register-direct configuration.  Each member has its own
// cross-workgroup split-K factor, which evens out the K depth of the
// members' workgroups, with the group's own partial-tile workspace and
// arrival counters.
static_assert(cbs::kGroupMax == CBS_GROUP_MAX, "group size limit differs from the header's");
struct cbs_group {
  int n = 0;
  int config = 0;
  int variant = 0;
  const cbs_layer *member[cbs::kGroupMax] = {};
  int slot[cbs::kGroupMax] = {};
  int splitk[cbs::kGroupMax] = {};
  float *d_ws[cbs::kGroupMax] = {};
  unsigned *d_counters[cbs::kGroupMax] = {};
};

namespace {

// --------------------------------------------------------------- shapes --

cbs_status validate(const cbs_conv_desc *d) {
  if (!d) return fail(CBS_EINVAL, "desc is NULL");
  if (d->n < 1 || d->c_in < 1 || d->h < 1 || d->w < 1 || d->c_out < 1)
    return fail(CBS_EINVAL, "n, c_in, h, w, c_out must be >= 1 (got %d %d %d %d %d)", d->n, d->c_in,
                d->h, d->w, d->c_out);
  if (d->k != 1 && d->k != 3) return fail(CBS_EUNSUPPORTED, "kernel size %d not in {1,3}", d->k);
  if (d->stride != 1 && d->stride != 2) return fail(CBS_EUNSUPPORTED, "stride %d not in {1,2}", d->stride);
  if (d->pad < 0 || d->pad > d->k / 2) return fail(CBS_EUNSUPPORTED, "pad %d not in [0, k/2]", d->pad);
  if (d->dtype != CBS_F32 && d->dtype != CBS_I8 && d->dtype != CBS_U8)
    return fail(CBS_EINVAL, "dtype %d unknown", d->dtype);
  if (d->dtype != CBS_F32 && !(d->in_scale > 0.0f && std::isfinite(d->in_scale)))
    return fail(CBS_EINVAL, "INT8 layer needs a finite in_scale > 0");
  if (!(d->bn_eps >= 0.0f) || !std::isfinite(d->bn_eps)) return fail(CBS_EINVAL, "bn_eps must be finite and >= 0");
  if (d->c_in > 4096 || d->c_out > 4096) return fail(CBS_EUNSUPPORTED, "channels above 4096");
  if (d->act != CBS_ACT_SILU && d->act != CBS_ACT_NONE) return fail(CBS_EINVAL, "act %d unknown", d->act);
  if (d->out_dtype != CBS_F32 && d->out_dtype != CBS_I8 && d->out_dtype != CBS_U8)
    return fail(CBS_EINVAL, "out_dtype %d unknown", d->out_dtype);
  if (d->out_dtype != CBS_F32 && !(d->out_scale > 0.0f && std::isfinite(d->out_scale)))
    return fail(CBS_EINVAL, "byte output needs a finite out_scale > 0");
  // zero points: in [0, 255] for uint8 tensors, 0 for every other dtype
  struct Zp {
    const char *what;
    int value;
    bool u8;
  } zps[3] = {{"in_zero_point", d->in_zero_point, d->dtype == CBS_U8},
              {"out_zero_point", d->out_zero_point, d->out_dtype == CBS_U8},
              {"res_zero_point", d->res_zero_point, d->out_dtype == CBS_U8 && d->res_c_stride > 0}};
  for (const Zp &z : zps) {
    if (z.u8 && (z.value < 0 || z.value > 255)) return fail(CBS_EINVAL, "%s %d not in [0, 255]", z.what, z.value);
    if (!z.u8 && z.value != 0) return fail(CBS_EINVAL, "%s %d set for a tensor that is not uint8", z.what, z.value);
  }
  const int oh = out_dim(d->h, d->k, d->stride, d->pad), ow = out_dim(d->w, d->k, d->stride, d->pad);
  if (oh < 1 || ow < 1) return fail(CBS_EINVAL, "empty output (%dx%d)", oh, ow);
  if (d->out_row_pitch != 0 && d->out_row_pitch < ow)
    return fail(CBS_EINVAL, "out_row_pitch %d < OW %d", d->out_row_pitch, ow);
  // channel slices: (stride 0, offset 0) is the dense layout; a slice needs
  // 4-aligned channel counts, offsets and strides, and must fit in the pixel
  struct Slice {
    const char *what;
    int stride, offset, channels;
  } slices[3] = {{"in", d->in_c_stride, d->in_c_offset, d->c_in - d->in2_channels},
                 {"out", d->out_c_stride, d->out_c_offset, d->c_out},
                 {"res", d->res_c_stride, d->res_c_offset, d->c_out}};
  for (const Slice &sl : slices) {
    if (sl.stride < 0 || sl.offset < 0)
      return fail(CBS_EINVAL, "%s_c_stride / %s_c_offset must be >= 0", sl.what, sl.what);
    if (sl.stride == 0) {
      if (sl.offset != 0) return fail(CBS_EINVAL, "%s_c_offset %d needs %s_c_stride > 0", sl.what, sl.offset, sl.what);
      continue;
    }
    if (sl.channels % 4 || sl.offset % 4 || sl.stride % 4)
      return fail(CBS_EINVAL, "%s slice: channels %d, offset %d and stride %d must be multiples of 4", sl.what,
                  sl.channels, sl.offset, sl.stride);
    if (sl.offset + sl.channels > sl.stride)
      return fail(CBS_EINVAL, "%s slice: offset %d + channels %d > stride %d", sl.what, sl.offset, sl.channels,
                  sl.stride);
  }
  if (d->res_c_stride > 0 && d->out_dtype != CBS_F32 && !(d->res_scale > 0.0f && std::isfinite(d->res_scale)))
    return fail(CBS_EINVAL, "byte residual needs a finite res_scale > 0");
  // second input: the last in2_channels of C_in, from a tensor of its own
  if (d->in2_channels < 0 || d->in2_c_stride < 0) return fail(CBS_EINVAL, "in2_channels / in2_c_stride must be >= 0");
  if (d->in2_channels == 0 && d->in2_c_stride != 0) return fail(CBS_EINVAL, "in2_c_stride set without in2_channels");
  if (d->in2_channels > 0) {
    if (d->dtype != CBS_F32 || d->k != 1 || d->stride != 1 || d->pad != 0)
      return fail(CBS_EUNSUPPORTED, "a second input needs an fp32 1x1 stride-1 layer");
    const int c1 = d->c_in - d->in2_channels;
    if (c1 < 16 || c1 % 16)
      return fail(CBS_EUNSUPPORTED, "with a second input the first supplies a positive multiple of 16 channels "
                                    "(got %d of %d)", c1, d->c_in);
    const int s2 = d->in2_c_stride ? d->in2_c_stride : round_up(d->in2_channels, 4);
    if (d->in2_channels % 4 || s2 % 4 || s2 < d->in2_channels)
      return fail(CBS_EINVAL, "second input: channels %d and stride %d must be multiples of 4, stride >= channels",
                  d->in2_channels, s2);
    if ((double)d->n * d->h * d->w * s2 * 4.0 >= 2147483648.0 - 64.0)
      return fail(CBS_EUNSUPPORTED, "second input above 2^31 bytes");
  }
  const int pitch = d->out_row_pitch ? d->out_row_pitch : ow;
  const int in_cs = d->in_c_stride ? d->in_c_stride : round_up(d->c_in - d->in2_channels, 4);
  const int out_cs = d->out_c_stride ? d->out_c_stride : round_up(d->c_out, 4);
  const double in_elems = (double)d->n * d->h * d->w * in_cs;
  const double out_elems = (double)d->n * oh * pitch * out_cs;
  const double res_elems = (double)d->n * oh * ow * d->res_c_stride;
  if (in_elems >= 2147483647.0 || out_elems >= 2147483647.0 || res_elems >= 2147483647.0)
    return fail(CBS_EUNSUPPORTED, "tensor above 2^31 elements");
  // the kernels address input and residual with 32-bit buffer offsets below 2^31
  const double in_bytes = in_elems * (d->dtype == CBS_F32 ? 4.0 : 1.0);
  const double res_bytes = res_elems * (d->out_dtype == CBS_F32 ? 4.0 : 1.0);
  const double out_bytes = out_elems * (d->out_dtype == CBS_F32 ? 4.0 : 1.0);
  if (in_bytes >= 2147483648.0 - 64.0) return fail(CBS_EUNSUPPORTED, "input above 2^31 bytes");
  if (out_bytes >= 2147483648.0 - 64.0) return fail(CBS_EUNSUPPORTED, "output above 2^31 bytes");
  if (res_bytes >= 2147483648.0 - 64.0) return fail(CBS_EUNSUPPORTED, "residual above 2^31 bytes");
  return CBS_OK;
}

// ------------------------------------------------------ kernel selection --

struct Choice {
  int config, splitk;
};

// Tiles of a configuration for this layer.
void tiles_of(const cbs_layer *L, int cfg, int *px_tiles, int *co_tiles) {
  const KernelConfig &c = config(cfg);
  if (c.lds == 2 || c.lds == 3) {  // halo tiles: whole TH x TW blocks of one image, all channels
    *co_tiles = 1;
    *px_tiles = L->d.n * ceil_div(L->oh, c.th) * ceil_div(L->ow, c.lds == 3 ? 2 * c.tw : c.tw);
    return;
  }
  if (c.lds == 4 || c.lds == 5) {  // conv_ws: channel groups x runs of 16-pixel blocks, about th workgroups per CU
    *co_tiles = ceil_div(L->co_blocks, c.cb * c.wco);
    const int blocks = ceil_div(L->M, 16);
    *px_tiles = std::max(1, std::min(blocks, (L->cus * c.th + *co_tiles / 2) / *co_tiles));
    return;
  }
  const int tco = c.cb * 16 * c.wco, tpx = c.pb * 16 * c.wpx;
  *co_tiles = ceil_div(L->co_blocks * 16, tco);
  *px_tiles = ceil_div(L->M, tpx);
}

// LDS bytes of a halo-tile workgroup: the input window (4-channel slots,
// rounded up to whole waves of slots) followed by all fragment-ordered weights.
// 4-channel slots per halo pixel in LDS: fp32 pixels of an even number of
// 16-byte slots get one zero slot more, so that the 16 pixels a fragment read
// touches (consecutive, or every other one for stride 2) fall on distinct LDS
// banks.
int halo_cq(const cbs_layer *L) {
  const int cq = L->cin_pad / 4;
  return (L->d.dtype == CBS_F32 && cq % 2 == 0) ? cq + 1 : cq;
}

// Halo width in pixels of a halo configuration (column pairs: 2*tw pixels
// at stride 1 plus the 3x3 border).
int halo_width(const cbs_layer *L, const KernelConfig &c) {
  return c.lds == 3 ? 2 * c.tw + 2 : (c.tw - 1) * L->d.stride + 3;
}

void halo_lds(const cbs_layer *L, int cfg, int *halo_bytes, int *smem_bytes) {
  const KernelConfig &c = config(cfg);
  const int s = L->d.stride;
  const int hh = (c.th - 1) * s + 3, hw = halo_width(L, c);
  const int slots = hh * hw * halo_cq(L);
  const int slot_bytes = L->d.dtype == CBS_F32 ? 16 : 4;
  *halo_bytes = round_up(slots, 64) * slot_bytes;
  *smem_bytes = *halo_bytes + (c.lds == 3 ? L->pair_steps : L->co_blocks * L->steps) * 1024;
}

// Rough cost model (cycles at one SIMD) used when the tile table has no entry:
// waves are spread over 1024 SIMDs, each wave runs its K slice on MFMA with a
// fixed per-wave overhead, split-K adds a publish/reduce phase.
double model_cost(const cbs_layer *L, int cfg, int splitk) {
  const KernelConfig &c = config(cfg);
  int pxt, cot;
  tiles_of(L, cfg, &pxt, &cot);
  const int kslices = splitk * c.wk;
  const double steps_per_wave = std::ceil((double)L->steps / kslices);
  const double mfma_step = L->d.dtype == CBS_F32 ? 4 * 32.0 : 16.0;
  const double load_step = 40.0 * (c.cb + c.pb);
  const double per_wave = steps_per_wave * std::max(mfma_step * c.cb * c.pb, load_step) + 1500.0;
  const double waves = (double)pxt * cot * splitk * c.wco * c.wpx * c.wk;
  const double rounds = std::ceil(waves / 1024.0);
  double cost = rounds * per_wave;
  if (splitk > 1) cost += 2500.0;
  // L2 -> CU traffic (bytes) against ~8 KB/cycle aggregate
  const double esz = L->d.dtype == CBS_F32 ? 4.0 : 1.0;
  const double kbytes = (double)L->steps * (L->d.dtype == CBS_F32 ? 16 : 64) * esz;
  const double traffic = kbytes * ((double)L->M * cot + (double)L->co_blocks * 16 * pxt);
  cost = std::max(cost, traffic / 8192.0);
  return cost;
}

bool config_fits(const cbs_layer *L, int cfg, int splitk) {
  const KernelConfig &c = config(cfg);
  if (splitk < 1 || splitk > 64) return false;
  if (c.lds && splitk != 1) return false;
  if (L->in2_ch && (c.lds != 4 || !(L->steps == 2 || L->steps == 3 || L->steps == 6 || L->steps == 12 ||
                                      L->steps == 24)))
    return false;  // a second input: weight-stationary 1x1 tiles, at the depths compiled for it
  if (c.lds == 4) {  // conv_ws: 1x1 stride 1, K steps (the last one may be partial) of the compiled depths
    if (L->d.k != 1 || L->d.stride != 1 || L->d.pad != 0) return false;
    const int ks = L->steps;
    // chunks per K step: 4 (fp32, or int8 with 16-channel chunks), 16 (int8 with 4-channel chunks)
    const int per_step = (L->d.dtype != CBS_F32 && L->chunk_ch == 4) ? 16 : 4;
    const bool partial = L->total_chunks < per_step * ks;
    if (partial && ks > 3) return false;  // partial last steps compiled for depths 1-3
    if (L->d.dtype == CBS_F32) {
      if (!(ks == 1 || ks == 2 || ks == 3 || ks == 4 || ks == 6 || ks == 8 || ks == 12 || ks == 16 || ks == 24))
        return false;
    } else {  // int8 and uint8: 64-channel K steps, depths 1-4 and 6
      if (!(ks == 1 || ks == 2 || ks == 3 || ks == 4 || ks == 6)) return false;
    }
    if (ks > ws_max_steps(c.cb)) return false;  // deepest K the launcher instantiates
  }
  if (c.lds == 5) {  // conv_ws with the window gather: fp32 3x3, K steps each within one tap, depths 9 and 18
    if (L->d.dtype != CBS_F32 || L->d.k != 3 || L->chunks_per_tap % 4 != 0) return false;
    if (!(L->steps == 9 || L->steps == 18)) return false;
    // its pixel arithmetic multiplies in 24 bits: pixel indices and strides below 2^23
    const int64_t lim = int64_t(1) << 23;
    if ((int64_t)L->d.n * L->d.h * L->d.w >= lim || (int64_t)L->d.n * L->oh >= lim || L->pitch >= lim ||
        L->in_cs >= lim)
      return false;
  }
  if (c.lds == 2 || c.lds == 3) {
    if (L->d.k != 3 || L->co_blocks > 4) return false;
    if (c.lds == 3 && !L->pair) return false;
    int hb, sb;
    halo_lds(L, cfg, &hb, &sb);
    if (sb > L->lds_max) return false;  // 160 KiB on gfx950
  }
  if (splitk > 1 && L->steps < splitk * c.wk) return false;
  int pxt, cot;
  tiles_of(L, cfg, &pxt, &cot);
  const double grid = (double)pxt * cot * splitk;
  return grid < 2147483647.0;
}

// Tile-table class of a layer (TileEntry::dtype): 0 fp32 and 1 int8 input
// with the plain epilogue (SiLU, fp32 output, no residual), 2 uint8 input,
// 3 int8 and 4 fp32 input with the general epilogue (byte output, identity
// activation or a residual).  Classes 2-4 fall back to the plain entry of
// their input type (uint8 layers run the int8 kernels with another gather and
// start value), which the sweep writes for every shape.
int table_class(const cbs_layer *L) {
  if (L->d.dtype == CBS_U8) return 2;
  const bool x = L->variant == VAR_F32_X || L->variant == VAR_I8_C16_X || L->variant == VAR_I8_C4_X;
  if (L->d.dtype == CBS_F32) return x ? 4 : 0;
  return x ? 3 : 1;
}

Choice choose(const cbs_layer *L) {
  // 1) the offline-tuned table: the entry of the layer's own class, else the
  // plain entry of its input type
  const int cls = table_class(L);
  const int fallback = (cls == 0 || cls == 4) ? 0 : 1;
  for (int key : {cls, fallback}) {
    for (const TileEntry &e : kTileTable) {
      if (e.n == L->d.n && e.c_in == L->d.c_in && e.c_out == L->d.c_out && e.h == L->d.h &&
          e.w == L->d.w && e.k == L->d.k && e.s == L->d.stride && e.dtype == key &&
          e.config < num_configs() && config_fits(L, e.config, e.splitk))
        return {e.config, e.splitk};
    }
  }
  // a second input runs on the weight-stationary 1x1 tiles only: the one whose
  // workgroup covers the fewest channel blocks at or above the layer's, else the widest
  if (L->in2_ch) {
    int pick = -1, pick_cov = 0;
    for (int cfg = 0; cfg < num_configs(); cfg++) {
      const KernelConfig &c = config(cfg);
      if (c.lds != 4 || !config_fits(L, cfg, 1)) continue;
      const int cov = c.cb * c.wco, need = L->co_blocks;
      const bool better = pick < 0 || (cov >= need && (pick_cov < need || cov < pick_cov)) ||
                          (cov < need && pick_cov < need && cov > pick_cov);
      if (better) pick = cfg, pick_cov = cov;
    }
    if (pick >= 0) return {pick, 1};
  }
  // 2) the cost model.  Cross-workgroup split-K is never picked here: its
  // partial-tile round trip through memory costs about a microsecond per
  // launch, which only a measurement can weigh against the better balance;
  // only the measured table (or the create-time tuner) may select it.
  Choice best{2, 1};
  double best_cost = 1e300;
  for (int cfg = 0; cfg < num_configs(); cfg++) {
    if (config(cfg).lds >= 2) continue;  // halo and weight-stationary tiles are chosen by measurement only
    for (int sk : {1}) {
      if (!config_fits(L, cfg, sk)) continue;
      const double cost = model_cost(L, cfg, sk);
      if (cost < best_cost * 0.999) {
        best_cost = cost;
        best = {cfg, sk};
      }
    }
  }
  return best;
}

// ----------------------------------------------------------- device side --

cbs_status dev_alloc(void **p, size_t bytes) {
  *p = nullptr;
  if (bytes == 0) return CBS_OK;
  hipError_t e = hipMalloc(p, bytes);
  if (e != hipSuccess) {
    *p = nullptr;
    return fail(CBS_ENOMEM, "hipMalloc(%zu): %s", bytes, hipGetErrorString(e));
  }
  return CBS_OK;
}

void release(cbs_layer *L) {
  if (!L) return;
  if (L->d_wfrag) (void)hipFree(L->d_wfrag);
  if (L->d_bias) (void)hipFree(L->d_bias);
  if (L->d_dq) (void)hipFree(L->d_dq);
  if (L->d_corr) (void)hipFree(L->d_corr);
  if (L->d_wfrag_pair) (void)hipFree(L->d_wfrag_pair);
  if (L->d_bias_pair) (void)hipFree(L->d_bias_pair);
  if (L->d_dq_pair) (void)hipFree(L->d_dq_pair);
  L->d_wfrag_pair = nullptr;
  L->d_bias_pair = L->d_dq_pair = nullptr;
  if (L->d_ws) (void)hipFree(L->d_ws);
  if (L->d_counters) (void)hipFree(L->d_counters);
  L->d_wfrag = nullptr;
  L->d_bias = L->d_dq = L->d_ws = nullptr;
  L->d_corr = nullptr;
  L->d_counters = nullptr;
  L->ws_cap = L->counters_cap = 0;
}

// Partial-tile bytes and arrival counters that configuration cfg with a
// cross-workgroup split of splitk needs for layer L (both 0 without a split).
void splitk_need(const cbs_layer *L, int cfg, int splitk, size_t *ws_bytes, size_t *counters) {
  *ws_bytes = 0;
  *counters = 0;
  if (splitk <= 1) return;
  const KernelConfig &c = config(cfg);
  int pxt, cot;
  tiles_of(L, cfg, &pxt, &cot);
  const size_t tiles = (size_t)pxt * cot;
  const size_t tile_vecs = (size_t)c.wco * c.wpx * c.cb * c.pb * 64;
  *ws_bytes = tiles * splitk * tile_vecs * 16;
  *counters = tiles;
}

// Whether the layer's current workspace already holds what (cfg, splitk) needs.
bool splitk_fits_workspace(const cbs_layer *L, int cfg, int splitk) {
  size_t ws, cnt;
  splitk_need(L, cfg, splitk, &ws, &cnt);
  return ws <= L->ws_cap && cnt <= L->counters_cap;
}

// Make the split-K workspace and the zeroed arrival counters hold what the
// layer's current configuration needs.  Runs at create, set_config and
// autotune only.  The workspace only grows, and only while no graph holds
// its address.
cbs_status setup_splitk(cbs_layer *L) {
  size_t ws, cnt;
  splitk_need(L, L->config, L->splitk, &ws, &cnt);
  if (ws <= L->ws_cap && cnt <= L->counters_cap) {
    L->ws_bytes = ws;
    L->counters_len = cnt;
    return CBS_OK;
  }
  if (L->graph_refs.load() > 0)
    return fail(CBS_EINVAL, "configuration %s with split-K %d needs a larger split-K workspace than the "
                            "layer holds, and a live graph holds the current one's address; destroy the "
                            "graph first", config(L->config).name, L->splitk);
  if (L->d_ws) (void)hipFree(L->d_ws);
  if (L->d_counters) (void)hipFree(L->d_counters);
  L->d_ws = nullptr;
  L->d_counters = nullptr;
  L->ws_cap = L->counters_cap = 0;
  L->ws_bytes = L->counters_len = 0;
  cbs_status st = dev_alloc((void **)&L->d_ws, ws);
  if (st != CBS_OK) return st;
  st = dev_alloc((void **)&L->d_counters, cnt * sizeof(unsigned));
  if (st != CBS_OK) return st;
  hipError_t e = hipMemset(L->d_counters, 0, cnt * sizeof(unsigned));
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) return fail(CBS_EDEVICE, "counter init: %s", hipGetErrorString(e));
  L->ws_cap = L->ws_bytes = ws;
  L->counters_cap = L->counters_len = cnt;
  return CBS_OK;
}

// Kernel arguments of one launch.  raw: the INT8 test hook, which stores
// int32 accumulators densely ([N][OH][pitch][C_out_pad]) with no epilogue.
// Multiply-shift divisor for d >= 1 (numerators below 2^31; see FastDiv).
FastDiv make_fastdiv(int d) {
  if (d < 1) d = 1;
  int l = 0;
  while ((1ull << l) < (unsigned long long)d) l++;
  FastDiv f;
  f.magic = (unsigned)(((1ull << 32) * ((1ull << l) - (unsigned long long)d)) / (unsigned long long)d + 1ull);
  f.shift = l;
  return f;
}

// Kernel arguments of one launch of layer L with configuration cfg and split-K
// factor splitk (the layer's own, or a group's).
ConvParams make_params(const cbs_layer *L, const void *in, void *out, const void *res, bool raw, int cfg,
                       int splitk, const void *in2 = nullptr) {
  ConvParams p;
  std::memset(&p, 0, sizeof(p));
  const size_t esz_in = L->d.dtype == CBS_F32 ? 4 : 1;
  const size_t esz_out = (raw || L->d.out_dtype == CBS_F32) ? 4 : 1;
  p.x = (const char *)in + (size_t)L->d.in_c_offset * esz_in;
  p.x_cs = L->in_cs;
  p.x_bytes = (unsigned)((size_t)L->d.n * L->d.h * L->d.w * L->in_cs * esz_in - (size_t)L->d.in_c_offset * esz_in);
  if (L->in2_ch) {  // second input (fp32): channels c1 .. C_in - 1
    p.x2 = in2;
    p.x2_cs = L->in2_cs;
    p.x2_bytes = (unsigned)((size_t)L->d.n * L->d.h * L->d.w * L->in2_cs * 4);
    p.c1 = L->d.c_in - L->in2_ch;
  }
  p.wfrag = L->d_wfrag;
  p.bias = L->d_bias;
  p.dq = L->d_dq;
  p.corr = L->d_corr;
  if (raw) {
    p.out = out;
    p.out_cs = L->cout_pad;
    p.out_bytes = (unsigned)((size_t)L->d.n * L->oh * L->pitch * L->cout_pad * 4);
  } else {
    p.out = (char *)out + (size_t)L->d.out_c_offset * esz_out;
    p.out_cs = L->out_cs;
    p.out_bytes = (unsigned)(((size_t)L->d.n * L->oh * L->pitch * L->out_cs - (size_t)L->d.out_c_offset) * esz_out);
    p.act = L->d.act == CBS_ACT_NONE ? ACT_NONE : ACT_SILU;
    const bool u8_out = L->d.out_dtype == CBS_U8;
    p.out_q = L->d.out_dtype != CBS_F32;
    p.out_scale = L->d.out_scale;
    // RN(1/s) in fp32: the double quotient rounded to float (one float of 24
    // bits times one of 25 cannot land within 2^-53 of 1 unless both are powers
    // of two, so the double rounding never changes the result)
    p.out_rcp = p.out_q ? (float)(1.0 / (double)L->d.out_scale) : 0.0f;
    p.out_zp = u8_out ? (float)L->d.out_zero_point : 0.0f;
    p.out_lo = u8_out ? 0.0f : -127.0f;
    p.out_hi = u8_out ? 255.0f : 127.0f;
    if (L->res_cs) {
      p.res = (const char *)res + (size_t)L->d.res_c_offset * esz_out;
      p.res_cs = L->res_cs;
      p.res_scale = L->d.res_scale;
      p.res_xor = u8_out ? 0u : 0x80808080u;
      p.res_zp = u8_out ? (float)L->d.res_zero_point : 128.0f;
      p.res_bytes = (unsigned)((size_t)L->M * L->res_cs * esz_out - (size_t)L->d.res_c_offset * esz_out);
    }
  }
  p.ws = splitk > 1 ? L->d_ws : nullptr;
  p.counters = splitk > 1 ? L->d_counters : nullptr;
  p.N = L->d.n;
  p.H = L->d.h;
  p.W = L->d.w;
  p.cin_pad = L->cin_pad;
  p.OH = L->oh;
  p.OW = L->ow;
  p.cout_pad = L->cout_pad;
  p.pitch = L->pitch;
  p.k = L->d.k;
  p.stride = L->d.stride;
  p.pad = L->d.pad;
  p.M = L->M;
  p.chunk_ch = L->chunk_ch;
  p.chunks_per_tap = L->chunks_per_tap;
  p.cpt_magic = L->cpt_magic;
  p.total_chunks = L->total_chunks;
  p.steps = L->steps;
  p.splitk = splitk;
  p.steps_per_split = ceil_div(L->steps, splitk);
  p.co_blocks = L->co_blocks;
  p.w_bytes = (unsigned)((size_t)L->co_blocks * L->steps * 64 * 16);
  const KernelConfig &kc = config(cfg);
  if (kc.lds == 2 || kc.lds == 3) {
    p.tiles_x = ceil_div(L->ow, kc.lds == 3 ? 2 * kc.tw : kc.tw);
    p.tiles_y = ceil_div(L->oh, kc.th);
    p.halo_cq = halo_cq(L);
    p.div_hcq = make_fastdiv(p.halo_cq);
    p.div_hwd = make_fastdiv(halo_width(L, kc));
    halo_lds(L, cfg, &p.halo_bytes, &p.smem_bytes);
  }
  if (kc.lds == 3) {  // column pairs: their own weights, K geometry and 16-row bias / dequant
    p.wfrag = L->d_wfrag_pair;
    p.bias = L->d_bias_pair;
    p.dq = L->d_dq_pair;
    p.total_chunks = L->pair_total_chunks;
    p.steps = L->pair_steps;
    p.steps_per_split = L->pair_steps;
    p.co_blocks = 1;
    p.w_bytes = (unsigned)((size_t)L->pair_steps * 64 * 16);
  }
  tiles_of(L, cfg, &p.px_tiles, &p.co_tiles);
  if (kc.lds == 4 || kc.lds == 5) {  // conv_ws runs: as equal as whole 16-pixel blocks allow
    const int blocks = ceil_div(L->M, 16);
    p.run_base = blocks / p.px_tiles;
    p.run_rem = blocks % p.px_tiles;
  }
  // Workgroup order (see tile_of in conv_kernels.h): pixel tiles inner when
  // the weights are larger than the input, so that each XCD's L2 fetches only
  // the weights of its own channel tiles.
  const double w_total = (double)p.w_bytes, x_total = (double)L->d.n * L->d.h * L->d.w * L->cin_pad * esz_in;
  p.px_inner = (w_total > x_total && p.co_tiles > 1) ? 1 : 0;
  p.inner_tiles = p.px_inner ? p.px_tiles : p.co_tiles;
  p.div_ow = make_fastdiv(p.OW);
  p.div_oh = make_fastdiv(p.OH);
  p.div_inner = make_fastdiv(p.inner_tiles);
  p.div_sk = make_fastdiv(p.splitk);
  p.div_tx = make_fastdiv(p.tiles_x);
  p.div_ty = make_fastdiv(p.tiles_y);
  return p;
}

// Split-K factors of a group's members under configuration cfg: the member
// with the shallowest K per wave keeps split-K 1, and each deeper member is
// split (up to 4 ways) towards that depth, so that no member's workgroups run
// several times longer than the others'.
void group_splits(const cbs_layer *const *m, int n, int cfg, int *sk) {
  const KernelConfig &c = config(cfg);
  if (c.lds) {  // LDS-staged tiles have no split-K
    for (int i = 0; i < n; i++) sk[i] = 1;
    return;
  }
  double shallowest = 1e300;
  for (int i = 0; i < n; i++) shallowest = std::min(shallowest, std::ceil((double)m[i]->steps / c.wk));
  for (int i = 0; i < n; i++) {
    const double depth = std::ceil((double)m[i]->steps / c.wk);
    int s = (int)std::lround(depth / shallowest);
    s = std::max(1, std::min(4, s));
    while (s > 1 && !config_fits(m[i], cfg, s)) s--;
    sk[i] = s;
  }
}

// Cost of a grouped launch (the model_cost terms): the members' waves share
// the 1024 SIMDs, and no member's wave can finish before its own K slice.
double group_cost(const cbs_layer *const *m, int n, int cfg, const int *sk) {
  const KernelConfig &c = config(cfg);
  double total = 0.0, longest = 0.0, split_cost = 0.0;
  for (int i = 0; i < n; i++) {
    const cbs_layer *L = m[i];
    int pxt, cot;
    tiles_of(L, cfg, &pxt, &cot);
    const double steps_per_wave = std::ceil((double)L->steps / (c.wk * sk[i]));
    const double mfma_step = L->d.dtype == CBS_F32 ? 4 * 32.0 : 16.0;
    const double load_step = 40.0 * (c.cb + c.pb);
    const double per_wave = steps_per_wave * std::max(mfma_step * c.cb * c.pb, load_step) + 1500.0;
    total += (double)pxt * cot * sk[i] * c.wco * c.wpx * c.wk * per_wave;
    longest = std::max(longest, per_wave);
    if (sk[i] > 1) split_cost = 2500.0;
  }
  return std::max(total / 1024.0, longest) + split_cost;
}

// Whether configuration cfg (with split-K factors sk) can run every member of a group.
bool group_config_fits(const cbs_layer *const *m, int n, int cfg, const int *sk) {
  if (cfg < 0 || cfg >= num_configs() || config(cfg).lds > 1) return false;  // register-direct or LDS-staged
  double grid = 0.0;
  for (int i = 0; i < n; i++) {
    if (!config_fits(m[i], cfg, sk[i])) return false;
    int pxt, cot;
    tiles_of(m[i], cfg, &pxt, &cot);
    grid += (double)pxt * cot * sk[i];
  }
  return grid < 2147483647.0;
}

void group_release(cbs_group *g) {
  for (int i = 0; i < cbs::kGroupMax; i++) {
    if (g->d_ws[i]) (void)hipFree(g->d_ws[i]);
    if (g->d_counters[i]) (void)hipFree(g->d_counters[i]);
    g->d_ws[i] = nullptr;
    g->d_counters[i] = nullptr;
  }
}

// The partial-tile workspace and zeroed arrival counters of the split members.
cbs_status group_setup_splitk(cbs_group *g) {
  const KernelConfig &c = config(g->config);
  for (int i = 0; i < g->n; i++) {
    if (g->splitk[i] <= 1) continue;
    int pxt, cot;
    tiles_of(g->member[i], g->config, &pxt, &cot);
    const size_t tiles = (size_t)pxt * cot;
    const size_t tile_vecs = (size_t)c.wco * c.wpx * c.cb * c.pb * 64;
    cbs_status st = dev_alloc((void **)&g->d_ws[i], tiles * g->splitk[i] * tile_vecs * 16);
    if (st == CBS_OK) st = dev_alloc((void **)&g->d_counters[i], tiles * sizeof(unsigned));
    if (st != CBS_OK) return st;
    hipError_t e = hipMemset(g->d_counters[i], 0, tiles * sizeof(unsigned));
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) return fail(CBS_EDEVICE, "group counter init: %s", hipGetErrorString(e));
  }
  return CBS_OK;
}

cbs_status launch(const cbs_layer *L, const void *in, void *out, const void *res, void *stream, bool raw = false,
                  const void *in2 = nullptr) {
  ConvParams p = make_params(L, in, out, res, raw, L->config, L->splitk, in2);
  hipError_t e = launch_conv(raw ? L->raw_variant : L->variant, L->config, p, (hipStream_t)stream);
  if (e != hipSuccess) return fail(CBS_ELAUNCH, "conv launch: %s", hipGetErrorString(e));
  return CBS_OK;
}

// Argument check of one step: buffers present, residual and second input given
// iff the layer has them.
cbs_status check_step(const cbs_layer *L, const void *in, const void *out, const void *res, const char *where,
                      int idx, const void *in2 = nullptr) {
  if (!L || !in || !out) return fail(CBS_EINVAL, "%s: null layer or buffer (entry %d)", where, idx);
  if (L->res_cs && !res)
    return fail(CBS_EINVAL, "%s: layer %d was created with a residual and needs one", where, idx);
  if (!L->res_cs && res) return fail(CBS_EINVAL, "%s: layer %d has no residual but one was given", where, idx);
  if (L->in2_ch && !in2)
    return fail(CBS_EINVAL, "%s: layer %d was created with a second input and needs one", where, idx);
  if (!L->in2_ch && in2)
    return fail(CBS_EINVAL, "%s: layer %d has no second input but one was given", where, idx);
  return CBS_OK;
}

}  // namespace

namespace cbs {

cbs_status report_error(cbs_status st, const char *what, const char *detail) {
  return fail(st, "%s: %s", what, detail ? detail : "");
}

cbs_status scratch_launch(const cbs_layer *L, const void *in, void *out, int32_t splitk, void *ws, size_t ws_cap,
                          unsigned *counters, size_t counters_cap, ConvParams *p, int *variant, int *cfg,
                          unsigned *tiles) {
  cbs_status st = check_step(L, in, out, nullptr, "run_layer_noalloc", 0);
  if (st != CBS_OK) return st;
  if (splitk < 0 || splitk > 64) return fail(CBS_EINVAL, "run_layer_noalloc: splitk %d not in [0, 64]", (int)splitk);
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != L->device)
    return fail(CBS_EINVAL, "run_layer_noalloc: the current device (%d) is not the layer's (%d)", dev, L->device);
  const int sk = splitk == 0 ? L->splitk : (int)splitk;
  if (!config_fits(L, L->config, sk))
    return fail(CBS_EUNSUPPORTED, "run_layer_noalloc: configuration %s cannot run this layer with split-K %d "
                                  "(a split needs a register-direct configuration and enough K steps)",
                config(L->config).name, sk);
  size_t need_ws, need_cnt;
  splitk_need(L, L->config, sk, &need_ws, &need_cnt);
  if (need_ws > ws_cap || need_cnt > counters_cap)
    return fail(CBS_EUNSUPPORTED, "run_layer_noalloc: split-K %d of configuration %s needs %zu bytes of partial "
                                  "tiles and %zu tickets; the static scratch holds %zu and %zu",
                sk, config(L->config).name, need_ws, need_cnt, ws_cap, counters_cap);
  *p = make_params(L, in, out, nullptr, false, L->config, sk);
  p->ws = need_ws ? (float *)ws : nullptr;
  p->counters = need_cnt ? counters : nullptr;
  *variant = L->variant;
  *cfg = L->config;
  *tiles = (unsigned)need_cnt;
  return CBS_OK;
}

}  // namespace cbs

namespace {

// ------------------------------------------------------------ create ----

cbs_status create_impl(const cbs_conv_desc *desc, const float *w, const float *gamma, const float *beta,
                       const float *mean, const float *var, const float *scale, const float *bias,
                       cbs_layer **out) {
  if (!out) return fail(CBS_EINVAL, "out is NULL");
  *out = nullptr;
  cbs_status st = validate(desc);
  if (st != CBS_OK) return st;
  if (!w) return fail(CBS_EINVAL, "weights are NULL");
  if (!scale && (!gamma || !beta || !mean || !var)) return fail(CBS_EINVAL, "BN parameters are NULL");
  if (scale && !bias) return fail(CBS_EINVAL, "bias is NULL");

  int dev_count = 0;
  if (hipGetDeviceCount(&dev_count) != hipSuccess || dev_count < 1) {
    (void)hipGetLastError();
    return fail(CBS_EDEVICE, "no HIP device");
  }

  cbs_layer *L = new (std::nothrow) cbs_layer();
  if (!L) return fail(CBS_ENOMEM, "host allocation");
  L->d = *desc;
  const cbs_conv_desc &d = L->d;
  if (hipGetDevice(&L->device) != hipSuccess) {
    delete L;
    return fail(CBS_EDEVICE, "hipGetDevice failed");
  }
  {
    int cus = 0, lds = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, L->device) == hipSuccess && cus > 0)
      L->cus = cus;
    else
      (void)hipGetLastError();
    if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, L->device) == hipSuccess &&
        lds >= 65536)
      L->lds_max = lds;
    else
      (void)hipGetLastError();
  }
  L->oh = out_dim(d.h, d.k, d.stride, d.pad);
  L->ow = out_dim(d.w, d.k, d.stride, d.pad);
  L->pitch = d.out_row_pitch ? d.out_row_pitch : L->ow;
  L->cin_pad = round_up(d.c_in, 4);
  L->cout_pad = round_up(d.c_out, 4);
  L->in2_ch = d.in2_channels;
  L->in2_cs = d.in2_channels ? (d.in2_c_stride ? d.in2_c_stride : round_up(d.in2_channels, 4)) : 0;
  L->in_cs = d.in_c_stride ? d.in_c_stride : (L->in2_ch ? d.c_in - L->in2_ch : L->cin_pad);
  L->out_cs = d.out_c_stride ? d.out_c_stride : L->cout_pad;
  L->res_cs = d.res_c_stride;
  L->co_blocks = ceil_div(L->cout_pad, 16);
  L->M = d.n * L->oh * L->ow;
  const int taps = d.k * d.k;
  int vec = 1;
  if (d.dtype == CBS_F32) {
    L->chunk_ch = 4;
    L->variant = VAR_F32;
    L->raw_variant = -1;
  } else if (L->cin_pad % 16 == 0 && L->in_cs % 16 == 0 && d.in_c_offset % 16 == 0) {
    // 16-channel chunks: one 16-byte load per lane, which needs 16-byte aligned pixels
    L->chunk_ch = 16;
    L->variant = d.dtype == CBS_U8 ? VAR_U8_C16_X : VAR_I8_C16;
    L->raw_variant = d.dtype == CBS_U8 ? VAR_U8_C16_RAW : VAR_I8_C16_RAW;
  } else {
    L->chunk_ch = 4;
    vec = 4;
    L->variant = d.dtype == CBS_U8 ? VAR_U8_C4_X : VAR_I8_C4;
    L->raw_variant = d.dtype == CBS_U8 ? VAR_U8_C4_RAW : VAR_I8_C4_RAW;
  }
  // the general epilogue only when an option needs it (uint8 layers always have it)
  if (d.act != CBS_ACT_SILU || d.out_dtype != CBS_F32 || d.res_c_stride != 0) {
    if (L->variant == VAR_F32) L->variant = VAR_F32_X;
    if (L->variant == VAR_I8_C16) L->variant = VAR_I8_C16_X;
    if (L->variant == VAR_I8_C4) L->variant = VAR_I8_C4_X;
  }
  L->chunks_per_tap = L->cin_pad / L->chunk_ch;
  L->total_chunks = taps * L->chunks_per_tap;
  const int chunks_per_step = 4 * vec;
  L->steps = ceil_div(L->total_chunks, chunks_per_step);
  // chunk -> tap by multiply-shift; checked for every chunk index the kernel decodes
  L->cpt_magic = (unsigned)(((1u << 20) + L->chunks_per_tap - 1) / L->chunks_per_tap);
  for (int c = 0; c < L->steps * chunks_per_step; c++) {
    if ((int)(((unsigned)c * L->cpt_magic) >> 20) != c / L->chunks_per_tap) {
      delete L;
      return fail(CBS_EUNSUPPORTED, "chunk decode not exact for this shape");
    }
  }

  // ---- fold batch norm in double
  const int per_co = d.c_in * taps;
  std::vector<double> wf((size_t)d.c_out * per_co), bf(d.c_out);
  for (int co = 0; co < d.c_out; co++) {
    double sc, b;
    if (scale) {
      sc = (double)scale[co];
      b = (double)bias[co];
    } else {
      sc = (double)gamma[co] / std::sqrt((double)var[co] + (double)d.bn_eps);
      b = (double)beta[co] - (double)mean[co] * sc;
    }
    for (int i = 0; i < per_co; i++) wf[(size_t)co * per_co + i] = (double)w[(size_t)co * per_co + i] * sc;
    bf[co] = b;
  }
  L->h_bias.assign(d.c_out, 0.f);
  for (int co = 0; co < d.c_out; co++) L->h_bias[co] = (float)bf[co];

  // ---- per-output-channel int8 quantisation (double)
  std::vector<float> dq;
  if (d.dtype != CBS_F32) {
    L->h_qw.assign((size_t)d.c_out * per_co, 0);
    L->h_sw.assign(d.c_out, 1.0);
    dq.assign((size_t)L->co_blocks * 16, 0.f);
    for (int co = 0; co < d.c_out; co++) {
      double m = 0.0;
      for (int i = 0; i < per_co; i++) m = std::max(m, std::fabs(wf[(size_t)co * per_co + i]));
      const double s = m > 0.0 ? m / 127.0 : 1.0;
      L->h_sw[co] = s;
      for (int i = 0; i < per_co; i++) {
        double q = std::nearbyint(wf[(size_t)co * per_co + i] / s);
        q = std::min(127.0, std::max(-127.0, q));
        L->h_qw[(size_t)co * per_co + i] = (int8_t)q;
      }
      dq[co] = (float)((double)d.in_scale * s);
    }
  } else {
    L->h_wfold.resize((size_t)d.c_out * per_co);
    for (size_t i = 0; i < wf.size(); i++) L->h_wfold[i] = (float)wf[i];
  }

  // ---- weights in MFMA fragment order: [co_block][step][lane][16 bytes]
  // lane = 16*g + r: output channel co_block*16 + r; chunks (4*step + g)*vec + j.
  const size_t frag_bytes = (size_t)L->co_blocks * L->steps * 64 * 16;
  if (frag_bytes >= ((size_t)1 << 31) - 2048) {
    delete L;
    return fail(CBS_EUNSUPPORTED, "weights above 2^31 bytes");
  }
  std::vector<unsigned char> frag(frag_bytes, 0);
  for (int cob = 0; cob < L->co_blocks; cob++)
    for (int s = 0; s < L->steps; s++)
      for (int lane = 0; lane < 64; lane++) {
        const int r = lane & 15, g = lane >> 4, co = cob * 16 + r;
        unsigned char *dst = &frag[(((size_t)cob * L->steps + s) * 64 + lane) * 16];
        if (co >= d.c_out) continue;
        for (int j = 0; j < vec; j++) {
          const int c = (4 * s + g) * vec + j;
          if (c >= L->total_chunks) continue;
          const int tap = c / L->chunks_per_tap;
          const int ci0 = (c % L->chunks_per_tap) * L->chunk_ch;
          const int kh = tap / d.k, kw = tap % d.k;
          for (int e = 0; e < L->chunk_ch; e++) {
            const int ci = ci0 + e;
            if (ci >= d.c_in) continue;
            const size_t src = (((size_t)co * d.c_in + ci) * d.k + kh) * d.k + kw;
            if (d.dtype == CBS_F32) {
              const float v = L->h_wfold[src];
              std::memcpy(dst + 4 * e, &v, 4);
            } else {
              dst[j * 4 + e] = (unsigned char)L->h_qw[src];
            }
          }
        }
      }

  // ---- column pairs (conv_halo with PAIR): for 3x3 stride-1 layers with at
  // most 8 output channels, row 8*h + co of one 16-row block is channel co of
  // pixel 2*j + h of the pair j, over the pair's 3 x 4 input window: the
  // weight of window tap (dy, dx) is W'[co, ci, dy, dx - h], zero where
  // dx - h is outside 0..2.  Same chunk order as above, 12 taps instead of 9.
  std::vector<unsigned char> frag_pair;
  std::vector<float> bias_pair, dq_pair;
  L->pair = d.k == 3 && d.stride == 1 && d.pad == 1 && L->cout_pad <= 8;
  if (L->pair) {
    L->pair_total_chunks = 12 * L->chunks_per_tap;
    L->pair_steps = ceil_div(L->pair_total_chunks, chunks_per_step);
    for (int c = 0; c < L->pair_steps * chunks_per_step; c++)
      if ((int)(((unsigned)c * L->cpt_magic) >> 20) != c / L->chunks_per_tap) L->pair = false;
  }
  if (L->pair) {
    frag_pair.assign((size_t)L->pair_steps * 64 * 16, 0);
    for (int s = 0; s < L->pair_steps; s++)
      for (int lane = 0; lane < 64; lane++) {
        const int r = lane & 15, g = lane >> 4, h = r >> 3, co = r & 7;
        unsigned char *dst = &frag_pair[((size_t)s * 64 + lane) * 16];
        if (co >= d.c_out) continue;
        for (int j = 0; j < vec; j++) {
          const int c = (4 * s + g) * vec + j;
          if (c >= L->pair_total_chunks) continue;
          const int tap = c / L->chunks_per_tap;
          const int ci0 = (c % L->chunks_per_tap) * L->chunk_ch;
          const int kh = tap >> 2, kw = (tap & 3) - h;
          if (kw < 0 || kw > 2) continue;
          for (int e = 0; e < L->chunk_ch; e++) {
            const int ci = ci0 + e;
            if (ci >= d.c_in) continue;
            const size_t src = (((size_t)co * d.c_in + ci) * 3 + kh) * 3 + kw;
            if (d.dtype == CBS_F32) {
              const float v = L->h_wfold[src];
              std::memcpy(dst + 4 * e, &v, 4);
            } else {
              dst[j * 4 + e] = (unsigned char)L->h_qw[src];
            }
          }
        }
      }
    bias_pair.assign(16, 0.f);
    dq_pair.assign(16, 0.f);
    for (int r = 0; r < 16; r++) {
      const int co = r & 7;
      if (co >= d.c_out) continue;
      bias_pair[r] = L->h_bias[co];
      if (d.dtype != CBS_F32) dq_pair[r] = dq[co];
    }
  }

  // ---- uint8 input: accumulator start values per border class (see
  // border_class in conv_kernels.h).  With T[co][tap] the sum of the channel's
  // int8 weights at a tap, Wsum[co] = sum_tap T and Win the sum over the taps
  // whose row (bit of rm) and column (bit of cm) lie inside the image, the
  // kernel's sum over q - 128 (and -128 on padding taps) plus
  // 128 Wsum - z Win is the sum over q - z on the taps inside the image.
  std::vector<int> corr;
  if (d.dtype == CBS_U8) {
    const int cpad16 = L->co_blocks * 16;
    corr.assign((size_t)64 * cpad16, 0);
    for (int co = 0; co < d.c_out; co++) {
      long long T[9] = {0}, wsum = 0;
      for (int ci = 0; ci < d.c_in; ci++)
        for (int t = 0; t < taps; t++) T[t] += L->h_qw[((size_t)co * d.c_in + ci) * taps + t];
      for (int t = 0; t < taps; t++) wsum += T[t];
      for (int rm = 0; rm < 8; rm++)
        for (int cm = 0; cm < 8; cm++) {
          long long win = 0;
          for (int i = 0; i < d.k; i++)
            for (int j = 0; j < d.k; j++)
              if (((rm >> i) & 1) && ((cm >> j) & 1)) win += T[i * d.k + j];
          const long long c = 128 * wsum - (long long)d.in_zero_point * win;
          if (c < INT32_MIN || c > INT32_MAX) {
            delete L;
            return fail(CBS_EUNSUPPORTED, "uint8 zero-point correction outside int32");
          }
          corr[(size_t)(rm * 8 + cm) * cpad16 + co] = (int)c;
        }
    }
  }

  // ---- kernel configuration
  const Choice ch = choose(L);
  L->config = ch.config;
  L->splitk = ch.splitk;

  // ---- device memory
  std::vector<float> biasv((size_t)L->co_blocks * 16, 0.f);
  for (int co = 0; co < d.c_out; co++) biasv[co] = L->h_bias[co];
  st = dev_alloc(&L->d_wfrag, frag_bytes);
  if (st == CBS_OK) st = dev_alloc((void **)&L->d_bias, biasv.size() * sizeof(float));
  if (st == CBS_OK && d.dtype != CBS_F32) st = dev_alloc((void **)&L->d_dq, dq.size() * sizeof(float));
  if (st == CBS_OK && d.dtype == CBS_U8) st = dev_alloc((void **)&L->d_corr, corr.size() * sizeof(int));
  if (st == CBS_OK && L->pair) st = dev_alloc(&L->d_wfrag_pair, frag_pair.size());
  if (st == CBS_OK && L->pair) st = dev_alloc((void **)&L->d_bias_pair, bias_pair.size() * sizeof(float));
  if (st == CBS_OK && L->pair && d.dtype != CBS_F32)
    st = dev_alloc((void **)&L->d_dq_pair, dq_pair.size() * sizeof(float));
  if (st == CBS_OK) st = setup_splitk(L);
  if (st == CBS_OK) {
    hipError_t e = hipMemcpy(L->d_wfrag, frag.data(), frag_bytes, hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipMemcpy(L->d_bias, biasv.data(), biasv.size() * sizeof(float), hipMemcpyHostToDevice);
    if (e == hipSuccess && d.dtype != CBS_F32)
      e = hipMemcpy(L->d_dq, dq.data(), dq.size() * sizeof(float), hipMemcpyHostToDevice);
    if (e == hipSuccess && d.dtype == CBS_U8)
      e = hipMemcpy(L->d_corr, corr.data(), corr.size() * sizeof(int), hipMemcpyHostToDevice);
    if (e == hipSuccess && L->pair)
      e = hipMemcpy(L->d_wfrag_pair, frag_pair.data(), frag_pair.size(), hipMemcpyHostToDevice);
    if (e == hipSuccess && L->pair)
      e = hipMemcpy(L->d_bias_pair, bias_pair.data(), bias_pair.size() * sizeof(float), hipMemcpyHostToDevice);
    if (e == hipSuccess && L->pair && d.dtype != CBS_F32)
      e = hipMemcpy(L->d_dq_pair, dq_pair.data(), dq_pair.size() * sizeof(float), hipMemcpyHostToDevice);
    if (e != hipSuccess) st = fail(CBS_EDEVICE, "weight upload: %s", hipGetErrorString(e));
  }
  if (st != CBS_OK) {
    release(L);
    delete L;
    return st;
  }
  *out = L;
  return CBS_OK;
}

}  // namespace

// ================================================================= C ABI ==

extern "C" {

cbs_status cbs_create_layer(const cbs_conv_desc *desc, const float *w_oihw, const float *gamma,
                            const float *beta, const float *mean, const float *var, cbs_layer **out) {
  return create_impl(desc, w_oihw, gamma, beta, mean, var, nullptr, nullptr, out);
}

cbs_status cbs_create_layer_folded(const cbs_conv_desc *desc, const float *w_oihw, const float *scale,
                                   const float *bias, cbs_layer **out) {
  if (!scale) {
    if (out) *out = nullptr;
    return fail(CBS_EINVAL, "scale is NULL");
  }
  return create_impl(desc, w_oihw, nullptr, nullptr, nullptr, nullptr, scale, bias, out);
}

void cbs_destroy_layer(cbs_layer *layer) {
  if (!layer) return;
  release(layer);
  delete layer;
}

cbs_status cbs_run_layer(const cbs_layer *layer, const void *in, void *out, void *stream) {
  cbs_status st = check_step(layer, in, out, nullptr, "run_layer", 0);
  if (st != CBS_OK) return st;
  return launch(layer, in, out, nullptr, stream);
}

cbs_status cbs_run_layer_res(const cbs_layer *layer, const void *in, void *out, const void *residual,
                             void *stream) {
  if (!residual) return fail(CBS_EINVAL, "run_layer_res: residual is NULL");
  cbs_status st = check_step(layer, in, out, residual, "run_layer_res", 0);
  if (st != CBS_OK) return st;
  return launch(layer, in, out, residual, stream);
}

cbs_status cbs_run_layer_in2(const cbs_layer *layer, const void *in, const void *in2, void *out,
                             const void *residual, void *stream) {
  if (!in2) return fail(CBS_EINVAL, "run_layer_in2: in2 is NULL");
  cbs_status st = check_step(layer, in, out, residual, "run_layer_in2", 0, in2);
  if (st != CBS_OK) return st;
  return launch(layer, in, out, residual, stream, false, in2);
}

cbs_status cbs_run_layer_list(cbs_layer *const *layers, int32_t n, const void *const *ins,
                              void *const *outs, void *stream) {
  if (n < 0 || (n > 0 && (!layers || !ins || !outs))) return fail(CBS_EINVAL, "run_layer_list: bad arguments");
  for (int32_t i = 0; i < n; i++) {
    cbs_status st = check_step(layers[i], ins[i], outs[i], nullptr, "run_layer_list", i);
    if (st == CBS_OK) st = launch(layers[i], ins[i], outs[i], nullptr, stream);
    if (st != CBS_OK) return st;
  }
  return CBS_OK;
}

cbs_status cbs_group_create(cbs_layer *const *layers, int32_t n, int32_t config_id, cbs_group **out) {
  if (!out) return fail(CBS_EINVAL, "group_create: out is NULL");
  *out = nullptr;
  if (!layers || n < 1 || n > kGroupMax)
    return fail(CBS_EINVAL, "group_create: needs 1 to %d layers (got %d)", kGroupMax, (int)n);
  for (int32_t i = 0; i < n; i++) {
    const cbs_layer *L = layers[i];
    if (!L) return fail(CBS_EINVAL, "group_create: layer %d is NULL", (int)i);
    if (L->res_cs) return fail(CBS_EUNSUPPORTED, "group_create: layer %d has a residual", (int)i);
    if (L->in2_ch) return fail(CBS_EUNSUPPORTED, "group_create: layer %d has a second input", (int)i);
    if (L->variant != layers[0]->variant || L->device != layers[0]->device)
      return fail(CBS_EUNSUPPORTED, "group_create: layer %d differs from layer 0 in kernel variant (dtype, "
                                    "input chunking or epilogue) or device", (int)i);
  }
  cbs_group *g = new cbs_group;
  g->n = n;
  g->variant = layers[0]->variant;
  // grid order: deepest K first, so that the longest workgroups start first
  for (int32_t i = 0; i < n; i++) g->slot[i] = i;
  std::stable_sort(g->slot, g->slot + n, [&](int a, int b) { return layers[a]->steps > layers[b]->steps; });
  for (int32_t i = 0; i < n; i++) g->member[i] = layers[g->slot[i]];
  int sk[kGroupMax];
  if (config_id >= 0) {
    const bool tiled = config_id < num_configs() && config(config_id).lds <= 1;
    if (tiled) group_splits(g->member, n, config_id, sk);
    if (!tiled || !group_config_fits(g->member, n, config_id, sk)) {
      delete g;
      return fail(CBS_EUNSUPPORTED, "group_create: configuration %d is not a register-direct or LDS-staged "
                                    "configuration that fits every layer", (int)config_id);
    }
    g->config = config_id;
  } else {
    double best = 1e300;
    g->config = -1;
    for (int cfg = 0; cfg < num_configs(); cfg++) {
      if (config(cfg).lds != 0) continue;
      group_splits(g->member, n, cfg, sk);
      if (!group_config_fits(g->member, n, cfg, sk)) continue;
      const double c = group_cost(g->member, n, cfg, sk);
      if (c < best * 0.999) {
        best = c;
        g->config = cfg;
      }
    }
    if (g->config < 0) {
      delete g;
      return fail(CBS_EUNSUPPORTED, "group_create: no register-direct configuration fits every layer");
    }
  }
  group_splits(g->member, n, g->config, g->splitk);
  cbs_status st = group_setup_splitk(g);
  if (st != CBS_OK) {
    group_release(g);
    delete g;
    return st;
  }
  *out = g;
  return CBS_OK;
}

cbs_status cbs_group_run(const cbs_group *group, const void *const *ins, void *const *outs, void *stream) {
  if (!group || !ins || !outs) return fail(CBS_EINVAL, "group_run: null group or buffer list");
  GroupArgs ga;
  std::memset(&ga, 0, sizeof(ga));
  long long grid = 0;
  for (int j = 0; j < kGroupMax; j++) ga.first[j] = INT_MAX;
  for (int j = 0; j < group->n; j++) {
    const int i = group->slot[j];
    const cbs_layer *L = group->member[j];
    cbs_status st = check_step(L, ins[i], outs[i], nullptr, "group_run", i);
    if (st != CBS_OK) return st;
    ga.p[j] = make_params(L, ins[i], outs[i], nullptr, false, group->config, group->splitk[j]);
    ga.p[j].ws = group->d_ws[j];
    ga.p[j].counters = group->d_counters[j];
    ga.first[j] = (int)grid;
    grid += (long long)ga.p[j].px_tiles * ga.p[j].co_tiles * group->splitk[j];
  }
  hipError_t e = launch_conv_group(group->variant, group->config, ga, (unsigned)grid, (hipStream_t)stream);
  if (e != hipSuccess) return fail(CBS_ELAUNCH, "group launch: %s", hipGetErrorString(e));
  return CBS_OK;
}

int32_t cbs_group_config(const cbs_group *group) { return group ? group->config : -1; }

void cbs_group_destroy(cbs_group *group) {
  if (!group) return;
  group_release(group);
  delete group;
}

cbs_status cbs_run_steps(const cbs_step *steps, int32_t n, void *stream) {
  if (n < 0 || (n > 0 && !steps)) return fail(CBS_EINVAL, "run_steps: bad arguments");
  for (int32_t i = 0; i < n; i++) {
    const cbs_step &t = steps[i];
    cbs_status st = check_step(t.layer, t.in, t.out, t.residual, "run_steps", i, t.in2);
    if (st == CBS_OK) st = launch(t.layer, t.in, t.out, t.residual, stream, false, t.in2);
    if (st != CBS_OK) return st;
  }
  return CBS_OK;
}

}  // extern "C"

namespace {

// One launch of a captured step list: a layer's own launch, or a grouped
// launch (group != nullptr) of the layers `slots` of the list.
struct Launch {
  int step = -1;
  cbs_group *group = nullptr;
  std::vector<int> slots;
};

// Capture a validated step list into an instantiated graph, as the given
// launches (in order).  The capture runs on a private stream (the caller's
// may be the null stream, which cannot be captured), at default priority.
// Every captured layer gets one graph reference, which keeps its split-K
// workspace in place until the graph is destroyed.  On success the graph owns
// the launches' groups; on failure they are destroyed.
cbs_status capture(const std::vector<cbs_step> &steps, const std::vector<Launch> &launches, cbs_graph **out) {
  cbs_graph *G = new (std::nothrow) cbs_graph();
  if (!G) {
    for (const Launch &l : launches) cbs_group_destroy(l.group);
    return fail(CBS_ENOMEM, "host allocation");
  }
  for (const cbs_step &t : steps) {
    t.layer->graph_refs.fetch_add(1);
    G->layers.push_back(t.layer);
  }
  for (const Launch &l : launches)
    if (l.group) G->groups.push_back(l.group);
  G->launches = (int)launches.size();
  hipStream_t cs = nullptr;
  hipError_t e = hipStreamCreateWithFlags(&cs, hipStreamNonBlocking);
  if (e != hipSuccess) {
    cbs_graph_destroy(G);
    return fail(CBS_EDEVICE, "capture stream: %s", hipGetErrorString(e));
  }
  e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
  cbs_status st = CBS_OK;
  if (e != hipSuccess) st = fail(CBS_EDEVICE, "begin capture: %s", hipGetErrorString(e));
  if (st == CBS_OK) {
    for (size_t i = 0; i < launches.size() && st == CBS_OK; i++) {
      const Launch &l = launches[i];
      if (!l.group) {
        const cbs_step &t = steps[l.step];
        st = launch(t.layer, t.in, t.out, t.residual, cs, false, t.in2);
      } else {
        std::vector<const void *> ins;
        std::vector<void *> outs;
        for (int k : l.slots) {
          ins.push_back(steps[k].in);
          outs.push_back(steps[k].out);
        }
        st = cbs_group_run(l.group, ins.data(), outs.data(), cs);
      }
    }
    hipGraph_t g = nullptr;
    e = hipStreamEndCapture(cs, &g);
    if (st == CBS_OK && e != hipSuccess) st = fail(CBS_EDEVICE, "end capture: %s", hipGetErrorString(e));
    G->graph = g;
  }
  if (st == CBS_OK) {
    e = hipGraphInstantiate(&G->exec, G->graph, nullptr, nullptr, 0);
    if (e != hipSuccess) st = fail(CBS_EDEVICE, "graph instantiate: %s", hipGetErrorString(e));
  }
  (void)hipStreamDestroy(cs);
  if (st != CBS_OK) {
    cbs_graph_destroy(G);
    return st;
  }
  *out = G;
  return CBS_OK;
}

// One launch per step, in order.
std::vector<Launch> plain_launches(size_t n) {
  std::vector<Launch> v(n);
  for (size_t i = 0; i < n; i++) v[i].step = (int)i;
  return v;
}

}  // namespace

extern "C" {

cbs_status cbs_graph_create(cbs_layer *const *layers, int32_t n, const void *const *ins, void *const *outs,
                            void *stream, cbs_graph **out) {
  (void)stream;
  if (!out) return fail(CBS_EINVAL, "graph_create: out is NULL");
  *out = nullptr;
  if (n < 1 || !layers || !ins || !outs) return fail(CBS_EINVAL, "graph_create: bad arguments");
  std::vector<cbs_step> steps(n);
  for (int32_t i = 0; i < n; i++) {
    cbs_status st = check_step(layers[i], ins[i], outs[i], nullptr, "graph_create", i);
    if (st != CBS_OK) return st;
    steps[i] = cbs_step{layers[i], ins[i], outs[i], nullptr};
  }
  return capture(steps, plain_launches(steps.size()), out);
}

cbs_status cbs_graph_create_steps(const cbs_step *steps, int32_t n, void *stream, cbs_graph **out) {
  (void)stream;
  if (!out) return fail(CBS_EINVAL, "graph_create_steps: out is NULL");
  *out = nullptr;
  if (n < 1 || !steps) return fail(CBS_EINVAL, "graph_create_steps: bad arguments");
  for (int32_t i = 0; i < n; i++) {
    cbs_status st = check_step(steps[i].layer, steps[i].in, steps[i].out, steps[i].residual, "graph_create_steps", i,
                               steps[i].in2);
    if (st != CBS_OK) return st;
  }
  return capture(std::vector<cbs_step>(steps, steps + n), plain_launches(n), out);
}

}  // extern "C"

namespace {

// Bytes a layer's run reads from its input pointer and writes from its output
// pointer (the whole pixel rows, slices included, guard pixels included).
int64_t in_span(const cbs_layer *L) {
  return (int64_t)L->d.n * L->d.h * L->d.w * L->in_cs * (L->d.dtype == CBS_F32 ? 4 : 1);
}
int64_t out_span(const cbs_layer *L) {
  return (int64_t)L->d.n * L->oh * L->pitch * L->out_cs * (L->d.out_dtype == CBS_F32 ? 4 : 1);
}
bool overlap(const void *a, int64_t na, const void *b, int64_t nb) {
  const char *pa = (const char *)a, *pb = (const char *)b;
  return pa < pb + nb && pb < pa + na;
}

// Microseconds per copy of the work that enqueue(stream) enqueues, timed as
// replays of a graph holding `reps` back-to-back copies of it on a private
// stream: the best of `rounds` replays after one warm-up replay.
template <class F>
cbs_status time_replays(F enqueue, int reps, int rounds, float *us) {
  hipStream_t cs = nullptr;
  hipGraph_t g = nullptr;
  hipGraphExec_t ex = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (hipStreamCreateWithFlags(&cs, hipStreamNonBlocking) != hipSuccess)
    return fail(CBS_EDEVICE, "timing: stream creation failed");
  cbs_status st = CBS_OK;
  if (hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal) != hipSuccess)
    st = fail(CBS_EDEVICE, "timing: begin capture failed");
  if (st == CBS_OK) {
    for (int i = 0; i < reps && st == CBS_OK; i++) st = enqueue(cs);
    const hipError_t e = hipStreamEndCapture(cs, &g);
    if (st == CBS_OK && e != hipSuccess) st = fail(CBS_EDEVICE, "timing: end capture: %s", hipGetErrorString(e));
  }
  if (st == CBS_OK && hipGraphInstantiate(&ex, g, nullptr, nullptr, 0) != hipSuccess)
    st = fail(CBS_EDEVICE, "timing: graph instantiate failed");
  if (st == CBS_OK && (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess))
    st = fail(CBS_EDEVICE, "timing: event creation failed");
  float best = 1e30f;
  if (st == CBS_OK && (hipGraphLaunch(ex, cs) != hipSuccess || hipStreamSynchronize(cs) != hipSuccess))
    st = fail(CBS_EDEVICE, "timing: warm-up replay failed");
  for (int r = 0; r < rounds && st == CBS_OK; r++) {
    float ms = 0.f;
    if (hipEventRecord(e0, cs) != hipSuccess || hipGraphLaunch(ex, cs) != hipSuccess ||
        hipEventRecord(e1, cs) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
        hipEventElapsedTime(&ms, e0, e1) != hipSuccess)
      st = fail(CBS_EDEVICE, "timing: replay failed");
    else
      best = std::min(best, ms);
  }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (ex) (void)hipGraphExecDestroy(ex);
  if (g) (void)hipGraphDestroy(g);
  (void)hipStreamDestroy(cs);
  *us = best * 1000.f / (float)reps;
  return st;
}

constexpr int kGroupTimingReps = 20, kGroupTimingRounds = 5;

}  // namespace

extern "C" {

cbs_status cbs_graph_create_grouped(cbs_layer *const *layers, int32_t n, const void *const *ins,
                                    void *const *outs, const int32_t *group_of, void *stream, cbs_graph **out) {
  (void)stream;
  if (!out) return fail(CBS_EINVAL, "graph_create_grouped: out is NULL");
  *out = nullptr;
  if (n < 1 || !layers || !ins || !outs) return fail(CBS_EINVAL, "graph_create_grouped: bad arguments");
  std::vector<cbs_step> steps(n);
  for (int32_t i = 0; i < n; i++) {
    cbs_status st = check_step(layers[i], ins[i], outs[i], nullptr, "graph_create_grouped", i);
    if (st != CBS_OK) return st;
    steps[i] = cbs_step{layers[i], ins[i], outs[i], nullptr};
  }
  if (!group_of) return capture(steps, plain_launches(steps.size()), out);

  // candidate groups, in order of their first member
  std::vector<int> ids;
  std::map<int, std::vector<int>> members;
  for (int32_t i = 0; i < n; i++) {
    const int g = group_of[i];
    if (g < -1) return fail(CBS_EINVAL, "graph_create_grouped: group_of[%d] = %d (must be >= -1)", (int)i, g);
    if (g < 0) continue;
    if (!members.count(g)) ids.push_back(g);
    members[g].push_back((int)i);
  }
  // Each group's launch takes the place of its last member, so that every
  // producer of a member's input runs before it.  That is only the same
  // computation if no member reads another member's output and no layer
  // between the group's first and last member depends on a member that it
  // would now run before.
  for (int g : ids) {
    const std::vector<int> &m = members[g];
    if ((int)m.size() > kGroupMax)
      return fail(CBS_EINVAL, "graph_create_grouped: group %d has %d layers (at most %d)", g, (int)m.size(),
                  kGroupMax);
    for (int a : m)
      for (int b : m) {
        if (a == b) continue;
        if (overlap(outs[a], out_span(layers[a]), ins[b], in_span(layers[b])) ||
            overlap(outs[a], out_span(layers[a]), outs[b], out_span(layers[b])))
          return fail(CBS_EINVAL, "graph_create_grouped: group %d: layer %d's output overlaps layer %d's input or "
                                  "output", g, a, b);
      }
    for (int j = m.front() + 1; j < m.back(); j++) {
      if (group_of[j] == g) continue;
      for (int a : m) {
        if (a > j) continue;
        if (overlap(outs[a], out_span(layers[a]), ins[j], in_span(layers[j])) ||
            overlap(outs[j], out_span(layers[j]), ins[a], in_span(layers[a])) ||
            overlap(outs[j], out_span(layers[j]), outs[a], out_span(layers[a])))
          return fail(CBS_EINVAL, "graph_create_grouped: group %d: layer %d between its members shares a buffer "
                                  "with member %d", g, j, a);
      }
    }
  }

  // measure each candidate: the members' separate launches against the group
  // under every register-direct and LDS-staged configuration that fits
  std::vector<GraphGroup> info;
  std::map<int, cbs_group *> kept;
  cbs_status st = CBS_OK;
  for (int g : ids) {
    const std::vector<int> &m = members[g];
    GraphGroup gi;
    gi.id = g;
    gi.members = (int)m.size();
    std::vector<cbs_layer *> ml;
    std::vector<const void *> mi;
    std::vector<void *> mo;
    for (int k : m) {
      ml.push_back(layers[k]);
      mi.push_back(ins[k]);
      mo.push_back(outs[k]);
    }
    float sep = 0.f;
    for (size_t k = 0; k < m.size() && st == CBS_OK; k++) {
      float us = 0.f;
      const cbs_layer *L = ml[k];
      const void *in = mi[k];
      void *o = mo[k];
      st = time_replays([&](hipStream_t cs) { return launch(L, in, o, nullptr, cs); }, kGroupTimingReps,
                        kGroupTimingRounds, &us);
      sep += us;
    }
    gi.us_separate = sep;
    cbs_group *best = nullptr;
    float best_us = 1e30f;
    for (int cfg = 0; cfg < num_configs() && st == CBS_OK && m.size() > 1; cfg++) {
      if (config(cfg).lds > 1) continue;
      cbs_group *grp = nullptr;
      if (cbs_group_create(ml.data(), (int32_t)ml.size(), cfg, &grp) != CBS_OK) continue;  // does not fit
      float us = 0.f;
      st = time_replays([&](hipStream_t cs) { return cbs_group_run(grp, mi.data(), mo.data(), cs); },
                        kGroupTimingReps, kGroupTimingRounds, &us);
      if (st == CBS_OK && us < best_us) {
        cbs_group_destroy(best);
        best = grp;
        best_us = us;
      } else {
        cbs_group_destroy(grp);
      }
    }
    if (best) {
      gi.config = best->config;
      gi.us_grouped = best_us;
    }
    if (best && st == CBS_OK && best_us < sep) {
      gi.kept = 1;
      kept[g] = best;
    } else {
      cbs_group_destroy(best);
    }
    info.push_back(gi);
  }
  if (st == CBS_OK && !ids.empty() && info.empty()) st = fail(CBS_EINVAL, "graph_create_grouped: no group");
  if (st != CBS_OK) {
    for (auto &kv : kept) cbs_group_destroy(kv.second);
    return st;
  }
  std::vector<Launch> launches;
  for (int32_t i = 0; i < n; i++) {
    const int g = group_of[i];
    if (g < 0 || !kept.count(g)) {
      Launch l;
      l.step = (int)i;
      launches.push_back(l);
    } else if (members[g].back() == (int)i) {
      Launch l;
      l.group = kept[g];
      l.slots = members[g];
      launches.push_back(l);
    }
  }
  st = capture(steps, launches, out);
  if (st == CBS_OK) (*out)->group_info = info;
  return st;
}

cbs_status cbs_graph_info(const cbs_graph *graph, int32_t *launches, int32_t *groups) {
  if (!graph) return fail(CBS_EINVAL, "graph_info: null graph");
  if (launches) *launches = graph->launches;
  if (groups) *groups = (int32_t)graph->group_info.size();
  return CBS_OK;
}

cbs_status cbs_graph_group_info(const cbs_graph *graph, int32_t i, cbs_graph_group_info_t *info) {
  if (!graph || !info) return fail(CBS_EINVAL, "graph_group_info: null argument");
  if (i < 0 || i >= (int32_t)graph->group_info.size())
    return fail(CBS_EINVAL, "graph_group_info: group %d out of range", (int)i);
  const GraphGroup &g = graph->group_info[i];
  std::memset(info, 0, sizeof(*info));
  info->group_id = g.id;
  info->members = g.members;
  info->kept = g.kept;
  info->config = g.config;
  info->us_grouped = g.us_grouped;
  info->us_separate = g.us_separate;
  return CBS_OK;
}

cbs_status cbs_graph_launch(const cbs_graph *graph, void *stream) {
  if (!graph || !graph->exec) return fail(CBS_EINVAL, "graph_launch: null graph");
  hipError_t e = hipGraphLaunch(graph->exec, (hipStream_t)stream);
  if (e != hipSuccess) return fail(CBS_ELAUNCH, "graph launch: %s", hipGetErrorString(e));
  return CBS_OK;
}

void cbs_graph_destroy(cbs_graph *graph) {
  if (!graph) return;
  if (graph->exec) (void)hipGraphExecDestroy(graph->exec);
  if (graph->graph) (void)hipGraphDestroy(graph->graph);
  for (cbs_group *g : graph->groups) cbs_group_destroy(g);
  for (const cbs_layer *L : graph->layers) L->graph_refs.fetch_sub(1);
  delete graph;
}

cbs_status cbs_layer_info(const cbs_layer *L, cbs_layer_info_t *info) {
  if (!L || !info) return fail(CBS_EINVAL, "layer_info: null argument");
  std::memset(info, 0, sizeof(*info));
  const cbs_conv_desc &d = L->d;
  info->c_in_pad = L->cin_pad;
  info->c_out_pad = L->cout_pad;
  info->oh = L->oh;
  info->ow = L->ow;
  info->out_row_pitch = L->pitch;
  info->dtype = d.dtype;
  const int64_t esz = d.dtype == CBS_F32 ? 4 : 1;
  const int64_t osz = d.out_dtype == CBS_F32 ? 4 : 1;
  info->in_bytes = (int64_t)d.n * d.h * d.w * L->in_cs * esz;
  info->out_bytes = (int64_t)d.n * L->oh * L->pitch * L->out_cs * osz;
  info->res_bytes = (int64_t)d.n * L->oh * L->ow * L->res_cs * osz;
  info->in2_bytes = (int64_t)d.n * d.h * d.w * L->in2_cs * 4;
  const int64_t kk = (int64_t)d.k * d.k;
  const int64_t out_elems = (int64_t)d.n * L->oh * L->ow * d.c_out;
  info->flops = 2 * out_elems * d.c_in * kk;
  info->alg_bytes = (int64_t)d.n * d.h * d.w * d.c_in * esz + (int64_t)d.c_out * d.c_in * kk * esz +
                    out_elems * osz * (L->res_cs ? 2 : 1) + 8 * (int64_t)d.c_out;
  info->config = L->config;
  info->splitk = L->splitk;
  int pxt, cot;
  tiles_of(L, L->config, &pxt, &cot);
  info->grid = pxt * cot * L->splitk;
  const KernelConfig &c = config(L->config);
  info->threads = 64 * c.wco * c.wpx * c.wk;
  std::snprintf(info->config_name, sizeof(info->config_name), "%s/sk%d", c.name, L->splitk);
  return CBS_OK;
}

cbs_status cbs_layer_set_config(cbs_layer *L, int32_t cfg, int32_t splitk) {
  if (!L) return fail(CBS_EINVAL, "set_config: null layer");
  if (cfg < 0 || cfg >= num_configs()) return fail(CBS_EINVAL, "config %d out of range", cfg);
  if (splitk < 0) return fail(CBS_EINVAL, "splitk %d < 0", splitk);
  if (splitk == 0) splitk = 1;
  if (!config_fits(L, cfg, splitk))
    return fail(CBS_EUNSUPPORTED, "config %s with splitk %d does not fit this layer", config(cfg).name, splitk);
  const int old_cfg = L->config, old_sk = L->splitk;
  L->config = cfg;
  L->splitk = splitk;
  cbs_status st = setup_splitk(L);
  if (st != CBS_OK) {
    L->config = old_cfg;
    L->splitk = old_sk;
    (void)setup_splitk(L);
  }
  return st;
}

int32_t cbs_num_configs(void) { return num_configs(); }

}  // extern "C"

namespace {

// Create-time tuning results, per device and per everything that changes a
// kernel's timing: shape, dtype, epilogue variant and channel strides.
using TuneKey = std::tuple<int, int, int, int, int, int, int, int, int, int, int, int, int, int>;
std::mutex g_tune_mu;
std::map<TuneKey, Choice> g_tune_cache;

TuneKey tune_key(const cbs_layer *L) {
  const cbs_conv_desc &d = L->d;
  return TuneKey{L->device, d.n, d.c_in, d.c_out, d.h, d.w, d.k, d.stride, d.pad, d.dtype, L->variant, L->in_cs,
                 L->out_cs, L->res_cs};
}

// Time per launch of `iters` back-to-back launches, captured as one graph and
// replayed (the best of three replays after a warm-up one), in ms: the way a
// captured list runs them.  An eager launch costs the GPU about 3 us of its
// own, which would hide the differences between configurations of small layers.
cbs_status time_config(cbs_layer *L, const void *in, void *out, const void *res, int iters, float *ms) {
  float us = 0.f;
  const cbs_status s = time_replays([&](hipStream_t cs) { return launch(L, in, out, res, cs); }, iters, 3, &us);
  *ms = us * 1e-3f;
  return s;
}

}  // namespace

extern "C" {

cbs_status cbs_layer_autotune(cbs_layer *L, const void *in, void *out, const void *residual, int32_t iters,
                              int32_t flags, void *stream, int32_t *config_out, int32_t *splitk_out) {
  cbs_status st = check_step(L, in, out, residual, "layer_autotune", 0);
  if (st != CBS_OK) return st;
  if (iters < 0 || iters > 100000) return fail(CBS_EINVAL, "layer_autotune: iters %d out of range", iters);
  if (flags & ~CBS_TUNE_FORCE) return fail(CBS_EINVAL, "layer_autotune: unknown flags 0x%x", flags);
  if (iters == 0) iters = 20;
  const TuneKey key = tune_key(L);
  Choice best{L->config, L->splitk};
  bool cached = false;
  if (!(flags & CBS_TUNE_FORCE)) {
    std::lock_guard<std::mutex> lk(g_tune_mu);
    auto it = g_tune_cache.find(key);
    if (it != g_tune_cache.end()) {
      best = it->second;
      cached = true;
    }
  }
  if (!cached) {
    // wait for the caller's stream: the timing runs on a private one
    if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess)
      return fail(CBS_EDEVICE, "layer_autotune: stream synchronisation failed");
    const int old_cfg = L->config, old_sk = L->splitk;
    float best_ms = 1e30f;
    st = CBS_OK;
    for (int cfg = 0; cfg < num_configs() && st == CBS_OK; cfg++) {
      for (int sk : {1, 2, 3, 4}) {
        if (!config_fits(L, cfg, sk)) continue;
        if (sk > 1) {  // cross-workgroup split-K only for grids that leave CUs idle
          int pxt, cot;
          tiles_of(L, cfg, &pxt, &cot);
          if ((long)pxt * cot >= 256) continue;
        }
        // a live graph holds the workspace's address: only what fits it
        if (L->graph_refs.load() > 0 && !splitk_fits_workspace(L, cfg, sk)) continue;
        L->config = cfg;
        L->splitk = sk;
        st = setup_splitk(L);
        float ms = 0.f;
        if (st == CBS_OK) st = time_config(L, in, out, residual, iters, &ms);
        if (st != CBS_OK) break;
        if (ms < best_ms) {
          best_ms = ms;
          best = {cfg, sk};
        }
      }
    }
    if (st != CBS_OK) {
      L->config = old_cfg;
      L->splitk = old_sk;
      (void)setup_splitk(L);
      return st;
    }
    std::lock_guard<std::mutex> lk(g_tune_mu);
    g_tune_cache[key] = best;
  }
  L->config = best.config;
  L->splitk = best.splitk;
  st = setup_splitk(L);
  if (st != CBS_OK) return st;
  if (config_out) *config_out = best.config;
  if (splitk_out) *splitk_out = best.splitk;
  return CBS_OK;
}

void cbs_autotune_clear_cache(void) {
  std::lock_guard<std::mutex> lk(g_tune_mu);
  g_tune_cache.clear();
}

const char *cbs_config_name(int32_t cfg) {
  if (cfg < 0 || cfg >= num_configs()) return nullptr;
  return config(cfg).name;
}

const char *cbs_last_error(void) { return g_last_error.c_str(); }

cbs_status cbs_pack_nhwc_f32(const float *nchw, float *nhwc, int32_t n, int32_t c, int32_t h, int32_t w,
                             int32_t c_pad, void *stream) {
  if (!nchw || !nhwc) return fail(CBS_EINVAL, "pack: null buffer");
  if (n < 0 || c < 1 || h < 0 || w < 0 || c_pad < c || c_pad % 4 != 0)
    return fail(CBS_EINVAL, "pack: bad sizes");
  if ((double)n * h * w * c_pad >= 2147483647.0) return fail(CBS_EUNSUPPORTED, "pack: tensor above 2^31 elements");
  hipError_t e = launch_pack_nhwc_f32(nchw, nhwc, n, c, h * w, c_pad, (hipStream_t)stream);
  if (e != hipSuccess) return fail(CBS_ELAUNCH, "pack launch: %s", hipGetErrorString(e));
  return CBS_OK;
}

cbs_status cbs_quantize_nhwc_i8(const float *nchw, int8_t *nhwc, float s_x, int32_t n, int32_t c, int32_t h,
                                int32_t w, int32_t c_pad, void *stream) {
  if (!nchw || !nhwc) return fail(CBS_EINVAL, "quantize: null buffer");
  if (!(s_x > 0.0f) || !std::isfinite(s_x)) return fail(CBS_EINVAL, "quantize: s_x must be finite and > 0");
  if (n < 0 || c < 1 || h < 0 || w < 0 || c_pad < c || c_pad % 4 != 0)
    return fail(CBS_EINVAL, "quantize: bad sizes");
  if ((double)n * h * w * c_pad >= 2147483647.0) return fail(CBS_EUNSUPPORTED, "quantize: tensor above 2^31 elements");
  hipError_t e = launch_quantize_nhwc_i8(nchw, nhwc, s_x, n, c, h * w, c_pad, (hipStream_t)stream);
  if (e != hipSuccess) return fail(CBS_ELAUNCH, "quantize launch: %s", hipGetErrorString(e));
  return CBS_OK;
}

cbs_status cbs_quantize_nhwc_u8(const float *nchw, uint8_t *nhwc, float s_x, int32_t z, int32_t n, int32_t c,
                                int32_t h, int32_t w, int32_t c_pad, void *stream) {
  if (!nchw || !nhwc) return fail(CBS_EINVAL, "quantize_u8: null buffer");
  if (!(s_x > 0.0f) || !std::isfinite(s_x)) return fail(CBS_EINVAL, "quantize_u8: s_x must be finite and > 0");
  if (z < 0 || z > 255) return fail(CBS_EINVAL, "quantize_u8: zero point %d not in [0, 255]", z);
  if (n < 0 || c < 1 || h < 0 || w < 0 || c_pad < c || c_pad % 4 != 0)
    return fail(CBS_EINVAL, "quantize_u8: bad sizes");
  if ((double)n * h * w * c_pad >= 2147483647.0)
    return fail(CBS_EUNSUPPORTED, "quantize_u8: tensor above 2^31 elements");
  hipError_t e = launch_quantize_nhwc_u8(nchw, nhwc, s_x, z, n, c, h * w, c_pad, (hipStream_t)stream);
  if (e != hipSuccess) return fail(CBS_ELAUNCH, "quantize_u8 launch: %s", hipGetErrorString(e));
  return CBS_OK;
}

cbs_status cbs_run_layer_raw_acc(const cbs_layer *L, const void *in, int32_t *acc, void *stream) {
  if (!L || !in || !acc) return fail(CBS_EINVAL, "run_layer_raw_acc: null layer or buffer");
  if (L->raw_variant < 0) return fail(CBS_EINVAL, "run_layer_raw_acc: not an INT8 layer");
  if ((double)L->d.n * L->oh * L->pitch * L->cout_pad * 4.0 >= 2147483648.0 - 64.0)
    return fail(CBS_EUNSUPPORTED, "run_layer_raw_acc: accumulator buffer above 2^31 bytes");
  return launch(L, in, acc, nullptr, stream, true);
}

cbs_status cbs_get_qweights(const cbs_layer *L, int8_t *q_oihw, double *s_w) {
  if (!L) return fail(CBS_EINVAL, "get_qweights: null layer");
  if (L->d.dtype == CBS_F32) return fail(CBS_EINVAL, "get_qweights: not an INT8 layer");
  if (q_oihw) std::memcpy(q_oihw, L->h_qw.data(), L->h_qw.size());
  if (s_w) std::memcpy(s_w, L->h_sw.data(), L->h_sw.size() * sizeof(double));
  return CBS_OK;
}

cbs_status cbs_get_folded(const cbs_layer *L, float *w_oihw, float *bias) {
  if (!L) return fail(CBS_EINVAL, "get_folded: null layer");
  if (w_oihw) {
    if (L->d.dtype != CBS_F32) return fail(CBS_EINVAL, "get_folded: INT8 layers keep quantised weights");
    std::memcpy(w_oihw, L->h_wfold.data(), L->h_wfold.size() * sizeof(float));
  }
  if (bias) std::memcpy(bias, L->h_bias.data(), L->h_bias.size() * sizeof(float));
  return CBS_OK;
}

}  // extern "C"
