#pragma once
// conv_kernels.h -- gfx950 kernels of libcbs: implicit-GEMM fused Conv2d +
// folded BN + SiLU on MFMA (fp32 and int8), as templates instantiated once
// per variant by cbs_variant.hip.
//
// The convolution is computed as the implicit GEMM described on the vision-rs
// "YOLO26N Inference Optimisation" page, section "NHWC migration -- What NHWC
// is and why it matters": rows = output pixels (n, oh, ow), K = (kh, kw, c_in)
// with c_in contiguous, columns = output channels.  Here the MFMA "A" operand
// is the weights (16 output channels per block) and the "B" operand is the
// gathered activations (16 output pixels per block), so every lane of the
// accumulator holds 4 consecutive output channels of one pixel and the
// epilogue stores one 16-byte NHWC vector per lane.
//
// K is walked in "chunks": 4 consecutive input channels of one tap (fp32 and
// small-channel int8) or 16 (int8 with C_in_pad % 16 == 0).  At each K step,
// lane group g = lane/16 of a wave loads chunk (4*step + g) (times 4 chunks
// for the small-channel int8 gather); the weights were laid out at create in
// exactly this order ("fragment order"), so each weight load is one
// contiguous 1 KiB read per wave.  Chunks that fall in the zero padding of
// the image, past K, or on pixels past the end of the tile are not loaded
// and count as zeros, which is the zero padding of the definition.
//
// Output pixels are indexed by their logical position m = (n*OH + oh)*OW + ow
// and stored at ((n*OH + oh)*pitch + ow), so a tail tile can never write into
// the guard pixels of a row or into the next row: the overflow documented in
// the same page's section "Bug fixed: TMA overflow" cannot happen by
// construction, whatever the tile shape.
//
// Small-M layers (batch 1 at 20x20 or 40x40) split K across the waves of a
// workgroup (reduced in LDS) and, optionally, across workgroups: each
// workgroup writes its partial tile to a workspace, and the last one to
// arrive (atomic ticket per tile) sums all partials in split order, runs the
// epilogue and re-arms the ticket, so no memset is ever needed and the result
// is bitwise deterministic.
#include "cbs_internal.h"
#include "conv_configs.h"


namespace cbs {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// Operand and epilogue traits of a variant: VEC = 4-channel chunks per lane
// and K step (int8 small-channel gather), ESIZE = bytes per activation, RAW =
// store int32 accumulators, X = general epilogue (act / residual / byte out),
// U8 = asymmetric uint8 activations.
template <int VAR> struct Var;
template <> struct Var<VAR_F32> {
  using Frag = f32x4; using Acc = f32x4;
  static constexpr int VEC = 1, ESIZE = 4;
  static constexpr bool I8 = false, RAW = false, X = false, U8 = false;
};
template <> struct Var<VAR_I8_C16> {
  using Frag = i32x4; using Acc = i32x4;
  static constexpr int VEC = 1, ESIZE = 1;
  static constexpr bool I8 = true, RAW = false, X = false, U8 = false;
};
template <> struct Var<VAR_I8_C4> {
  using Frag = i32x4; using Acc = i32x4;
  static constexpr int VEC = 4, ESIZE = 1;
  static constexpr bool I8 = true, RAW = false, X = false, U8 = false;
};
template <> struct Var<VAR_I8_C16_RAW> : Var<VAR_I8_C16> { static constexpr bool RAW = true; };
template <> struct Var<VAR_I8_C4_RAW> : Var<VAR_I8_C4> { static constexpr bool RAW = true; };
template <> struct Var<VAR_F32_X> : Var<VAR_F32> { static constexpr bool X = true; };
template <> struct Var<VAR_I8_C16_X> : Var<VAR_I8_C16> { static constexpr bool X = true; };
template <> struct Var<VAR_I8_C4_X> : Var<VAR_I8_C4> { static constexpr bool X = true; };
template <> struct Var<VAR_U8_C16_X> : Var<VAR_I8_C16> { static constexpr bool X = true, U8 = true; };
template <> struct Var<VAR_U8_C4_X> : Var<VAR_I8_C4> { static constexpr bool X = true, U8 = true; };
template <> struct Var<VAR_U8_C16_RAW> : Var<VAR_I8_C16> { static constexpr bool RAW = true, U8 = true; };
template <> struct Var<VAR_U8_C4_RAW> : Var<VAR_I8_C4> { static constexpr bool RAW = true, U8 = true; };

// uint8 codes q enter the signed int8 MFMA as q ^ 0x80 = q - 128.
constexpr int kU8Flip = (int)0x80808080u;


// Buffer resource word 3 (data format) for the gfx9 family, and an offset
// that every buffer of this library lies below (sizes are checked < 2^31 at
// create): loads at it return zero.
constexpr int kRsrcWord3 = 0x00020000;
constexpr unsigned kOutOfRange = 0x80000000u;

// A compile-time flag passed to a generic lambda.
template <bool B> struct BoolC { static constexpr bool value = B; };

// SiLU(z) = z / (1 + e^-z), with the hardware exponential and reciprocal
// (each within about one ulp): a correctly rounded division costs ten
// instructions per value, which made the epilogue of the small layers the
// largest VALU cost of the kernel.  For z < -88, e^-z is +inf, the reciprocal
// 0 and y = -0 (the true value is below 1e-36 in magnitude).
__device__ __forceinline__ float silu_f(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// Kernel arguments arrive through scalar loads from the argument block.  Left
// to itself the compiler re-reads the ones that only the epilogue uses after
// the main loop (to free SGPRs), which puts one more dependent memory round
// trip at the end of every launch.  Pinning them at entry (an empty asm that
// "modifies" the value, so it cannot be re-read) keeps them in SGPRs from the
// start.  The build checks that no argument load follows the first MFMA.
template <class T>
__device__ __forceinline__ void pin_sgpr(T &v) {
  asm volatile("" : "+s"(v));
}

// A pinned pointer no longer carries the compiler's knowledge that kernel
// pointer arguments point to global memory, so every access through one names
// the global address space explicitly (otherwise it becomes a slower FLAT
// access, which also waits on the LDS counter).
#define CBS_GLOBAL __attribute__((address_space(1)))
template <class T>
__device__ __forceinline__ CBS_GLOBAL T *gmem(const void *ptr) {
  return (CBS_GLOBAL T *)ptr;
}

// Every argument the kernels read, pinned at entry: the compiler then issues
// all argument loads at once and waits for them once, instead of spreading
// them over two or three dependent rounds (it sinks loads towards their first
// use), each costing a memory round trip before the first operand load.
template <bool U8>
__device__ __forceinline__ void pin_common_args(ConvParams &p, int &nblocks) {
  pin_sgpr(nblocks);  // the grid size comes from the dispatch's own argument area
  pin_sgpr(p.x);
  pin_sgpr(p.wfrag);
  pin_sgpr(p.bias);
  pin_sgpr(p.dq);
  pin_sgpr(p.out);
  pin_sgpr(p.res);
  if (U8) pin_sgpr(p.corr);
  pin_sgpr(p.H);
  pin_sgpr(p.W);
  pin_sgpr(p.x_cs);
  pin_sgpr(p.k);
  pin_sgpr(p.stride);
  pin_sgpr(p.pad);
  pin_sgpr(p.chunk_ch);
  pin_sgpr(p.chunks_per_tap);
  pin_sgpr(p.cpt_magic);
  pin_sgpr(p.total_chunks);
  pin_sgpr(p.steps);
  pin_sgpr(p.co_blocks);
  pin_sgpr(p.x_bytes);
  pin_sgpr(p.w_bytes);
  pin_sgpr(p.cout_pad);
  pin_sgpr(p.out_cs);
  pin_sgpr(p.res_cs);
  pin_sgpr(p.res_bytes);
  pin_sgpr(p.out_bytes);
  pin_sgpr(p.act);
  pin_sgpr(p.out_q);
  pin_sgpr(p.out_scale);
  pin_sgpr(p.out_rcp);
  pin_sgpr(p.out_zp);
  pin_sgpr(p.out_lo);
  pin_sgpr(p.out_hi);
  pin_sgpr(p.res_scale);
  pin_sgpr(p.res_xor);
  pin_sgpr(p.res_zp);
  pin_sgpr(p.OH);
  pin_sgpr(p.OW);
  pin_sgpr(p.pitch);
}

// The pixel-tiled kernels (conv_igemm, conv_lds) also decompose pixel and
// workgroup indices; conv_igemm alone reduces split-K partial tiles.
template <bool U8>
__device__ __forceinline__ void pin_tiled_args(ConvParams &p, int &nblocks, bool splitk_args) {
  pin_common_args<U8>(p, nblocks);
  pin_sgpr(p.M);
  pin_sgpr(p.inner_tiles);
  pin_sgpr(p.px_inner);
  pin_sgpr(p.div_ow.magic);
  pin_sgpr(p.div_ow.shift);
  pin_sgpr(p.div_oh.magic);
  pin_sgpr(p.div_oh.shift);
  pin_sgpr(p.div_inner.magic);
  pin_sgpr(p.div_inner.shift);
  if (splitk_args) {
    pin_sgpr(p.ws);
    pin_sgpr(p.counters);
    pin_sgpr(p.splitk);
    pin_sgpr(p.steps_per_split);
    pin_sgpr(p.div_sk.magic);
    pin_sgpr(p.div_sk.shift);
  }
}

// conv_halo: the tile grid and the LDS halo layout.
template <bool U8>
__device__ __forceinline__ void pin_halo_args(ConvParams &p, int &nblocks) {
  pin_common_args<U8>(p, nblocks);
  pin_sgpr(p.cin_pad);
  pin_sgpr(p.tiles_x);
  pin_sgpr(p.tiles_y);
  pin_sgpr(p.halo_bytes);
  pin_sgpr(p.div_tx.magic);
  pin_sgpr(p.div_tx.shift);
  pin_sgpr(p.div_ty.magic);
  pin_sgpr(p.div_ty.shift);
  pin_sgpr(p.halo_cq);
  pin_sgpr(p.div_hcq.magic);
  pin_sgpr(p.div_hcq.shift);
  pin_sgpr(p.div_hwd.magic);
  pin_sgpr(p.div_hwd.shift);
}

__device__ __forceinline__ int fdiv(int n, FastDiv f) {
  return (int)((__umulhi((unsigned)n, f.magic) + (unsigned)n) >> f.shift);
}

// Output tile of a logical workgroup index.  Each XCD runs a contiguous range
// of logical indices (see the remap in the kernels), so the inner dimension
// decides what one XCD's L2 shares: with channel tiles inner (the default)
// an XCD takes a few pixel tiles with all their channel tiles and fetches the
// whole weight array; with pixel tiles inner it takes a few channel tiles
// with all pixels and fetches only their weights.  The host picks pixel tiles
// inner when the weights outweigh the input.
__device__ __forceinline__ void tile_of(const ConvParams &p, int t, int &px_tile, int &co_tile) {
  const int outer = fdiv(t, p.div_inner);
  const int inner = t - outer * p.inner_tiles;
  px_tile = p.px_inner ? inner : outer;
  co_tile = p.px_inner ? outer : inner;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void *)base, 0, (int)bytes, kRsrcWord3);
}

// Output stores are buffer stores at system scope (sc0 sc1: written through
// the L2 to memory).  The line stays in the L2 for a next layer that reads it,
// but it is not dirty when the kernel ends, so the end-of-kernel write-back
// of the L2 has less to do: measured 2-3% shorter lists at batch 1 than with
// plain stores (non-temporal stores were faster at batch 16 but slower for
// chained layers and int8 output).  The range is the layer's output buffer,
// so a store outside it is dropped.
constexpr int kStoreWriteThrough = 1 | 16;  // sc0 | sc1
constexpr int kLoadBypass = 1 | 16;         // sc0 | sc1 on a load: served from memory, not a cache
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
// Hand-over of split-K partial tiles from the workgroups that compute them to
// the last one to arrive, which may run on another XCD (another L2).  By
// default the partials are written through to memory, each wave waits for its
// stores to complete before the ticket is taken, and the last workgroup reads
// them with loads that bypass the caches: no cache-wide operation.  Built with
// CBS_SPLITK_FENCED=1, the hand-over is the HIP memory model's own instead:
// plain stores and loads, an agent-scope release fence in every wave before
// the ticket and an agent-scope acquire fence after it (a write-back and an
// invalidation of the L2), kept to measure what the fences cost.
#ifndef CBS_SPLITK_FENCED
#define CBS_SPLITK_FENCED 0
#endif
constexpr int kPartialStore = CBS_SPLITK_FENCED ? 0 : kStoreWriteThrough;
constexpr int kPartialLoad = CBS_SPLITK_FENCED ? 0 : kLoadBypass;
// every wave, after its partial stores, before the workgroup barrier and the ticket
__device__ __forceinline__ void partials_published() {
  if constexpr (CBS_SPLITK_FENCED)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  else
    __builtin_amdgcn_s_waitcnt(0);  // every partial store of this wave has completed
}
// every wave of the last workgroup, after the barrier that follows the ticket
__device__ __forceinline__ void partials_acquired() {
  if constexpr (CBS_SPLITK_FENCED) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

template <class T>
__device__ __forceinline__ void store16(const ConvParams &p, unsigned byte_off, T v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rsrc(p.out, p.out_bytes), byte_off, 0,
                                         kStoreWriteThrough);
}
__device__ __forceinline__ void store4(const ConvParams &p, unsigned byte_off, unsigned v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, rsrc(p.out, p.out_bytes), byte_off, 0, kStoreWriteThrough);
}

// The fused epilogue of one lane: output channels co0 .. co0+3 of one pixel.
// z holds the pre-activation values (accumulator + folded bias, dequantised
// for int8); opix is the pixel's storage index ((n*OH + oh)*pitch + ow) and m
// its logical index ((n*OH + oh)*OW + ow), which addresses the dense-row
// residual.  Order: activation, then the residual add, then (byte output) the
// quantiser of the next layer's input, so the codes are exactly those the
// graph-entry quantiser would produce from this layer's fp32 output.  act, the
// residual and the output type are kernel arguments: every branch here is
// wave-uniform.
template <bool X>
__device__ __forceinline__ void epilogue_store(const ConvParams &p, __amdgpu_buffer_rsrc_t rr, f32x4 z, int opix,
                                               int m, int co0, bool ok = true) {
  f32x4 y;
  // plain: SiLU, fp32 store (also the general variant's path when no option is set)
  if (!X || (p.act == ACT_SILU && !p.res_cs && !p.out_q)) {
#pragma unroll
    for (int i = 0; i < 4; i++) y[i] = silu_f(z[i]);
    store16(p, ok ? (unsigned)(opix * p.out_cs + co0) * 4u : kOutOfRange, y);
    return;
  }
  if (p.act == ACT_NONE) {
    y = z;
  } else {
#pragma unroll
    for (int i = 0; i < 4; i++) y[i] = silu_f(z[i]);
  }
  if (p.res_cs) {
    const unsigned e = (unsigned)(m * p.res_cs + co0);  // element index (masked lanes read nothing)
    if (p.out_q) {
      // byte codes: int8 as (b ^ 0x80) - 128, uint8 as b - z_r (both exact in fp32)
      const unsigned w = __builtin_amdgcn_raw_buffer_load_b32(rr, ok ? e : kOutOfRange, 0, 0) ^ p.res_xor;
#pragma unroll
      for (int i = 0; i < 4; i++) y[i] += p.res_scale * ((float)((w >> (8 * i)) & 0xffu) - p.res_zp);
    } else {
      y += __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rr, ok ? e * 4u : kOutOfRange, 0, 0));
    }
  }
  const unsigned o = (unsigned)(opix * p.out_cs + co0);  // element index; byte offsets stay below 2^31
  if (p.out_q) {
    // q = clamp(rne(fp32(y / s)) + z_y, lo, hi) with the correctly rounded
    // quotient from Markstein's correction step: with r = RN(1/s), q0 = RN(y r),
    // e = y - q0 s (exact in one FMA), RN(q0 + e r) = RN(y / s) for quotients
    // in the normal range.  y is first limited to +-256 s, which changes no
    // code (beyond it every code is clamped to an end of the range anyway) and
    // keeps q0 finite.
    const float s = p.out_scale, r = p.out_rcp, lim = 256.0f * s;
    unsigned word = 0;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const float yc = fminf(fmaxf(y[i], -lim), lim);
      const float q0 = yc * r;
      const float e = __builtin_fmaf(-q0, s, yc);
      float t = rintf(__builtin_fmaf(e, r, q0)) + p.out_zp;
      t = fminf(fmaxf(t, p.out_lo), p.out_hi);
      word |= ((unsigned)((int)t & 0xff)) << (8 * i);
    }
    store4(p, ok ? o : kOutOfRange, word);
  } else {
    store16(p, ok ? o * 4u : kOutOfRange, y);
  }
}

// uint8 input: a correction, added to each block's sum over K, turns the sum
// the MFMAs form into the one of the definition.  The gathered operand is q - 128
// inside the image and -128 on the padding taps (out-of-range loads read 0,
// flipped like every other byte), so with Wsum[co] the sum of the channel's
// int8 weights and Win[co] the sum of its weights on the taps inside the image,
//   sum_in q_w (q - z) = MFMA sum + 128 Wsum[co] - z Win[co].
// Win depends on the pixel only through which window rows and columns lie
// inside the image: bit i of the row mask says row i does, likewise for the
// columns, and the class rows * 8 + cols indexes a [64][co_blocks*16] table
// set up at create.
__device__ __forceinline__ int border_class(const ConvParams &p, int iy0, int ix0) {
  const unsigned kmask = (1u << p.k) - 1u;
  unsigned rm = 0, cm = 0;
#pragma unroll
  for (int i = 0; i < 3; i++) {
    rm |= (unsigned)((unsigned)(iy0 + i) < (unsigned)p.H) << i;
    cm |= (unsigned)((unsigned)(ix0 + i) < (unsigned)p.W) << i;
  }
  return (int)((rm & kmask) * 8u + (cm & kmask));
}

// Correction of the accumulator of output channels co0 .. co0+3 at a pixel of
// border class cls (zero unless the variant has uint8 input).  The kernels
// fetch it with the epilogue operands and add it once the K slices of the block
// are summed, so that no MFMA waits for it.
template <class V>
__device__ __forceinline__ typename V::Acc zp_correction(const ConvParams &p, int cls, int co0) {
  if constexpr (V::U8) {
    const __amdgpu_buffer_rsrc_t cr = rsrc(p.corr, (unsigned)(64 * p.co_blocks * 64));
    return __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                         cr, (unsigned)((cls * p.co_blocks * 16 + co0) * 4), 0, 0));
  } else {
    return typename V::Acc{};
  }
}

// Decoded K chunk: tap offset (dy, dx) and first channel.
struct Chunk {
  int dy, dx, ci;
  bool ok;
};

__device__ __forceinline__ Chunk decode_chunk(const ConvParams &p, int c) {
  Chunk r;
  const int tap = (int)(((unsigned)c * p.cpt_magic) >> 20);
  r.ci = (c - tap * p.chunks_per_tap) * p.chunk_ch;
  r.dy = (p.k == 1) ? 0 : ((tap * 11) >> 5);  // tap / 3 for tap < 9
  r.dx = tap - r.dy * p.k;
  r.ok = c < p.total_chunks;
  return r;
}

// The same for the column-pair halo kernel: taps run over a 3 x 4 window.
__device__ __forceinline__ Chunk decode_chunk_pair(const ConvParams &p, int c) {
  Chunk r;
  const int tap = (int)(((unsigned)c * p.cpt_magic) >> 20);
  r.ci = (c - tap * p.chunks_per_tap) * p.chunk_ch;
  r.dy = tap >> 2;
  r.dx = tap & 3;
  r.ok = c < p.total_chunks;
  return r;
}

// Workgroups are dispatched round-robin over the 8 XCDs; this remaps a
// workgroup id to a logical tile so that each XCD receives a contiguous range
// of logical tiles (the co tiles and K splits of one pixel tile then share
// that XCD's L2).
__device__ __forceinline__ int xcd_major(int nblocks, int bid) {
  const int per = nblocks >> 3, rem = nblocks & 7, xcd = bid & 7, loc = bid >> 3;
  return xcd * per + min(xcd, rem) + loc;  // branch-free form of the XCD-major order
}

// Workgroup `bid` of a grid of nblocks runs logical tile
// xcd_major(nblocks, bid) - first of the layer described by p (its pixel
// tile, channel tile and K split); first is the layer's first logical tile
// in a grouped launch, 0 otherwise.
template <int VAR, int CB, int PB, int WCO, int WPX, int WK, int PF>
__device__ __forceinline__ void igemm_workgroup(const ConvParams &p, const int nblocks, const int bid,
                                                const int first) {
  using V = Var<VAR>;
  using Frag = typename V::Frag;
  using Acc = typename V::Acc;
  const int lane = threadIdx.x & 63;
  // The wave index is made explicitly wave-uniform: every condition that
  // guards an MFMA below depends only on it, so it compiles to a scalar
  // branch.  (MFMA ignores EXEC; an MFMA under a per-lane mask would run.)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wk = wave % WK;
  const int wco = (wave / WK) % WCO;
  const int wpx = wave / (WK * WCO);
  const int slot = wco + WCO * wpx;
  const int r = lane & 15, g = lane >> 4;

  const int logical = xcd_major(nblocks, bid) - first;
  const int tile = fdiv(logical, p.div_sk);
  const int split = logical - tile * p.splitk;
  int px_tile, co_tile;
  tile_of(p, tile, px_tile, co_tile);

  // The 16-pixel blocks of this wave: lane r owns pixel r of each block.
  int pixbase[PB], iy0[PB], ix0[PB], outpix[PB];
  bool mval[PB];
#pragma unroll
  for (int b = 0; b < PB; b++) {
    const int m = ((px_tile * WPX + wpx) * PB + b) * 16 + r;
    mval[b] = m < p.M;
    const int mm = mval[b] ? m : 0;
    const int t = fdiv(mm, p.div_ow);
    const int ow = mm - t * p.OW;
    const int n = fdiv(t, p.div_oh);
    const int oh = t - n * p.OH;
    iy0[b] = oh * p.stride - p.pad;
    ix0[b] = ow * p.stride - p.pad;
    pixbase[b] = (n * p.H + iy0[b]) * p.W + ix0[b];
    outpix[b] = (n * p.OH + oh) * p.pitch + ow;
  }
  const int cob0 = (co_tile * WCO + wco) * CB;
  // Weights: a per-lane offset of the block (out of range for blocks past the
  // end) plus a wave-uniform step offset in the scalar operand.
  unsigned wvoff[CB];
#pragma unroll
  for (int cb = 0; cb < CB; cb++)
    wvoff[cb] = (cob0 + cb) < p.co_blocks ? ((unsigned)((cob0 + cb) * p.steps) * 64u + (unsigned)lane) * 16u
                                          : kOutOfRange;
  // Epilogue operands are fetched now, so their latency overlaps the main loop
  // (out-of-range channels read as zero).
  f32x4 ep_bias[CB], ep_dq[CB];
  Acc ep_corr[CB][PB];  // uint8 input: the zero-point correction of each block
  {
    const __amdgpu_buffer_rsrc_t br =
        __builtin_amdgcn_make_buffer_rsrc((void *)p.bias, 0, (int)(p.co_blocks * 64), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t dr =
        __builtin_amdgcn_make_buffer_rsrc((void *)p.dq, 0, V::I8 ? (int)(p.co_blocks * 64) : 0, kRsrcWord3);
#pragma unroll
    for (int cb = 0; cb < CB; cb++) {
      const unsigned off = (unsigned)(((cob0 + cb) * 16 + 4 * g) * 4);
      ep_bias[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
      ep_dq[cb] = f32x4{1.f, 1.f, 1.f, 1.f};
      if constexpr (!V::RAW) ep_bias[cb] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(br, off, 0, 0));
      if constexpr (V::I8 && !V::RAW) ep_dq[cb] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(dr, off, 0, 0));
    }
#pragma unroll
    for (int b = 0; b < PB; b++) {
      const int cls = V::U8 ? border_class(p, iy0[b], ix0[b]) : 0;
#pragma unroll
      for (int cb = 0; cb < CB; cb++) ep_corr[cb][b] = zp_correction<V>(p, cls, (cob0 + cb) * 16 + 4 * g);
    }
  }
  const int s_begin = split * p.steps_per_split;
  const int s_end = min(p.steps, s_begin + p.steps_per_split);

  // Every operand load is a branch-free buffer load: an out-of-range byte
  // offset returns zeros, which supplies the image's zero padding, the pixel
  // tail, the K tail and output-channel blocks past the end without any
  // condition around a load (so the compiler can count loads in flight and
  // wait only for the oldest one).
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc((void *)p.wfrag, 0, (int)p.w_bytes, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc((void *)p.x, 0, (int)p.x_bytes, kRsrcWord3);
  auto load = [&](int s, Frag(&aa)[CB], Frag(&bb)[PB]) {
#pragma unroll
    for (int cb = 0; cb < CB; cb++)
      aa[cb] = __builtin_bit_cast(Frag, __builtin_amdgcn_raw_buffer_load_b128(wr, wvoff[cb], s * 1024, 0));
    if constexpr (V::VEC == 1) {
      const Chunk c = decode_chunk(p, s * 4 + g);
      const int doff = (c.dy * p.W + c.dx) * p.x_cs + c.ci;
#pragma unroll
      for (int b = 0; b < PB; b++) {
        const int iy = iy0[b] + c.dy, ix = ix0[b] + c.dx;
        const bool v = c.ok && mval[b] && (unsigned)iy < (unsigned)p.H && (unsigned)ix < (unsigned)p.W;
        const unsigned off = v ? (unsigned)(pixbase[b] * p.x_cs + doff) * (unsigned)V::ESIZE : kOutOfRange;
        bb[b] = __builtin_bit_cast(Frag, __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0));
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const Chunk c = decode_chunk(p, (s * 4 + g) * 4 + j);
        const int doff = (c.dy * p.W + c.dx) * p.x_cs + c.ci;
#pragma unroll
        for (int b = 0; b < PB; b++) {
          const int iy = iy0[b] + c.dy, ix = ix0[b] + c.dx;
          const bool v = c.ok && mval[b] && (unsigned)iy < (unsigned)p.H && (unsigned)ix < (unsigned)p.W;
          const unsigned off = v ? (unsigned)(pixbase[b] * p.x_cs + doff) : kOutOfRange;
          bb[b][j] = (int)__builtin_amdgcn_raw_buffer_load_b32(xr, off, 0, 0);
        }
      }
    }
  };

  Acc acc[CB][PB];
#pragma unroll
  for (int cb = 0; cb < CB; cb++)
#pragma unroll
    for (int b = 0; b < PB; b++) acc[cb][b] = Acc{};

  // Independent accumulators are interleaved so consecutive MFMAs never wait
  // on each other's result.  uint8 codes are flipped here, at their use: a
  // flip next to the prefetching load would make the wave wait for it there.
  auto mma = [&](const Frag(&aa)[CB], const Frag(&bb_in)[PB]) {
    Frag bb[PB];
#pragma unroll
    for (int b = 0; b < PB; b++) {
      if constexpr (V::U8)
        bb[b] = bb_in[b] ^ kU8Flip;
      else
        bb[b] = bb_in[b];
    }
    if constexpr (!V::I8) {
#pragma unroll
      for (int j = 0; j < 4; j++)
#pragma unroll
        for (int cb = 0; cb < CB; cb++)
#pragma unroll
          for (int b = 0; b < PB; b++)
            acc[cb][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(aa[cb][j], bb[b][j], acc[cb][b], 0, 0, 0);
    } else {
#pragma unroll
      for (int cb = 0; cb < CB; cb++)
#pragma unroll
        for (int b = 0; b < PB; b++)
          acc[cb][b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(aa[cb], bb[b], acc[cb][b], 0, 0, 0);
    }
  };

  // Main loop: a ring of PF register sets keeps the loads of the next PF K
  // steps of this wave in flight while the MFMAs of the current step run
  // (small layers are latency-bound otherwise).  Loads past the wave's last
  // step are clamped onto it, so every round issues the same loads.  The
  // rounds in which all PF slots hold real steps run their MFMAs with no
  // condition, and the last, partial round is peeled off: a branch around
  // each slot's MFMAs stops the compiler from interleaving them with the next
  // step's loads and address arithmetic, which a lone wave on a SIMD needs to
  // keep the matrix unit busy (8-12% on the batch-1 3x3 layers).
  {
    const int s0 = s_begin + wk;
    if (s0 < s_end) {
      const int s_last = s0 + ((s_end - 1 - s0) / WK) * WK;
      Frag a[PF][CB], b[PF][PB];
#pragma unroll
      for (int i = 0; i < PF; i++) load(min(s0 + i * WK, s_last), a[i], b[i]);
      int s = s0;
      for (; s + (PF - 1) * WK < s_end; s += PF * WK) {
#pragma unroll
        for (int i = 0; i < PF; i++) {
          mma(a[i], b[i]);
          load(min(s + (i + PF) * WK, s_last), a[i], b[i]);
        }
      }
#pragma unroll
      for (int i = 0; i < PF; i++)
        if (s + i * WK < s_end) mma(a[i], b[i]);
    }
  }

  // The WK waves of a workgroup hold partial sums of the same output blocks.
  // After the exchange below, block (cb, b) is finished -- reduced, split-K
  // combined and stored -- by wave (cb * PB + b) % WK, so the reduction and the
  // epilogue are spread over all WK waves instead of serialised on one.
  auto mine = [&](int cb, int b) { return WK == 1 || (cb * PB + b) % WK == wk; };

  // Reduce the WK K-slices through LDS, in slice order (the same order for
  // every block, so the result does not depend on which wave sums it).
  if constexpr (WK > 1) {
    __shared__ Acc red[WK * WCO * WPX * CB * PB][64];
#pragma unroll
    for (int cb = 0; cb < CB; cb++)
#pragma unroll
      for (int b = 0; b < PB; b++)
        red[((wk * WCO * WPX + slot) * CB + cb) * PB + b][lane] = acc[cb][b];
    __syncthreads();
#pragma unroll
    for (int cb = 0; cb < CB; cb++)
#pragma unroll
      for (int b = 0; b < PB; b++) {
        if (!mine(cb, b)) continue;
        Acc sum = red[(slot * CB + cb) * PB + b][lane];
        for (int w = 1; w < WK; w++) sum += red[((w * WCO * WPX + slot) * CB + cb) * PB + b][lane];
        acc[cb][b] = sum;
      }
  }

  // Cross-workgroup split-K: publish the partial tile, take a ticket; the
  // last workgroup of the tile sums every partial in split order.  No fence is
  // needed: the partials are written through the L2 to memory (as the outputs
  // are) and the stores have completed before the ticket is taken, and the
  // last workgroup reads them with loads that bypass the caches.  An
  // agent-scope fence instead writes back and invalidates the whole L2, which
  // made every split-K launch 15-20 us slower.
  if (p.splitk > 1) {
    __shared__ int s_last;
    constexpr int TILE_VECS = WCO * WPX * CB * PB * 64;
    const __amdgpu_buffer_rsrc_t wsr =
        rsrc((const char *)p.ws + (size_t)tile * p.splitk * TILE_VECS * 16, (unsigned)(p.splitk * TILE_VECS * 16));
#pragma unroll
    for (int cb = 0; cb < CB; cb++)
#pragma unroll
      for (int b = 0; b < PB; b++)
        if (mine(cb, b))
          __builtin_amdgcn_raw_buffer_store_b128(
              __builtin_bit_cast(u32x4, acc[cb][b]), wsr,
              (unsigned)((split * TILE_VECS + ((slot * CB + cb) * PB + b) * 64 + lane) * 16), 0, kPartialStore);
    partials_published();
    __syncthreads();
    if (threadIdx.x == 0) {
      const unsigned prev =
          __hip_atomic_fetch_add(gmem<unsigned>(p.counters) + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = (prev == (unsigned)(p.splitk - 1));
    }
    __syncthreads();
    if (!s_last) return;
    partials_acquired();
#pragma unroll
    for (int cb = 0; cb < CB; cb++)
#pragma unroll
      for (int b = 0; b < PB; b++) {
        if (!mine(cb, b)) continue;
        Acc sum = Acc{};
        for (int sp = 0; sp < p.splitk; sp++) {
          const Acc v = (sp == split) ? acc[cb][b]
                                      : __builtin_bit_cast(Acc, __builtin_amdgcn_raw_buffer_load_b128(
                                                                    wsr,
                                                                    (unsigned)((sp * TILE_VECS +
                                                                                ((slot * CB + cb) * PB + b) * 64 + lane) *
                                                                               16),
                                                                    0, kPartialLoad));
          sum += v;
        }
        acc[cb][b] = sum;
      }
    if (threadIdx.x == 0)
      __hip_atomic_store(gmem<unsigned>(p.counters) + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // uint8 input: the block's sum over all K is complete here (and held by the
  // wave that finishes it), so the zero-point correction is added once.
  if constexpr (V::U8) {
#pragma unroll
    for (int cb = 0; cb < CB; cb++)
#pragma unroll
      for (int b = 0; b < PB; b++) acc[cb][b] += ep_corr[cb][b];
  }

  // Epilogue: bias (+ dequant), activation, residual, output conversion in
  // registers; masked NHWC stores of 4 channels per lane.
  const __amdgpu_buffer_rsrc_t rr = rsrc(p.res, p.res_bytes);
#pragma unroll
  for (int cb = 0; cb < CB; cb++) {
    const int co0 = (cob0 + cb) * 16 + 4 * g;
    if (co0 >= p.cout_pad) continue;
    if constexpr (V::RAW) {
#pragma unroll
      for (int b = 0; b < PB; b++)
        if (mine(cb, b) && mval[b]) store16(p, (unsigned)(outpix[b] * p.out_cs + co0) * 4u, acc[cb][b]);
    } else {
      const f32x4 bias = ep_bias[cb];
      const f32x4 dq = ep_dq[cb];
#pragma unroll
      for (int b = 0; b < PB; b++) {
        if (!mine(cb, b) || !mval[b]) continue;
        f32x4 z;
#pragma unroll
        for (int i = 0; i < 4; i++) {
          if constexpr (V::I8)
            z[i] = (float)acc[cb][b][i] * dq[i] + bias[i];
          else
            z[i] = acc[cb][b][i] + bias[i];
        }
        epilogue_store<V::X>(p, rr, z, outpix[b], ((px_tile * WPX + wpx) * PB + b) * 16 + r, co0);
      }
    }
  }
}

template <int VAR, int CB, int PB, int WCO, int WPX, int WK, int PF>
__global__ __launch_bounds__(64 * WCO * WPX * WK) void conv_igemm(ConvParams p) {
  int nblocks = gridDim.x;
  pin_tiled_args<Var<VAR>::U8>(p, nblocks, true);
  igemm_workgroup<VAR, CB, PB, WCO, WPX, WK, PF>(p, nblocks, blockIdx.x, 0);
}

// The parameters of group member i, read from the kernel-argument segment
// (GroupArgs::p starts it) with scalar loads at a wave-uniform offset.
__device__ __forceinline__ ConvParams group_member(int i) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef const __attribute__((address_space(4))) ConvParams *kernarg_params;
  return ((kernarg_params)__builtin_amdgcn_kernarg_segment_ptr())[i];
#else
  (void)i;  // the host pass of the kernel sources has no kernel-argument segment
  return ConvParams{};
#endif
}

// Several independent layers of one kernel variant in one launch: the grid
// is the members' grids laid end to end (in the XCD-major logical order), and
// each workgroup runs the tile of the member its logical index falls in.  The
// member's parameters are read from the kernel-argument segment at a
// wave-uniform offset (scalar loads, a second round after ga.first).
template <int VAR, int CB, int PB, int WCO, int WPX, int WK, int PF>
__global__ __launch_bounds__(64 * WCO * WPX * WK) void conv_igemm_group(GroupArgs ga) {
  int nblocks = gridDim.x;
  const int logical = xcd_major(nblocks, blockIdx.x);
  int member = 0, first = 0;
#pragma unroll
  for (int j = 1; j < kGroupMax; j++) {
    const bool in_later = logical >= ga.first[j];  // unused slots hold INT_MAX
    member += in_later ? 1 : 0;
    first = in_later ? ga.first[j] : first;
  }
  member = __builtin_amdgcn_readfirstlane(member);
  first = __builtin_amdgcn_readfirstlane(first);
  ConvParams p = group_member(member);
  pin_tiled_args<Var<VAR>::U8>(p, nblocks, true);
  igemm_workgroup<VAR, CB, PB, WCO, WPX, WK, PF>(p, nblocks, blockIdx.x, first);
}


// ------------------------------------------------------ LDS-staged kernel --
// The workgroup stages KS K-steps of weight and activation fragments in LDS
// (same fragment order and branch-free buffer loads as above); its WM x WN
// waves split the output tile and read their operands from LDS, so each
// fetched byte feeds several waves.  Used for the larger (batch-16, 80x80 and
// up) layers, where the register-direct kernel is bound by vector-memory issue
// rather than by MFMA.
//
// Two ways to fill a stage:
//   NS == 0: loads into registers, written to the other of two LDS buffers
//            after the current stage's MFMAs (the loads of one stage ahead are
//            in flight during the MFMAs);
//   NS >= 2: direct-to-LDS buffer loads into a ring of NS buffers, NS - 1
//            stages ahead.  A fragment of one wave is 64 lanes x 16 bytes laid
//            out lane after lane, which is exactly what a 16-byte load to LDS
//            writes, so the data never passes through registers: no staging
//            registers, no LDS writes, and the loads of several stages are in
//            flight at once.  Out-of-range offsets write zeros, as the
//            register loads read them.  Only variants with one 16-byte chunk
//            per lane can do this (the 4-byte gather of the small-channel
//            int8 variants needs a lane stride of 16 bytes in LDS); the others
//            take the register path whatever NS says.

struct Pix {
  int base, iy0, ix0, out;
  int xb;  // base * x_cs: element offset of the window's top-left tap (may be negative in the padding)
  bool ok;
};

__device__ __forceinline__ Pix pixel_of(const ConvParams &p, int m) {
  Pix q;
  q.ok = m < p.M;
  const int mm = q.ok ? m : 0;
  const int t = fdiv(mm, p.div_ow);
  const int ow = mm - t * p.OW;
  const int n = fdiv(t, p.div_oh);
  const int oh = t - n * p.OH;
  q.iy0 = oh * p.stride - p.pad;
  q.ix0 = ow * p.stride - p.pad;
  q.base = (n * p.H + q.iy0) * p.W + q.ix0;
  q.xb = q.base * p.x_cs;
  q.out = (n * p.OH + oh) * p.pitch + ow;
  return q;
}

// Byte offset of the 16-byte activation fragment of one lane (one chunk per
// lane, VEC == 1): pixel q, K chunk `cg` (= 4*step + g); out of range (read as
// zeros) in the image's zero padding, past K and past the last pixel.
template <class V>
__device__ __forceinline__ unsigned gather_off(const ConvParams &p, const Pix &q, int cg) {
  const Chunk c = decode_chunk(p, cg);
  const int iy = q.iy0 + c.dy, ix = q.ix0 + c.dx;
  const bool v = c.ok && q.ok && (unsigned)iy < (unsigned)p.H && (unsigned)ix < (unsigned)p.W;
  return v ? (unsigned)(q.base * p.x_cs + (c.dy * p.W + c.dx) * p.x_cs + c.ci) * (unsigned)V::ESIZE : kOutOfRange;
}

// The activation fragment of one lane: pixel q, K chunk group `cg` (= 4*step + g).
template <class V>
__device__ __forceinline__ typename V::Frag gather(const ConvParams &p, __amdgpu_buffer_rsrc_t xr, const Pix &q,
                                                   int cg) {
  using Frag = typename V::Frag;
  if constexpr (V::VEC == 1) {
    return __builtin_bit_cast(Frag, __builtin_amdgcn_raw_buffer_load_b128(xr, gather_off<V>(p, q, cg), 0, 0));
  } else {
    Frag f;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const Chunk c = decode_chunk(p, cg * 4 + j);
      const int iy = q.iy0 + c.dy, ix = q.ix0 + c.dx;
      const bool v = c.ok && q.ok && (unsigned)iy < (unsigned)p.H && (unsigned)ix < (unsigned)p.W;
      const unsigned off = v ? (unsigned)(q.base * p.x_cs + (c.dy * p.W + c.dx) * p.x_cs + c.ci) : kOutOfRange;
      f[j] = (int)__builtin_amdgcn_raw_buffer_load_b32(xr, off, 0, 0);
    }
    return f;
  }
}

// s_waitcnt with vmcnt = n and the LDS/scalar counter at 0 (expcnt left
// alone), in the gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8.
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit field");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

// Workgroup barrier that waits only for what the caller waited for: a
// __syncthreads() would also wait for every vector-memory load of the wave,
// including the direct-to-LDS loads of the stages still in flight.  The empty
// asm statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One 16-byte direct-to-LDS buffer load per lane: lane l's 16 bytes land at
// dst + 16 l (dst wave-uniform).
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, void *dst, unsigned off) {
  typedef __attribute__((address_space(3))) void *lds_ptr;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)dst, 16, off, 0, 0, 0);
}

// SWZ (one 16-byte chunk per lane): the activation loads of a fragment go pixel by pixel --
// lane 4q + j loads chunk j ^ sw(q) of pixel q, sw(q) = (q >> 1) & 3 -- so
// four consecutive lanes read one pixel's 64 contiguous bytes (when the four
// chunks of a step lie in one tap) instead of 16 bytes of four pixels; the
// MFMA side then reads lane (r, g)'s operand from slot 4r + (g ^ sw(r)), and
// the XOR keeps each group of 8 lanes of a 16-byte LDS read on distinct banks.
// Workgroup `bid` of a grid of nblocks runs logical tile
// xcd_major(nblocks, bid) - first of the layer described by p (first: the
// layer's first logical tile in a grouped launch, 0 otherwise).
template <int VAR, int MB, int NB, int WM, int WN, int KS, int NS, bool SWZ>
__device__ __forceinline__ void lds_workgroup(const ConvParams &p, const int nblocks, const int bid,
                                              const int first) {
  using V = Var<VAR>;
  using Frag = typename V::Frag;
  using Acc = typename V::Acc;
  constexpr int NT = 64 * WM * WN;
  constexpr int BMB = MB * WM, BNB = NB * WN;     // 16-pixel and 16-channel blocks per workgroup
  constexpr int SB = BMB + BNB;                   // fragment blocks per K step
  constexpr int NA = KS * BNB * 64 / NT;          // weight slots per thread per stage
  constexpr int NX = KS * BMB * 64 / NT;          // activation slots per thread per stage
  static_assert((KS * BNB * 64) % NT == 0 && (KS * BMB * 64) % NT == 0, "stage must split evenly over threads");
  constexpr bool DMA = NS >= 2 && V::VEC == 1;    // direct-to-LDS ring (see above)
  constexpr bool SW = SWZ && V::VEC == 1;
  constexpr int NBUF = DMA ? NS : 2;
  __shared__ Frag lds[NBUF][KS * SB * 64];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (see conv_igemm)
  const int wm = wave % WM, wn = wave / WM;
  const int r = lane & 15, g = lane >> 4;

  const int logical = xcd_major(nblocks, bid) - first;
  int px_tile, co_tile;
  tile_of(p, logical, px_tile, co_tile);

  // pixels of this thread's activation slots (the same for every stage)
  const int lq = lane >> 2, lj = (lane & 3) ^ ((lq >> 1) & 3);  // SW: pixel and chunk this lane loads
  Pix xpix[NX];
#pragma unroll
  for (int i = 0; i < NX; i++) {
    const int j = tid + i * NT;
    const int pxb = (j >> 6) % BMB;
    xpix[i] = pixel_of(p, (px_tile * BMB + pxb) * 16 + (SW ? lq : r));
  }
  // SW: the LDS slot that holds this lane's MFMA operand (pixel r, chunk g)
  const int bslot = SW ? 4 * r + (g ^ ((r >> 1) & 3)) : lane;
  // epilogue operands of this wave's blocks
  f32x4 ep_bias[NB], ep_dq[NB];
  {
    const __amdgpu_buffer_rsrc_t br =
        __builtin_amdgcn_make_buffer_rsrc((void *)p.bias, 0, (int)(p.co_blocks * 64), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t dr =
        __builtin_amdgcn_make_buffer_rsrc((void *)p.dq, 0, V::I8 ? (int)(p.co_blocks * 64) : 0, kRsrcWord3);
#pragma unroll
    for (int nb = 0; nb < NB; nb++) {
      const unsigned off = (unsigned)((((co_tile * BNB + wn * NB + nb) * 16) + 4 * g) * 4);
      ep_bias[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
      ep_dq[nb] = f32x4{1.f, 1.f, 1.f, 1.f};
      if constexpr (!V::RAW) ep_bias[nb] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(br, off, 0, 0));
      if constexpr (V::I8 && !V::RAW) ep_dq[nb] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(dr, off, 0, 0));
    }
  }

  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc((void *)p.wfrag, 0, (int)p.w_bytes, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc((void *)p.x, 0, (int)p.x_bytes, kRsrcWord3);
  const int nst = (p.steps + KS - 1) / KS;

  // Direct-to-LDS issue of stage st into buffer buf: every thread issues
  // exactly NA + NX loads (stages past the end load zeros), so the number of
  // loads in flight per stage is a compile-time constant.  Slot i of a
  // thread is fragment block (j >> 6) of the stage, j = tid + i * NT, which is
  // wave-uniform: the LDS destination of each load is one wave-uniform base,
  // to which the hardware adds lane * 16.
  auto dma_issue = [&](int st, int buf) {
#pragma unroll
    for (int i = 0; i < NA; i++) {
      const int jw = wave + i * (NT / 64);
      const int ks = jw / BNB, blk = jw % BNB;
      const int s = st * KS + ks;
      const unsigned off = s < p.steps
                               ? ((unsigned)((co_tile * BNB + blk) * p.steps + s) * 64u + (unsigned)lane) * 16u
                               : kOutOfRange;
      load_lds16(wr, &lds[buf][(ks * SB + blk) * 64], off);
    }
#pragma unroll
    for (int i = 0; i < NX; i++) {
      const int jw = wave + i * (NT / 64);
      const int ks = jw / BMB, pxb = jw % BMB;
      const int s = st * KS + ks;
      load_lds16(xr, &lds[buf][(ks * SB + BNB + pxb) * 64], gather_off<V>(p, xpix[i], s * 4 + (SW ? lj : g)));
    }
  };

  Frag ra[DMA ? 1 : NA], rx[DMA ? 1 : NX];
  auto gload = [&](int st) {
#pragma unroll
    for (int i = 0; i < NA; i++) {
      const int j = tid + i * NT;
      const int ks = j / (BNB * 64), blk = (j >> 6) % BNB;
      const int s = st * KS + ks;
      const unsigned off = s < p.steps
                               ? ((unsigned)((co_tile * BNB + blk) * p.steps + s) * 64u + (unsigned)lane) * 16u
                               : kOutOfRange;
      ra[i] = __builtin_bit_cast(Frag, __builtin_amdgcn_raw_buffer_load_b128(wr, off, 0, 0));
    }
#pragma unroll
    for (int i = 0; i < NX; i++) {
      const int j = tid + i * NT;
      const int ks = j / (BMB * 64);
      const int s = st * KS + ks;
      rx[i] = gather<V>(p, xr, xpix[i], s * 4 + (SW ? lj : g));
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NA; i++) {
      const int j = tid + i * NT;
      const int ks = j / (BNB * 64), blk = (j >> 6) % BNB;
      lds[buf][(ks * SB + blk) * 64 + lane] = ra[i];
    }
#pragma unroll
    for (int i = 0; i < NX; i++) {
      const int j = tid + i * NT;
      const int ks = j / (BMB * 64), pxb = (j >> 6) % BMB;
      // uint8 codes are flipped here, when the stage is written to LDS, not
      // next to the loads, which are still in flight during the MFMAs
      if constexpr (V::U8)
        lds[buf][(ks * SB + BNB + pxb) * 64 + lane] = rx[i] ^ kU8Flip;
      else
        lds[buf][(ks * SB + BNB + pxb) * 64 + lane] = rx[i];
    }
  };

  Acc acc[NB][MB];
#pragma unroll
  for (int nb = 0; nb < NB; nb++)
#pragma unroll
    for (int mb = 0; mb < MB; mb++) acc[nb][mb] = Acc{};
  // uint8 input: zero-point corrections, fetched now and added after the loop
  Acc ep_corr[NB][MB];
#pragma unroll
  for (int mb = 0; mb < MB; mb++) {
    int cls = 0;
    if constexpr (V::U8) {
      const Pix q = pixel_of(p, (px_tile * BMB + wm * MB + mb) * 16 + r);
      cls = border_class(p, q.iy0, q.ix0);
    }
#pragma unroll
    for (int nb = 0; nb < NB; nb++) ep_corr[nb][mb] = zp_correction<V>(p, cls, (co_tile * BNB + wn * NB + nb) * 16 + 4 * g);
  }

  auto compute = [&](int buf) {
#pragma unroll
    for (int ks = 0; ks < KS; ks++) {
      Frag a[NB], b[MB];
#pragma unroll
      for (int nb = 0; nb < NB; nb++) a[nb] = lds[buf][(ks * SB + wn * NB + nb) * 64 + lane];
#pragma unroll
      for (int mb = 0; mb < MB; mb++) {
        b[mb] = lds[buf][(ks * SB + BNB + wm * MB + mb) * 64 + bslot];
        // uint8 codes reach the direct-to-LDS ring unflipped (zeros where the
        // loads were out of range, which become -128 like every padding code)
        if constexpr (DMA && V::U8) b[mb] ^= kU8Flip;
      }
      if constexpr (!V::I8) {
#pragma unroll
        for (int jj = 0; jj < 4; jj++)
#pragma unroll
          for (int nb = 0; nb < NB; nb++)
#pragma unroll
            for (int mb = 0; mb < MB; mb++)
              acc[nb][mb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[nb][jj], b[mb][jj], acc[nb][mb], 0, 0, 0);
      } else {
#pragma unroll
        for (int nb = 0; nb < NB; nb++)
#pragma unroll
          for (int mb = 0; mb < MB; mb++)
            acc[nb][mb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[nb], b[mb], acc[nb][mb], 0, 0, 0);
      }
    }
  };

  if constexpr (DMA) {
    // Ring of NS buffers: stages st + 1 .. st + NS - 2 stay in flight while
    // stage st is waited for.  Per iteration: wait until at most (NS - 2)
    // stages of this thread's loads are outstanding (loads complete in
    // order, so stage st has landed) and until this wave's LDS reads are done,
    // then a barrier (every wave's part of stage st has landed, and every wave
    // has finished reading the buffer the next issue overwrites, which held
    // stage st - 1), then issue stage st + NS - 1, then the MFMAs of stage st.
    constexpr int L = NA + NX;
#pragma unroll
    for (int i = 0; i < NS - 1; i++) dma_issue(i, i);
    int st = 0, buf = 0;
    for (; st + NS - 1 < nst; st++) {
      wait_vm_lgkm0<(NS - 2) * L>();
      lds_barrier();
      dma_issue(st + NS - 1, buf == 0 ? NS - 1 : buf - 1);
      compute(buf);
      buf = buf == NS - 1 ? 0 : buf + 1;
    }
    // the last NS - 1 stages (or all, for short K): nothing more is issued
    wait_vm_lgkm0<0>();
    lds_barrier();
    for (; st < nst; st++) {
      compute(buf);
      buf = buf == NS - 1 ? 0 : buf + 1;
    }
  } else {
    gload(0);
    sstore(0);
    __syncthreads();
    // Every stage but the last fetches the next one while its MFMAs run, with
    // no condition around the loads (a branch would keep the compiler from
    // overlapping them, as in conv_igemm); the last stage is peeled off.
    int st = 0;
    for (; st + 1 < nst; st++) {
      gload(st + 1);
      compute(st & 1);
      sstore((st + 1) & 1);
      __syncthreads();
    }
    compute(st & 1);
  }

  if constexpr (V::U8) {
#pragma unroll
    for (int nb = 0; nb < NB; nb++)
#pragma unroll
      for (int mb = 0; mb < MB; mb++) acc[nb][mb] += ep_corr[nb][mb];
  }
  const __amdgpu_buffer_rsrc_t rr = rsrc(p.res, p.res_bytes);
#pragma unroll
  for (int nb = 0; nb < NB; nb++) {
    const int co0 = (co_tile * BNB + wn * NB + nb) * 16 + 4 * g;
    if (co0 >= p.cout_pad) continue;
#pragma unroll
    for (int mb = 0; mb < MB; mb++) {
      const int m = (px_tile * BMB + wm * MB + mb) * 16 + r;
      const Pix q = pixel_of(p, m);
      if (!q.ok) continue;
      if constexpr (V::RAW) {
        store16(p, (unsigned)(q.out * p.out_cs + co0) * 4u, acc[nb][mb]);
      } else {
        f32x4 z;
#pragma unroll
        for (int i = 0; i < 4; i++) {
          if constexpr (V::I8)
            z[i] = (float)acc[nb][mb][i] * ep_dq[nb][i] + ep_bias[nb][i];
          else
            z[i] = acc[nb][mb][i] + ep_bias[nb][i];
        }
        epilogue_store<V::X>(p, rr, z, q.out, m, co0);
      }
    }
  }
}


template <int VAR, int MB, int NB, int WM, int WN, int KS, int NS, bool SWZ = false>
__global__ __launch_bounds__(64 * WM * WN) void conv_lds(ConvParams p) {
  int nblocks = gridDim.x;
  pin_tiled_args<Var<VAR>::U8>(p, nblocks, false);
  lds_workgroup<VAR, MB, NB, WM, WN, KS, NS, SWZ>(p, nblocks, blockIdx.x, 0);
}

// Several independent layers in one launch on LDS-staged tiles (see
// conv_igemm_group; these tiles have no split-K).
template <int VAR, int MB, int NB, int WM, int WN, int KS, int NS, bool SWZ = false>
__global__ __launch_bounds__(64 * WM * WN) void conv_lds_group(GroupArgs ga) {
  int nblocks = gridDim.x;
  const int logical = xcd_major(nblocks, blockIdx.x);
  int member = 0, first = 0;
#pragma unroll
  for (int j = 1; j < kGroupMax; j++) {
    const bool in_later = logical >= ga.first[j];  // unused slots hold INT_MAX
    member += in_later ? 1 : 0;
    first = in_later ? ga.first[j] : first;
  }
  member = __builtin_amdgcn_readfirstlane(member);
  first = __builtin_amdgcn_readfirstlane(first);
  ConvParams p = group_member(member);
  pin_tiled_args<Var<VAR>::U8>(p, nblocks, false);
  lds_workgroup<VAR, MB, NB, WM, WN, KS, NS, SWZ>(p, nblocks, blockIdx.x, first);
}

// ------------------------------------------------------ halo-tile kernel --
// For 3x3 layers with few channels (the 3-channel stem and the 8..32-channel
// layers at 80..320 pixels) the implicit-GEMM gather re-reads every input
// pixel up to nine times.  Here a workgroup owns a TH x TW block of output
// pixels of one image and all (<= 64) output channels: it copies the input
// window it needs (the halo, all channels) and the layer's fragment-ordered
// weights straight into LDS with direct-to-LDS buffer loads (out-of-range
// offsets supply the zero padding), then runs every tap of the convolution
// from LDS on MFMA.  This is the direct-convolution path for the stem.
//
// PAIR: column pairs.  With at most 8 output channels, a 16-row MFMA block
// would be half padding.  Instead row 8*h + co of the block is output channel
// co of the pixel 2*j + h of the pair j, and the pair's K row runs over its
// 3 x 4 input window (tap = 4*dy + dx, dx = 0..3), with the weight of tap
// (dy, dx) in row 8*h + co equal to W'[co, ., dy, dx - h] (zero where dx - h
// falls outside 0..2).  The host lays out those weights (and a 16-row bias
// with each channel's value twice); here a "pixel" of the tile is a pair: the
// tile is TH x TW pairs, pair (ly, lx) starts at halo column 2*lx, and each
// lane stores its 4 channels to pixel 2*j + (g >> 1), channels 4*(g & 1)..+3.
template <int VAR, int TH, int TW, int NBMAX, bool EXACT, bool PAIR = false>
__global__ __launch_bounds__(256) void conv_halo(ConvParams p) {
  using V = Var<VAR>;
  using Frag = typename V::Frag;
  using Acc = typename V::Acc;
  // NBMAX (1, 2 or 4) bounds the 16-channel output blocks at compile time, so
  // accumulators and epilogue operands take registers only for blocks that can
  // exist: a 16-channel layer keeps a quarter of the 64-channel footprint and
  // runs at a higher occupancy.  EXACT: the layer has exactly NBMAX blocks, so
  // the block loops need no run-time bound (a branch in the tap loop would keep
  // the compiler from overlapping the LDS reads with the MFMAs).
  constexpr int MB = TH * TW / 64;  // 16-pixel blocks per wave (4 waves)
  static_assert(TH * TW % 64 == 0, "tile must split into 4 waves of 16-pixel blocks");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  int nblocks = gridDim.x;
  pin_halo_args<V::U8>(p, nblocks);
  typedef __attribute__((address_space(3))) void *lds_ptr;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (see conv_igemm)
  const int r = lane & 15, g = lane >> 4;

  const int nb_ = nblocks, bid = blockIdx.x;
  const int per = nb_ >> 3, rem = nb_ & 7, xcd = bid & 7, loc = bid >> 3;
  const int logical = xcd * per + min(xcd, rem) + loc;  // branch-free form of the XCD-major order
  const int rest = fdiv(logical, p.div_tx);
  const int tx = logical - rest * p.tiles_x;
  const int n = fdiv(rest, p.div_ty);
  const int ty = rest - n * p.tiles_y;

  static_assert(!PAIR || (NBMAX == 1 && EXACT), "column pairs: one 16-row block");
  const int st_ = PAIR ? 1 : p.stride;
  const int HWd = PAIR ? 2 * TW + 2 : (TW - 1) * st_ + 3;  // halo width in pixels
  const int HH = (TH - 1) * st_ + 3;                        // halo height
  const int oh0 = ty * TH, ow0 = tx * (PAIR ? 2 * TW : TW);
  const int iy0 = oh0 * st_ - p.pad, ix0 = ow0 * st_ - p.pad;
  const int cq = p.cin_pad >> 2;                 // 4-channel slots per pixel
  const int cql = p.halo_cq;                     // slots per pixel in LDS (cq, or cq + 1: see below)
  constexpr int SLOT = 4 * V::ESIZE;             // bytes of a 4-channel slot
  const int halo_slots = HH * HWd * cql;

  // 1) input halo and weights -> LDS (all loads in flight, no register round trip)
  {
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc((void *)p.x, 0, (int)p.x_bytes, kRsrcWord3);
    for (int base = wave * 64; base < halo_slots; base += 256) {
      const int sl = base + lane;
      const int px = fdiv(sl, p.div_hcq);
      const int q = sl - px * cql;  // q == cq: the padding slot, loaded as zeros
      const int hy = fdiv(px, p.div_hwd);
      const int hx = px - hy * HWd;
      const int iy = iy0 + hy, ix = ix0 + hx;
      const bool v = sl < halo_slots && q < cq && (unsigned)iy < (unsigned)p.H && (unsigned)ix < (unsigned)p.W;
      const unsigned off = v ? (unsigned)(((n * p.H + iy) * p.W + ix) * p.x_cs + 4 * q) * (unsigned)V::ESIZE
                             : kOutOfRange;
      if constexpr (SLOT == 16)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_ptr)(smem + base * SLOT), 16, off, 0, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_ptr)(smem + base * SLOT), 4, off, 0, 0, 0);
    }
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc((void *)p.wfrag, 0, (int)p.w_bytes, kRsrcWord3);
    const int wslots = (int)(p.w_bytes >> 4);
    for (int base = wave * 64; base < wslots; base += 256)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_ptr)(smem + p.halo_bytes + base * 16), 16,
                                               (unsigned)(base + lane) * 16u, 0, 0, 0);
  }
  // epilogue operands meanwhile
  const int nbl = EXACT ? NBMAX : p.co_blocks;  // <= NBMAX, uniform
  f32x4 ep_bias[NBMAX], ep_dq[NBMAX];
  {
    const __amdgpu_buffer_rsrc_t br =
        __builtin_amdgcn_make_buffer_rsrc((void *)p.bias, 0, (int)(p.co_blocks * 64), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t dr =
        __builtin_amdgcn_make_buffer_rsrc((void *)p.dq, 0, V::I8 ? (int)(p.co_blocks * 64) : 0, kRsrcWord3);
#pragma unroll
    for (int nb = 0; nb < NBMAX; nb++) {
      const unsigned off = (unsigned)((nb * 16 + 4 * g) * 4);
      ep_bias[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
      ep_dq[nb] = f32x4{1.f, 1.f, 1.f, 1.f};
      if constexpr (!V::RAW) ep_bias[nb] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(br, off, 0, 0));
      if constexpr (V::I8 && !V::RAW) ep_dq[nb] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(dr, off, 0, 0));
    }
  }
  Acc acc[NBMAX][MB];
#pragma unroll
  for (int mb = 0; mb < MB; mb++) {
    int cls = 0;
    if constexpr (V::U8) {
      // the correction of a row is that of its own pixel's 3x3 window (with
      // column pairs, pixel 2j + (g >> 1); the fourth window column has zero
      // weight in that row)
      const int pi = (wave * MB + mb) * 16 + r;
      const int ox = PAIR ? ow0 + 2 * (pi % TW) + (g >> 1) : ow0 + pi % TW;
      cls = border_class(p, (oh0 + pi / TW) * st_ - p.pad, ox * st_ - p.pad);
    }
#pragma unroll
    for (int nb = 0; nb < NBMAX; nb++)
      acc[nb][mb] = nb < nbl ? zp_correction<V>(p, cls, PAIR ? 4 * (g & 1) : nb * 16 + 4 * g) : Acc{};
  }

  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // 2) every tap from LDS: lane (r, g) of block mb holds pixel r of that block
  // An fp32 pixel of an even number of 16-byte slots would put the 16
  // pixels of a fragment read on repeating LDS banks; the host pads it to an
  // odd number of slots (a zero slot), which makes those reads conflict-free.
  const int pix_bytes = cql * SLOT;
  unsigned lb[MB];  // byte offset in the halo of pixel r of each of this wave's blocks
#pragma unroll
  for (int mb = 0; mb < MB; mb++) {
    const int pi = (wave * MB + mb) * 16 + r;
    const int ly = pi / TW, lx = pi % TW;
    lb[mb] = (unsigned)((PAIR ? ly * HWd + 2 * lx : (ly * st_) * HWd + lx * st_) * pix_bytes);
  }
  const unsigned char *wl = smem + p.halo_bytes + lane * 16;  // this lane's slot of each weight fragment
  // One K step.  Only the last step can hold chunks past K (every chunk of the
  // steps before it is below total_chunks), so only it masks: elsewhere the
  // operands go to the MFMAs as read.
  auto step = [&](int s, auto last) {
    constexpr bool MASK = decltype(last)::value;
    Frag a[NBMAX];
#pragma unroll
    for (int nb = 0; nb < NBMAX; nb++)
      a[nb] = nb < nbl ? *(const Frag *)(wl + (nb * p.steps + s) * 1024) : Frag{};
    Frag b[MB];
    if constexpr (V::VEC == 1) {
      Chunk c = PAIR ? decode_chunk_pair(p, s * 4 + g) : decode_chunk(p, s * 4 + g);
      if (MASK && !c.ok) c.dy = c.dx = c.ci = 0;  // past K: read a valid slot, then zero it
      const unsigned woff = (unsigned)((c.dy * HWd + c.dx) * pix_bytes + c.ci * V::ESIZE);
#pragma unroll
      for (int mb = 0; mb < MB; mb++) {
        // 16-byte aligned (pixels are whole 16-byte slots and a chunk starts a
        // slot): said explicitly, so the read is one ds_read_b128, whose lanes
        // the slot padding spreads over distinct banks, and not two 8-byte
        // reads, which it does not
        Frag v = *(const Frag *)__builtin_assume_aligned(smem + (lb[mb] + woff), 16);
        if constexpr (V::U8) v ^= kU8Flip;  // zero-filled padding becomes -128, as in conv_igemm
        b[mb] = (!MASK || c.ok) ? v : Frag{};
      }
    } else {
#pragma unroll
      for (int mb = 0; mb < MB; mb++) b[mb] = Frag{};
#pragma unroll
      for (int j = 0; j < 4; j++) {
        Chunk c = PAIR ? decode_chunk_pair(p, (s * 4 + g) * 4 + j) : decode_chunk(p, (s * 4 + g) * 4 + j);
        if (MASK && !c.ok) c.dy = c.dx = c.ci = 0;
        const unsigned woff = (unsigned)((c.dy * HWd + c.dx) * pix_bytes + c.ci);
#pragma unroll
        for (int mb = 0; mb < MB; mb++) {
          int v = *(const int *)(smem + (lb[mb] + woff));
          if constexpr (V::U8) v ^= kU8Flip;
          b[mb][j] = (!MASK || c.ok) ? v : 0;
        }
      }
    }
#pragma unroll
    for (int nb = 0; nb < NBMAX; nb++) {
      if (nb >= nbl) break;
      if constexpr (!V::I8) {
#pragma unroll
        for (int jj = 0; jj < 4; jj++)
#pragma unroll
          for (int mb = 0; mb < MB; mb++)
            acc[nb][mb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[nb][jj], b[mb][jj], acc[nb][mb], 0, 0, 0);
      } else {
#pragma unroll
        for (int mb = 0; mb < MB; mb++)
          acc[nb][mb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[nb], b[mb], acc[nb][mb], 0, 0, 0);
      }
    }
  };
  // two steps per iteration, so that the next step's LDS reads can be issued
  // under the current step's MFMAs
  int s = 0;
  for (; s + 1 < p.steps - 1; s += 2) {
    step(s, BoolC<false>{});
    step(s + 1, BoolC<false>{});
  }
  if (s < p.steps - 1) step(s, BoolC<false>{});
  step(p.steps - 1, BoolC<true>{});

  // 3) epilogue, masked to the image and to the real channels
  const __amdgpu_buffer_rsrc_t rr = rsrc(p.res, p.res_bytes);
#pragma unroll
  for (int nb = 0; nb < NBMAX; nb++) {
    if (nb >= nbl) break;
    const int co0 = PAIR ? 4 * (g & 1) : nb * 16 + 4 * g;
    if (co0 >= p.cout_pad) continue;
#pragma unroll
    for (int mb = 0; mb < MB; mb++) {
      const int pi = (wave * MB + mb) * 16 + r;
      const int oh = oh0 + pi / TW, ow = PAIR ? ow0 + 2 * (pi % TW) + (g >> 1) : ow0 + pi % TW;
      if (oh >= p.OH || ow >= p.OW) continue;
      const int opix = (n * p.OH + oh) * p.pitch + ow;
      if constexpr (V::RAW) {
        store16(p, (unsigned)(opix * p.out_cs + co0) * 4u, acc[nb][mb]);
      } else {
        f32x4 z;
#pragma unroll
        for (int i = 0; i < 4; i++) {
          if constexpr (V::I8)
            z[i] = (float)acc[nb][mb][i] * ep_dq[nb][i] + ep_bias[nb][i];
          else
            z[i] = acc[nb][mb][i] + ep_bias[nb][i];
        }
        epilogue_store<V::X>(p, rr, z, opix, (n * p.OH + oh) * p.OW + ow, co0);
      }
    }
  }
}

// ------------------------------------------------ weight-stationary 1x1 --
// 1x1 stride-1 layers at large M (the batch-16 1x1 convolutions with 16-384
// input channels).  There the output is thousands of 16-pixel blocks
// deep but only a few channel blocks wide, K is short (1-24 K steps), and a
// tile of the other kernels pays its prologue (weights, first activations)
// and its epilogue once per 64-128 pixels.  Here a workgroup of WCO x WPX
// waves owns WCO*CBW channel blocks and a contiguous run of pixel blocks (the
// WPX waves on the same channel blocks take every WPX-th block of it); each wave
// loads the weights of its CBW channel blocks for all KS steps into registers
// once, then streams the run's pixel blocks through them.  The activations of
// the next block are loaded (into a second register set) while the current
// block's MFMAs and epilogue run.  Runs differ by at
// most one block, so the work is spread evenly over the grid, which the host
// sizes to a few workgroups per CU.  The input pixel of an output pixel is its
// logical index (1x1, stride 1, no padding).
//
// GATHER: the same for small-weight 3x3 layers with 16 or 32 (padded) input
// channels, 9 or 18 K steps: K step s then lies in tap 9s/KS, so the tap of
// every step is known at compile time and a block needs one offset per tap
// (the pixel's window corner plus the tap's fixed displacement, or out of
// range where the tap falls in the padding), computed where the 1x1 form
// computes its single offset; the 16-channel steps of one tap read at
// immediate offsets from it.  The block's output pixel index comes with its
// offsets, and the pixel arithmetic uses 24-bit multiplies (full rate, where
// 32-bit ones take four issue cycles), which the host allows only for
// tensors whose pixel and element indices fit (below 2^23).  WPX waves of a
// workgroup share the channel blocks and take every WPX-th block of the run.
//
// PARTIAL (1x1): C_in is not a multiple of 16, so the last K step holds fewer
// than four chunks; that step has its own offset, out of range for the lanes
// whose chunk lies past C_in.
//
// int8 and uint8 activations (1x1): a K step is 64 channels and one 16x16x64
// MFMA; the dequantising epilogue, the raw int32 accumulators and the uint8
// zero-point start value (the interior border class: a 1x1 window without
// padding never leaves the image) follow the other kernels.  A lane's 16 bytes
// of a step are 16 consecutive channels of one pixel with 16- and with
// 4-channel chunks alike (a 1x1 layer's weights are laid out the same way for
// both); with 4-channel chunks (a C_in that is not a multiple of 16) the pixel
// is only 4-byte aligned, so a lane reads them as four 4-byte loads, the last
// step's masked one by one past C_in.
//
// IN2 (fp32 1x1): the input channels are a concatenation of two tensors, the
// first c1 (a multiple of 16, so every K step lies in one of them) from x and
// the rest from x2: K step s reads x below step c1/16 and x2 from there, at a
// per-lane offset of its own (out of range, in the last step, for lanes past
// the second tensor's channels).
template <int VAR, int CBW, int WCO, int KS, int WPX = 1, bool GATHER = false, bool PARTIAL = false,
          bool IN2 = false>
__global__ __launch_bounds__(64 * WCO * WPX) void conv_ws(ConvParams p) {
  using V = Var<VAR>;
  static_assert(!V::I8 || !GATHER, "int8: 1x1 only");
  static_assert(!IN2 || (!V::I8 && !GATHER && !PARTIAL), "second input: fp32 1x1");
  constexpr int CH = V::I8 ? 16 : 4;  // channels of one lane's chunk
  using Frag = typename V::Frag;
  using Acc = typename V::Acc;
  int nblocks = gridDim.x;
  pin_tiled_args<V::U8>(p, nblocks, false);
  pin_sgpr(p.run_base);
  pin_sgpr(p.run_rem);
  if constexpr (IN2) {
    pin_sgpr(p.x2);
    pin_sgpr(p.x2_cs);
    pin_sgpr(p.x2_bytes);
    pin_sgpr(p.c1);
  }
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: MFMA guards are scalar
  const int wpx = wave % WPX, wco = wave / WPX;
  const int r = lane & 15, g = lane >> 4;
  int run, co_tile;
  tile_of(p, xcd_major(nblocks, blockIdx.x), run, co_tile);
  const int b0 = run * p.run_base + min(run, p.run_rem) + wpx;  // this wave's first block
  const int b1 = run * p.run_base + min(run, p.run_rem) + p.run_base + (run < p.run_rem ? 1 : 0);
  const int cob0 = (co_tile * WCO + wco) * CBW;

  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc((void *)p.wfrag, 0, (int)p.w_bytes, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc((void *)p.x, 0, (int)p.x_bytes, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t xr2 =
      __builtin_amdgcn_make_buffer_rsrc((void *)p.x2, 0, IN2 ? (int)p.x2_bytes : 0, kRsrcWord3);
  const int s1 = IN2 ? p.c1 >> 4 : KS;  // IN2: the first K step of the second input
  // Offsets of pixel block b (zero-filled past the run or past M).  1x1: lane
  // (g, r) reads channels 16s + 4g .. +3 of pixel 16b + r for K step s.
  // GATHER: channels 16j + 4g .. +3 of tap t of pixel 16b + r's window for
  // K step s = t * KS/9 + j.
  static_assert(!GATHER || KS == 9 || KS == 18, "gathered K depths: 9 or 18 steps");
  static_assert(!(GATHER && PARTIAL), "partial K steps: 1x1 only");
  constexpr int NOFF = GATHER ? 9 : IN2 ? 3 : PARTIAL ? 2 : 1;
  constexpr int SPT = GATHER ? KS / 9 : KS;  // K steps per offset
  unsigned tap_off[NOFF];
  if constexpr (GATHER) {
#pragma unroll
    for (int t = 0; t < 9; t++) tap_off[t] = (unsigned)(((t / 3) * p.W + t % 3) * p.x_cs) * 4u;
  }
  auto block_offs = [&](int b, unsigned(&o)[NOFF], int &opix) {
    const int m = b * 16 + r;
    if constexpr (GATHER) {
      const bool ok = b < b1 && m < p.M;
      const int mm = ok ? m : 0;
      const int t = fdiv(mm, p.div_ow);  // n * OH + oh
      const int ow = mm - __mul24(t, p.OW);
      const int n = fdiv(t, p.div_oh);
      const int oh = t - __mul24(n, p.OH);
      const int iy0 = __mul24(oh, p.stride) - p.pad, ix0 = __mul24(ow, p.stride) - p.pad;
      const int xb = __mul24(__mul24(__mul24(n, p.H) + iy0, p.W) + ix0, p.x_cs);  // window corner, elements
      opix = __mul24(t, p.pitch) + ow;
      const unsigned lb = (unsigned)(xb + 4 * g) * 4u;  // wraps for corners in the padding
      bool rv[3], cv[3];
#pragma unroll
      for (int d = 0; d < 3; d++) {
        rv[d] = ok && (unsigned)(iy0 + d) < (unsigned)p.H;
        cv[d] = (unsigned)(ix0 + d) < (unsigned)p.W;
      }
#pragma unroll
      for (int tp = 0; tp < 9; tp++) o[tp] = (rv[tp / 3] && cv[tp % 3]) ? lb + tap_off[tp] : kOutOfRange;
    } else {
      (void)opix;
      o[0] = (b < b1 && m < p.M) ? (unsigned)(m * p.x_cs + CH * g) * (unsigned)V::ESIZE : kOutOfRange;
      if constexpr (PARTIAL) o[NOFF - 1] = 4 * (KS - 1) + g < p.total_chunks ? o[0] : kOutOfRange;
      if constexpr (IN2) {
        // second input: its own pixel stride; the last K step masks the lanes past its channels
        o[1] = (b < b1 && m < p.M) ? (unsigned)(m * p.x2_cs + 4 * g) * 4u : kOutOfRange;
        o[2] = 4 * (KS - 1) + g < p.total_chunks ? o[1] : kOutOfRange;
      }
    }
  };
  // 4-channel chunks: bit j says chunk 4 (4 (KS-1) + g) + j of the last K step lies inside C_in
  unsigned last_mask = 0;
  if constexpr (V::I8 && V::VEC == 4) {
#pragma unroll
    for (int j = 0; j < 4; j++) last_mask |= (unsigned)(4 * (4 * (KS - 1) + g) + j < p.total_chunks) << j;
  }
  auto load_block = [&](const unsigned(&o)[NOFF], Frag(&dst)[KS]) {
    if constexpr (V::I8 && V::VEC == 4) {
      // chunk 4 (4s + g) + j of K step s is dword j of the lane's 16 bytes
#pragma unroll
      for (int s = 0; s < KS; s++)
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const unsigned oj = (s == KS - 1 && !((last_mask >> j) & 1u)) ? kOutOfRange : o[0];
          dst[s][j] = (int)__builtin_amdgcn_raw_buffer_load_b32(xr, oj, s * 64 + 4 * j, 0);
        }
      return;
    }
#pragma unroll
    for (int s = 0; s < KS; s++) {
      if constexpr (IN2) {
        // steps below s1 read the first input, the rest the second (s1 is uniform)
        if (s < s1)
          dst[s] = __builtin_bit_cast(Frag, __builtin_amdgcn_raw_buffer_load_b128(xr, o[0], s * 64, 0));
        else
          dst[s] = __builtin_bit_cast(
              Frag, __builtin_amdgcn_raw_buffer_load_b128(xr2, o[s == KS - 1 ? 2 : 1], (s - s1) * 64, 0));
        continue;
      }
      const unsigned os = GATHER ? o[s / SPT] : o[s == KS - 1 ? NOFF - 1 : 0];
      dst[s] = __builtin_bit_cast(Frag, __builtin_amdgcn_raw_buffer_load_b128(xr, os, (s % SPT) * 64, 0));
    }
  };
  Frag ba[KS], bb[KS];  // activations of the current and of the next pixel block
  int op_cur = 0, op_nxt = 0;  // GATHER: output pixels of the current and the next block
  {
    unsigned o0[NOFF];
    block_offs(b0, o0, op_cur);
    load_block(o0, ba);
  }
  // this wave's weights (zero for channel blocks past the end), bias, int8
  // dequant factors and uint8 start values
  Frag a[CBW][KS];
  f32x4 bias[CBW], dq[CBW];
  Acc acc0[CBW];
  {
    const __amdgpu_buffer_rsrc_t br =
        __builtin_amdgcn_make_buffer_rsrc((void *)p.bias, 0, (int)(p.co_blocks * 64), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t dr =
        __builtin_amdgcn_make_buffer_rsrc((void *)p.dq, 0, V::I8 ? (int)(p.co_blocks * 64) : 0, kRsrcWord3);
#pragma unroll
    for (int cb = 0; cb < CBW; cb++) {
      const unsigned wv = (cob0 + cb) < p.co_blocks
                              ? ((unsigned)((cob0 + cb) * p.steps) * 64u + (unsigned)lane) * 16u
                              : kOutOfRange;
#pragma unroll
      for (int s = 0; s < KS; s++)
        a[cb][s] = __builtin_bit_cast(Frag, __builtin_amdgcn_raw_buffer_load_b128(wr, wv, s * 1024, 0));
      bias[cb] = __builtin_bit_cast(
          f32x4, __builtin_amdgcn_raw_buffer_load_b128(br, (unsigned)(((cob0 + cb) * 16 + 4 * g) * 4), 0, 0));
      dq[cb] = f32x4{1.f, 1.f, 1.f, 1.f};
      if constexpr (V::I8 && !V::RAW)
        dq[cb] = __builtin_bit_cast(
            f32x4, __builtin_amdgcn_raw_buffer_load_b128(dr, (unsigned)(((cob0 + cb) * 16 + 4 * g) * 4), 0, 0));
      acc0[cb] = zp_correction<V>(p, V::U8 ? border_class(p, 0, 0) : 0, (cob0 + cb) * 16 + 4 * g);
    }
  }
  const __amdgpu_buffer_rsrc_t rr = rsrc(p.res, p.res_bytes);
  // One pixel block, in three phases kept apart by scheduling barriers:
  //  1. every load of block b + WPX into `nxt`, at offsets computed before
  //     the previous block's stores (below);
  //  2. the MFMAs on `cur` (the compiler would otherwise sink the loads below
  //     them and leave the next block's latency exposed);
  //  3. the offsets of block b + 2 WPX, then the epilogue and its stores.
  // A VALU write to a register that a store still reads waits until the store
  // has completed, so nothing but loads and MFMAs follows the stores until the
  // next block's epilogue, a whole block of MFMAs later.
  unsigned off[NOFF];
  block_offs(b0 + WPX, off, op_nxt);
  auto block = [&](int b, const Frag(&cur)[KS], Frag(&nxt)[KS]) {
    load_block(off, nxt);
    __builtin_amdgcn_sched_barrier(0);
    Acc acc[CBW];
#pragma unroll
    for (int cb = 0; cb < CBW; cb++) acc[cb] = acc0[cb];
#pragma unroll
    for (int s = 0; s < KS; s++) {
      if constexpr (V::I8) {
        const Frag bs = V::U8 ? (cur[s] ^ kU8Flip) : cur[s];
#pragma unroll
        for (int cb = 0; cb < CBW; cb++) acc[cb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[cb][s], bs, acc[cb], 0, 0, 0);
      } else {
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
          for (int cb = 0; cb < CBW; cb++)
            acc[cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[cb][s][j], cur[s][j], acc[cb], 0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    int op_next2 = 0;
    block_offs(b + 2 * WPX, off, op_next2);
    // epilogue: 4 channels of pixel 16b + r per lane and channel block
    const int m = b * 16 + r;
    if (m < p.M) {
      int opix = op_cur;
      if constexpr (!GATHER) {
        const int t = fdiv(m, p.div_ow);
        const int ow = m - t * p.OW;
        const int n = fdiv(t, p.div_oh);
        const int oh = t - n * p.OH;
        opix = (n * p.OH + oh) * p.pitch + ow;
      }
#pragma unroll
      for (int cb = 0; cb < CBW; cb++) {
        const int co0 = (cob0 + cb) * 16 + 4 * g;
        if (co0 >= p.cout_pad) continue;
        if constexpr (V::RAW) {
          store16(p, (unsigned)(opix * p.out_cs + co0) * 4u, acc[cb]);
        } else {
          f32x4 z;
#pragma unroll
          for (int i = 0; i < 4; i++) {
            if constexpr (V::I8)
              z[i] = (float)acc[cb][i] * dq[cb][i] + bias[cb][i];
            else
              z[i] = acc[cb][i] + bias[cb][i];
          }
          epilogue_store<V::X>(p, rr, z, opix, m, co0);
        }
      }
    }
    op_cur = op_nxt;
    op_nxt = op_next2;
    __builtin_amdgcn_sched_barrier(0);
  };
  // The prologue's loads are waited for here, so that the loop is entered with
  // nothing in flight.
  __builtin_amdgcn_s_waitcnt(0);
  for (int b = b0; b < b1; b += 2 * WPX) {
    block(b, ba, bb);
    if (b + WPX < b1) block(b + WPX, bb, ba);
  }
}

// ---------------------------------------------------------------- launch --
template <int VAR, int CB, int PB, int WCO, int WPX, int WK, int PF>
static hipError_t launch_one(const ConvParams &p, hipStream_t stream) {
  const unsigned grid = (unsigned)p.px_tiles * (unsigned)p.co_tiles * (unsigned)p.splitk;
  hipLaunchKernelGGL((conv_igemm<VAR, CB, PB, WCO, WPX, WK, PF>), dim3(grid), dim3(64 * WCO * WPX * WK), 0,
                     stream, p);
  return hipGetLastError();
}

template <int VAR, int MB, int NB, int WM, int WN, int KS, int NS = 0, bool SWZ = false>
static hipError_t launch_lds(const ConvParams &p, hipStream_t stream) {
  if (p.splitk != 1) return hipErrorInvalidValue;
  const unsigned grid = (unsigned)p.px_tiles * (unsigned)p.co_tiles;
  hipLaunchKernelGGL((conv_lds<VAR, MB, NB, WM, WN, KS, NS, SWZ>), dim3(grid), dim3(64 * WM * WN), 0, stream, p);
  return hipGetLastError();
}

template <int VAR, int TH, int TW>
static hipError_t launch_halo(const ConvParams &p, hipStream_t stream) {
  if (p.splitk != 1 || p.co_blocks < 1 || p.co_blocks > 4 || p.k != 3) return hipErrorInvalidValue;
  const unsigned grid = (unsigned)p.px_tiles;
  const unsigned smem = (unsigned)p.smem_bytes;
  if (p.co_blocks == 1)
    hipLaunchKernelGGL((conv_halo<VAR, TH, TW, 1, true>), dim3(grid), dim3(256), smem, stream, p);
  else if (p.co_blocks == 2)
    hipLaunchKernelGGL((conv_halo<VAR, TH, TW, 2, true>), dim3(grid), dim3(256), smem, stream, p);
  else if (p.co_blocks == 4)
    hipLaunchKernelGGL((conv_halo<VAR, TH, TW, 4, true>), dim3(grid), dim3(256), smem, stream, p);
  else
    hipLaunchKernelGGL((conv_halo<VAR, TH, TW, 4, false>), dim3(grid), dim3(256), smem, stream, p);
  return hipGetLastError();
}

// Column-pair halo tiles: one 16-row block (8 channels x 2 pixels).
template <int VAR, int TH, int TW>
static hipError_t launch_halo_pair(const ConvParams &p, hipStream_t stream) {
  if (p.splitk != 1 || p.co_blocks != 1 || p.k != 3 || p.stride != 1 || p.cout_pad > 8) return hipErrorInvalidValue;
  hipLaunchKernelGGL((conv_halo<VAR, TH, TW, 1, true, true>), dim3((unsigned)p.px_tiles), dim3(256),
                     (unsigned)p.smem_bytes, stream, p);
  return hipGetLastError();
}

// Weight-stationary tiles: the K depth is a template argument (the weights of
// all K steps sit in registers), instantiated for the depths the configuration
// lists allow.
template <int VAR, int CBW, int WCO, int KS, int WPX = 1, bool GATHER = false, bool PARTIAL = false,
          bool IN2 = false>
static hipError_t launch_ws_k(const ConvParams &p, hipStream_t stream) {
  hipLaunchKernelGGL((conv_ws<VAR, CBW, WCO, KS, WPX, GATHER, PARTIAL, IN2>), dim3((unsigned)p.px_tiles * (unsigned)p.co_tiles),
                     dim3(64 * WCO * WPX), 0, stream, p);
  return hipGetLastError();
}
// Weight-stationary tiles with the window gather (configurations G.*): the K
// depths of 3x3 layers with 16 or 32 input channels.
template <int VAR, int CBW, int WPX>
static hipError_t launch_wsg(const ConvParams &p, hipStream_t stream) {
  if constexpr (VAR != VAR_F32 && VAR != VAR_F32_X) {
    (void)p, (void)stream;
    return hipErrorInvalidValue;
  } else {
    if (p.splitk != 1 || p.k != 3 || p.chunk_ch != 4 || (p.chunks_per_tap & 3) != 0) return hipErrorInvalidValue;
    switch (p.steps) {
      case 9: return launch_ws_k<VAR, CBW, 1, 9, WPX, true>(p, stream);
      case 18: return launch_ws_k<VAR, CBW, 1, 18, WPX, true>(p, stream);
      default: return hipErrorInvalidValue;
    }
  }
}
template <int VAR, int CBW, int WCO, int WPX>
static hipError_t launch_ws(const ConvParams &p, hipStream_t stream) {
  using V = Var<VAR>;
  if constexpr (V::I8) {
    // K steps of 64 channels: depths 1-4 and 6, a partial last step at 1-3
    // (4-channel chunks: a C_in that is not a multiple of 16, always partial)
    if (p.splitk != 1 || p.k != 1 || p.stride != 1 || p.pad != 0 || p.chunk_ch != (V::VEC == 1 ? 16 : 4))
      return hipErrorInvalidValue;
    if (p.total_chunks < (V::VEC == 1 ? 4 : 16) * p.steps) {
      switch (p.steps) {
        case 1: return launch_ws_k<VAR, CBW, WCO, 1, WPX, false, true>(p, stream);
        case 2: return launch_ws_k<VAR, CBW, WCO, 2, WPX, false, true>(p, stream);
        case 3: return launch_ws_k<VAR, CBW, WCO, 3, WPX, false, true>(p, stream);
        default: return hipErrorInvalidValue;
      }
    }
    switch (p.steps) {
      case 1: return launch_ws_k<VAR, CBW, WCO, 1, WPX>(p, stream);
      case 2: return launch_ws_k<VAR, CBW, WCO, 2, WPX>(p, stream);
      case 3: return launch_ws_k<VAR, CBW, WCO, 3, WPX>(p, stream);
      case 4: return launch_ws_k<VAR, CBW, WCO, 4, WPX>(p, stream);
      case 6: return launch_ws_k<VAR, CBW, WCO, 6, WPX>(p, stream);
      default: return hipErrorInvalidValue;
    }
  } else {
    if (p.splitk != 1 || p.k != 1 || p.stride != 1 || p.pad != 0 || p.chunk_ch != 4) return hipErrorInvalidValue;
    constexpr int kMax = ws_max_steps(CBW);  // deepest K that fits the registers without spilling
    if (p.x2) {  // a second input: the concatenation depths of a C3k2 block's last 1x1 (1.5 to 24 steps)
      if (p.c1 <= 0 || (p.c1 & 15) || 16 * p.steps <= p.c1) return hipErrorInvalidValue;
      switch (p.steps) {
        case 2: return launch_ws_k<VAR, CBW, WCO, 2, WPX, false, false, true>(p, stream);
        case 3: return launch_ws_k<VAR, CBW, WCO, 3, WPX, false, false, true>(p, stream);
        case 6: return launch_ws_k<VAR, CBW, WCO, 6, WPX, false, false, true>(p, stream);
        case 12:
          if constexpr (kMax >= 12) return launch_ws_k<VAR, CBW, WCO, 12, WPX, false, false, true>(p, stream);
          return hipErrorInvalidValue;
        case 24:
          if constexpr (kMax >= 24) return launch_ws_k<VAR, CBW, WCO, 24, WPX, false, false, true>(p, stream);
          return hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
      }
    }
    if (p.total_chunks < 4 * p.steps) {  // a partial last K step: depths 1-3 only
      switch (p.steps) {
        case 1: return launch_ws_k<VAR, CBW, WCO, 1, WPX, false, true>(p, stream);
        case 2: return launch_ws_k<VAR, CBW, WCO, 2, WPX, false, true>(p, stream);
        case 3: return launch_ws_k<VAR, CBW, WCO, 3, WPX, false, true>(p, stream);
        default: return hipErrorInvalidValue;
      }
    }
    switch (p.steps) {
      case 1: return launch_ws_k<VAR, CBW, WCO, 1, WPX>(p, stream);
      case 2: return launch_ws_k<VAR, CBW, WCO, 2, WPX>(p, stream);
      case 3: return launch_ws_k<VAR, CBW, WCO, 3, WPX>(p, stream);
      case 4: return launch_ws_k<VAR, CBW, WCO, 4, WPX>(p, stream);
      case 6: return launch_ws_k<VAR, CBW, WCO, 6, WPX>(p, stream);
      case 8: return launch_ws_k<VAR, CBW, WCO, 8, WPX>(p, stream);
      case 12:
        if constexpr (kMax >= 12) return launch_ws_k<VAR, CBW, WCO, 12, WPX>(p, stream);
        return hipErrorInvalidValue;
      case 16:
        if constexpr (kMax >= 16) return launch_ws_k<VAR, CBW, WCO, 16, WPX>(p, stream);
        return hipErrorInvalidValue;
      case 24:
        if constexpr (kMax >= 24) return launch_ws_k<VAR, CBW, WCO, 24, WPX>(p, stream);
        return hipErrorInvalidValue;
      default: return hipErrorInvalidValue;
    }
  }
}

template <int VAR, int MB, int NB, int WM, int WN, int KS, int NS = 0, bool SWZ = false>
static hipError_t launch_group_lds(const GroupArgs &g, unsigned grid, hipStream_t stream) {
  hipLaunchKernelGGL((conv_lds_group<VAR, MB, NB, WM, WN, KS, NS, SWZ>), dim3(grid), dim3(64 * WM * WN), 0, stream, g);
  return hipGetLastError();
}

template <int VAR, int CB, int PB, int WCO, int WPX, int WK, int PF>
static hipError_t launch_group_one(const GroupArgs &g, unsigned grid, hipStream_t stream) {
  hipLaunchKernelGGL((conv_igemm_group<VAR, CB, PB, WCO, WPX, WK, PF>), dim3(grid), dim3(64 * WCO * WPX * WK), 0,
                     stream, g);
  return hipGetLastError();
}

// Grouped launch of variant VAR with register-direct or LDS-staged configuration `cfg`.
template <int VAR>
static hipError_t launch_group_variant(int cfg, const GroupArgs &g, unsigned grid, hipStream_t stream) {
  switch (cfg) {
#define X(id, cb, pb, wco, wpx, wk, pf, name) \
  case id:                                    \
    return launch_group_one<VAR, cb, pb, wco, wpx, wk, pf>(g, grid, stream);
    CBS_CONFIG_LIST(X)
    CBS_CONFIG_LIST_EXT(X)
#undef X
#define X(id, mb, nb, wm, wn, ks, name) \
  case id:                              \
    return launch_group_lds<VAR, mb, nb, wm, wn, ks>(g, grid, stream);
    CBS_LDS_CONFIG_LIST(X)
    CBS_LDS_CONFIG_LIST_EXT(X)
#undef X
#define X(id, mb, nb, wm, wn, ks, ns, name) \
  case id:                                  \
    return launch_group_lds<VAR, mb, nb, wm, wn, ks, ns>(g, grid, stream);
    CBS_LDS_RING_CONFIG_LIST(X)
#undef X
#define X(id, mb, nb, wm, wn, ks, ns, name) \
  case id:                                  \
    return launch_group_lds<VAR, mb, nb, wm, wn, ks, ns, true>(g, grid, stream);
    CBS_LDS_RING_SWZ_CONFIG_LIST(X)
#undef X
    default:
      return hipErrorInvalidValue;
  }
}

// Launch configuration `cfg` of variant VAR.
template <int VAR>
static hipError_t launch_variant(int cfg, const ConvParams &p, hipStream_t stream) {
  switch (cfg) {
#define X(id, cb, pb, wco, wpx, wk, pf, name) \
  case id:                                    \
    return launch_one<VAR, cb, pb, wco, wpx, wk, pf>(p, stream);
    CBS_CONFIG_LIST(X)
#undef X
#define X(id, mb, nb, wm, wn, ks, name) \
  case id:                              \
    return launch_lds<VAR, mb, nb, wm, wn, ks>(p, stream);
    CBS_LDS_CONFIG_LIST(X)
#undef X
#define X(id, th, tw, name) \
  case id:                  \
    return launch_halo<VAR, th, tw>(p, stream);
    CBS_HALO_CONFIG_LIST(X)
#undef X
#define X(id, cb, pb, wco, wpx, wk, pf, name) \
  case id:                                    \
    return launch_one<VAR, cb, pb, wco, wpx, wk, pf>(p, stream);
    CBS_CONFIG_LIST_EXT(X)
#undef X
#define X(id, mb, nb, wm, wn, ks, name) \
  case id:                              \
    return launch_lds<VAR, mb, nb, wm, wn, ks>(p, stream);
    CBS_LDS_CONFIG_LIST_EXT(X)
#undef X
#define X(id, mb, nb, wm, wn, ks, ns, name) \
  case id:                                  \
    return launch_lds<VAR, mb, nb, wm, wn, ks, ns>(p, stream);
    CBS_LDS_RING_CONFIG_LIST(X)
#undef X
#define X(id, th, tw, name) \
  case id:                  \
    return launch_halo_pair<VAR, th, tw>(p, stream);
    CBS_HALO_PAIR_CONFIG_LIST(X)
#undef X
#define X(id, mb, nb, wm, wn, ks, ns, name) \
  case id:                                  \
    return launch_lds<VAR, mb, nb, wm, wn, ks, ns, true>(p, stream);
    CBS_LDS_RING_SWZ_CONFIG_LIST(X)
#undef X
#define X(id, cbw, wco, wpx, occ, name) \
  case id:                              \
    return launch_ws<VAR, cbw, wco, wpx>(p, stream);
    CBS_WS_CONFIG_LIST(X) CBS_WS_CONFIG_LIST_EXT(X)
#undef X
#define X(id, cbw, wpx, occ, name) \
  case id:                         \
    return launch_wsg<VAR, cbw, wpx>(p, stream);
    CBS_WSG_CONFIG_LIST(X)
#undef X
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace cbs
