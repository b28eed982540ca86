/*
 * cbs.h -- C ABI of libcbs, fused Conv2d + folded BatchNorm + SiLU ("cbs") for
 * AMD Instinct MI355X (gfx950), in FP32 and INT8.
 *
 * The operation (cited from the pages it comes from):
 *   - "YOLO26N Inference Optimisation" (vision-rs docs), section "nsys
 *     kernel-level breakdown" and "Key observations" 1-3: one fused
 *     convolution + batch norm + SiLU op is where the inference time goes;
 *     section "Baseline benchmark": batch norm is folded into the weights at
 *     load; section "Improvements" #1 and #3: one code path with a tile chosen
 *     per layer shape; section "NHWC migration": NHWC activations, weights as
 *     [C_out][kH][kW][C_in], the convolution as an implicit GEMM
 *     A[N*OH*OW, C_in*kH*kW] x B[C_in*kH*kW, C_out]; section "Bug fixed: TMA
 *     overflow": tail tiles must never write past the logical output row.
 *   - "Edge optimisation of YOLO26" (edge-optimization README), "Highlights"
 *     and "Design notes": INT8 with one symmetric weight scale per output
 *     channel and one percentile-calibrated activation scale per tensor.
 *
 * Per output element (n, oh, ow, co), with x~ the zero-padded input:
 *   conv = sum_{ci,i,j} W'[co,ci,i,j] * x~[n, oh*s - p + i, ow*s - p + j, ci]
 *   y    = SiLU(conv + b'[co]),  SiLU(z) = z / (1 + exp(-z))
 * where, folded at create time in double precision,
 *   sc[co] = gamma[co] / sqrt(var[co] + eps),  W' = W * sc,  b' = beta - mean * sc.
 * INT8 (dtype CBS_I8):
 *   s_w[co] = max|W'[co,:]| / 127 (1 for an all-zero channel),
 *   q_w = clamp(rne(W' / s_w), -127, 127)                        (double)
 *   q_x = clamp(rne(fp32(x / s_x)), -127, 127)                   (fp32 divide)
 *   acc = sum q_w * q_x                                          (exact int32)
 *   y   = SiLU(float(acc) * f[co] + b'[co]),  f[co] = fp32(s_x * s_w[co])
 *
 * Fused epilogue and I/O options (descriptor fields after bn_eps), from the
 * same vision-rs page, section "Improvements" #6 (a conv reads a channel_cat
 * result as slices of its producers, so no cat kernel runs) and #7 (bias and
 * residual adds happen in the conv epilogue, while the results are still in
 * registers), and section "NHWC migration -- Op-by-op impact across the
 * graph" (bias add, cat and chunk disappear into the conv); and from the
 * edge-optimization README ("Highlights": the network runs in INT8 end to end):
 *   act = CBS_ACT_NONE:  y = conv + b'          (the page's plain conv2d_forward
 *                                                 + nchw_bias_add, via create_layer_folded)
 *   residual:            y = act(...) + r        (r fp32; for int8 output r = res_scale * q_r)
 *   out_dtype = CBS_I8:  q_y = clamp(rne(fp32(y / s_y)), -127, 127), the quantiser of the
 *                        next INT8 layer's input (s_y = its s_x), applied to the fp32 y.
 *
 * Asymmetric activations (edge-optimization README, "Design notes": ONNX
 * Runtime quantises activations asymmetrically to uint8, with symmetric
 * per-channel weights, since activations after SiLU are mostly positive):
 *   dtype = CBS_U8:      q_x = clamp(rne(fp32(x / s_x)) + z_x, 0, 255), z_x = in_zero_point;
 *                        acc = sum over the taps inside the image of q_w * (q_x - z_x)
 *                        (exact int32: zero padding is a real zero, the code z_x), then
 *                        the INT8 epilogue above.  Weights are quantised as for CBS_I8.
 *   out_dtype = CBS_U8:  q_y = clamp(rne(fp32(y / s_y)) + z_y, 0, 255), z_y = out_zero_point.
 *   residual of a CBS_U8 output: r = res_scale * (q_r - res_zero_point).
 *
 * Layouts (all device buffers are caller-owned):
 *   input  : NHWC [N][H][W][in_c_stride]; fp32 for CBS_F32, int8 for CBS_I8,
 *            uint8 for CBS_U8; the layer reads channels in_c_offset ..
 *            in_c_offset + C_in_pad - 1.  Dense (in_c_stride = 0): the stride is
 *            C_in_pad = round_up(C_in, 4) and padded lanes must hold 0 (any code
 *            for CBS_U8, whose padded lanes meet zero weights).  Slice (in_c_stride > 0): C_in,
 *            in_c_offset and in_c_stride are multiples of 4 and
 *            in_c_offset + C_in <= in_c_stride (a channel_chunk / channel_cat
 *            slice read in place).
 *   output : NHWC [N][OH][out_row_pitch][out_c_stride], fp32 or int8
 *            (out_dtype); the layer writes channels out_c_offset ..
 *            out_c_offset + C_out_pad - 1 of pixels ow < OW and nothing else:
 *            the out_row_pitch - OW guard pixels after every row and all other
 *            channels are never touched.  Dense: stride C_out_pad, padded
 *            channels get 0.  Slice: C_out, out_c_offset and out_c_stride are
 *            multiples of 4 and out_c_offset + C_out <= out_c_stride (writing
 *            into a channel_cat buffer in place).
 *   second input (in2_channels > 0; fp32 1x1 stride-1 layers): the layer's
 *            input channels are the concatenation of the first input's C_in -
 *            in2_channels channels (a positive multiple of 16; in_c_stride and
 *            in_c_offset describe that input as usual, dense stride C_in -
 *            in2_channels) and the second input's in2_channels channels, NHWC
 *            [N][H][W][in2_c_stride] from channel 0 (in2_channels and
 *            in2_c_stride multiples of 4).  The producers of a concatenation can
 *            then write dense rows instead of slices of a wider pixel, and the
 *            consumer reads both tensors (run with cbs_run_layer_in2 or steps
 *            that name the second input).
 *   residual (res_c_stride > 0): NHWC [N][OH][OW][res_c_stride] (dense rows,
 *            like an input), of the output's dtype; the layer reads channels
 *            res_c_offset .. res_c_offset + C_out - 1.  C_out, res_c_offset and
 *            res_c_stride are multiples of 4, res_c_offset + C_out <= res_c_stride.
 *            It may share a buffer with the output when their channel ranges
 *            are disjoint.
 *   weights: host OIHW fp32 [C_out][C_in][k][k], copied at create.
 *
 * Execution: every cbs_run_* call only enqueues kernels on the given stream
 * (a hipStream_t passed as void*, NULL = the null stream): no allocation, no
 * memset, no copy, no synchronisation.  A layer may be run from one stream at
 * a time (its split-K workspace is per layer); distinct layers may run
 * concurrently.  Device faults surface at the caller's next synchronisation.
 *
 * Errors: every entry point returns a cbs_status; nothing throws or aborts.
 * cbs_last_error() gives a message for the calling thread's last failure.
 */
#ifndef CBS_H_
#define CBS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t cbs_status;
#define CBS_OK 0
#define CBS_EINVAL (-1)       /* bad argument (null pointer, negative size, ...) */
#define CBS_EUNSUPPORTED (-2) /* valid but not supported (k not in {1,3}, stride not in {1,2}, ...) */
#define CBS_ENOMEM (-3)       /* device or host allocation failed at create */
#define CBS_EDEVICE (-4)      /* no usable HIP device, or a HIP runtime call failed */
#define CBS_ELAUNCH (-5)      /* a kernel launch was rejected */

#define CBS_F32 0
#define CBS_I8 1
#define CBS_U8 2 /* asymmetric uint8 codes with a zero point */

#define CBS_ACT_SILU 0 /* y = SiLU(z) (the default) */
#define CBS_ACT_NONE 1 /* y = z: plain convolution + bias */

typedef struct cbs_layer cbs_layer; /* opaque: one fused conv layer on one device */
typedef struct cbs_graph cbs_graph; /* opaque: a captured layer list */
typedef struct cbs_group cbs_group; /* opaque: independent layers run by one launch */

typedef struct cbs_conv_desc {
    int32_t n;             /* batch, >= 1 */
    int32_t c_in;          /* input channels, >= 1 */
    int32_t h, w;          /* input height and width, >= 1 */
    int32_t c_out;         /* output channels, >= 1 */
    int32_t k;             /* kernel size: 1 or 3 */
    int32_t stride;        /* 1 or 2 */
    int32_t pad;           /* zero padding, 0 <= pad <= k/2 */
    int32_t dtype;         /* CBS_F32, CBS_I8 or CBS_U8 */
    int32_t out_row_pitch; /* output pixels between consecutive (n, oh) rows, >= OW; 0 means OW */
    float in_scale;        /* CBS_I8 / CBS_U8: per-tensor activation scale s_x > 0; ignored for CBS_F32 */
    float bn_eps;          /* batch-norm epsilon >= 0, used as (double)bn_eps */
    /* ---- fused epilogue and I/O (all-zero = the plain layer described above) ---- */
    int32_t act;           /* CBS_ACT_SILU (0) or CBS_ACT_NONE */
    int32_t out_dtype;     /* CBS_F32 (0): fp32 output; CBS_I8 / CBS_U8: codes of scale out_scale */
    float out_scale;       /* out_dtype CBS_I8 / CBS_U8: per-tensor output scale s_y > 0 */
    int32_t in_c_stride;   /* channels between consecutive input pixels; 0 = C_in_pad (dense) */
    int32_t in_c_offset;   /* first input channel of this layer within a pixel (0 when dense) */
    int32_t out_c_stride;  /* channels between consecutive output pixels; 0 = C_out_pad (dense) */
    int32_t out_c_offset;  /* first output channel written within a pixel (0 when dense) */
    int32_t res_c_stride;  /* residual: channels between its pixels; 0 = no residual */
    int32_t res_c_offset;  /* residual: first channel within its pixel */
    float res_scale;       /* out_dtype CBS_I8 / CBS_U8 with a residual: scale of its codes, > 0 */
    /* ---- zero points of uint8 tensors, in [0, 255]; must be 0 for other dtypes ---- */
    int32_t in_zero_point;  /* dtype CBS_U8: z_x */
    int32_t out_zero_point; /* out_dtype CBS_U8: z_y */
    int32_t res_zero_point; /* out_dtype CBS_U8 with a residual: zero point of its codes */
    /* ---- second input (a channel concatenation kept as two dense tensors); 0 = none ---- */
    int32_t in2_channels;  /* the last in2_channels of the C_in channels come from the second input */
    int32_t in2_c_stride;  /* channels between its pixels; 0 = round_up(in2_channels, 4) (dense) */
} cbs_conv_desc;

typedef struct cbs_layer_info_t {
    int32_t c_in_pad, c_out_pad;  /* padded channel counts of input and output */
    int32_t oh, ow;               /* output height and width */
    int32_t out_row_pitch;        /* pixels per output row (>= ow) */
    int32_t dtype;                /* CBS_F32, CBS_I8 or CBS_U8 */
    int64_t in_bytes;             /* size of the input buffer run_layer reads (N*H*W*in_c_stride*b_in) */
    int64_t out_bytes;            /* size of the output buffer run_layer writes into
                                     (N*OH*pitch*out_c_stride*b_out; guards included) */
    int64_t flops;                /* 2*N*OH*OW*C_out*C_in*k*k (logical channels) */
    int64_t alg_bytes;            /* N*H*W*C_in*b_in + C_out*C_in*k*k*b_w + N*OH*OW*C_out*b_out
                                     (+ the same again for a residual) + 8*C_out */
    int32_t config;               /* kernel configuration index in use */
    int32_t splitk;               /* workgroups that share one output tile along K */
    int32_t grid;                 /* workgroups per launch */
    int32_t threads;              /* threads per workgroup */
    char config_name[48];         /* human-readable configuration name */
    int64_t res_bytes;            /* size of the residual buffer read (0 without residual) */
    int64_t in2_bytes;            /* size of the second input buffer read (0 without one) */
} cbs_layer_info_t;

/*
 * Create a layer: validate the descriptor, fold batch norm (double), re-lay
 * the weights into MFMA fragment order, quantise them for CBS_I8, pick the
 * kernel configuration for this shape from the tile table, and copy
 * everything to the current HIP device (for CBS_U8 also the zero-point
 * correction of the accumulators: 64 * round_up(C_out, 16) int32).  Host arrays: w_oihw has
 * C_out*C_in*k*k floats; gamma, beta, mean, var have C_out floats each; all
 * are copied and may be freed afterwards.  On success *out owns device memory
 * until cbs_destroy_layer.  Errors: CBS_EINVAL, CBS_EUNSUPPORTED, CBS_ENOMEM,
 * CBS_EDEVICE (no device).  *out is set to NULL on failure.
 */
cbs_status cbs_create_layer(const cbs_conv_desc *desc, const float *w_oihw, const float *gamma,
                            const float *beta, const float *mean, const float *var,
                            cbs_layer **out);

/*
 * Same as cbs_create_layer with batch norm already folded into a per-channel
 * scale and bias: W' = W * scale[co] (double), b' = bias[co].  scale = 1,
 * bias = b gives a plain convolution + bias + SiLU.
 */
cbs_status cbs_create_layer_folded(const cbs_conv_desc *desc, const float *w_oihw,
                                   const float *scale, const float *bias, cbs_layer **out);

/* Release a layer's device and host memory.  NULL is a no-op.  The caller
 * must make sure no enqueued run of the layer is still pending. */
void cbs_destroy_layer(cbs_layer *layer);

/*
 * Enqueue the fused layer on `stream`: in (device, layout above) -> out
 * (device, layout above).  in and out must not overlap.  Errors: CBS_EINVAL
 * (null layer or buffer, or a layer created with a residual or a second
 * input), CBS_ELAUNCH.
 */
cbs_status cbs_run_layer(const cbs_layer *layer, const void *in, void *out, void *stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops where hipMalloc is not allowed): cbs_run_layer with
 * the cross-workgroup split-K factor chosen per call (splitk >= 1, or 0 for
 * the layer's own), whose partial tiles and arrival tickets live in a fixed
 * array of the library on each device ("scratch": CBS_NOALLOC_PARTIAL_BYTES
 * of partial tiles and CBS_NOALLOC_TICKETS tickets, held by every device the
 * library runs on until the process ends) instead of a workspace of the layer.
 * No call allocates or frees anything (the first call on a device looks up
 * the array's address).  Same layouts, arguments and results as
 * cbs_run_layer; a split needs the layer's configuration to be register-direct.
 * It enqueues a small kernel that clears the tickets it uses, then the
 * layer's kernel.  Every call on one device shares that device's array:
 * calls whose runs overlap on one device (other streams, other threads) race
 * and give wrong results; calls in one stream are ordered and safe.
 * Errors: CBS_EINVAL (null layer or buffer, a layer with a residual, splitk
 * outside [0, 64], a current device other than the layer's),
 * CBS_EUNSUPPORTED (the configuration cannot run that split, or the run needs
 * more partial-tile bytes or tickets than the array holds), CBS_EDEVICE,
 * CBS_ELAUNCH.
 */
#define CBS_NOALLOC_PARTIAL_BYTES (8u << 20)
#define CBS_NOALLOC_TICKETS 16384u
cbs_status cbs_run_layer_noalloc(const cbs_layer *layer, const void *in, void *out, int32_t splitk,
                                 void *stream);

/*
 * Same for a layer created with a residual (res_c_stride > 0): residual is
 * the device tensor added after the activation (layout above).  CBS_EINVAL if
 * the layer has no residual or residual is NULL.
 */
/*
 * Run a layer created with a second input (in2_channels > 0): `in` holds the
 * first C_in - in2_channels input channels and `in2` the rest, each with its
 * own pixel stride (a concatenation read from two tensors, "YOLO26N Inference
 * Optimisation", section "Improvements": the channel_cat and channel_chunk
 * operations become pointer arithmetic).  `residual` as in cbs_run_layer_res,
 * NULL when the layer has none.  Layers without a second input are rejected
 * (CBS_EINVAL), and so are layers with one in every other run entry point.
 */
cbs_status cbs_run_layer_in2(const cbs_layer *layer, const void *in, const void *in2, void *out,
                             const void *residual, void *stream);

cbs_status cbs_run_layer_res(const cbs_layer *layer, const void *in, void *out, const void *residual,
                             void *stream);

/*
 * Enqueue layers[0..n-1] in order on one stream, layer i reading ins[i] and
 * writing outs[i] (any of them may alias another layer's output to chain
 * layers).  Stops at the first failing launch and returns its status.  The
 * whole shape table of a network runs back to back with nothing between the
 * convolutions: no per-call memset or scratch allocation ("YOLO26N Inference
 * Optimisation", "Improvements" #5, persistent scratch) and no layout change
 * inside the graph ("NHWC migration", the all-or-nothing constraint).
 */
cbs_status cbs_run_layer_list(cbs_layer *const *layers, int32_t n, const void *const *ins,
                              void *const *outs, void *stream);

/*
 * Capture the same layer list, with these buffers, into a HIP graph and
 * instantiate it (the capture runs on a private stream; `stream` is unused).
 * The layers and buffers must outlive the graph.  The graph keeps the
 * addresses of each layer's split-K workspace in its kernel arguments, so
 * while it exists cbs_layer_set_config refuses a configuration that would
 * need a larger workspace (CBS_EINVAL), and cbs_layer_autotune skips such
 * configurations; a replay always runs the configurations captured.  This is
 * the vision-rs page's CUDA-graph replay of the whole forward pass ("YOLO26N
 * Inference Optimisation": the runtime line of its header, and "Baseline
 * benchmark", which credits graph capture for beating eager PyTorch).
 */
cbs_status cbs_graph_create(cbs_layer *const *layers, int32_t n, const void *const *ins,
                            void *const *outs, void *stream, cbs_graph **out);

/*
 * The same capture with independent layers merged into grouped launches
 * (see cbs_group_create) where that measures faster: the page's observation
 * that a small kernel leaves the GPU nearly idle while every launch costs a
 * few microseconds ("YOLO26N Inference Optimisation", "Key observations" 1
 * and 4), applied to layers that do not depend on each other, such as the
 * three scales of a detection head.
 *
 * group_of[i] >= 0 names layer i's candidate group, -1 leaves it alone;
 * group_of == NULL is cbs_graph_create.  A group has at most CBS_GROUP_MAX
 * layers of one kernel variant without residual (cbs_group_create's rules).
 * Its launch takes the place of its last member in the list, so no member may
 * read or overlap another member's output, and no layer between its first
 * and last member may read a member's output or write a member's input or
 * output: all of this is checked on the buffer ranges the layers read and
 * write (CBS_EINVAL otherwise).  For each candidate the library times, on
 * these buffers, its members' separate launches and the grouped launch under
 * every register-direct and LDS-staged configuration that fits (each as
 * replays of 20 back-to-back launches, best of 5), and keeps the fastest
 * grouped launch only if it beats the separate ones.  This blocks for the
 * timing, writes the outputs as runs do, and allocates the groups' split-K
 * workspaces, which the graph owns.  Errors as cbs_graph_create, plus
 * CBS_EINVAL for a bad grouping.
 */
cbs_status cbs_graph_create_grouped(cbs_layer *const *layers, int32_t n, const void *const *ins,
                                    void *const *outs, const int32_t *group_of, void *stream,
                                    cbs_graph **out);

/* Kernel launches per replay of a graph, and the number of candidate groups
 * it was created with (0 unless by cbs_graph_create_grouped).  Either pointer
 * may be NULL. */
cbs_status cbs_graph_info(const cbs_graph *graph, int32_t *launches, int32_t *groups);

typedef struct cbs_graph_group_info_t {
    int32_t group_id;  /* the caller's group id */
    int32_t members;   /* layers in the group */
    int32_t kept;      /* 1: runs as one grouped launch; 0: its members run separately */
    int32_t config;    /* configuration of the fastest grouped launch (-1: none fit) */
    float us_grouped;  /* measured microseconds of that grouped launch */
    float us_separate; /* measured microseconds of the members' separate launches, summed */
} cbs_graph_group_info_t;

/* What cbs_graph_create_grouped measured and chose for candidate group i
 * (0 <= i < the count from cbs_graph_info, in order of first member). */
cbs_status cbs_graph_group_info(const cbs_graph *graph, int32_t i, cbs_graph_group_info_t *info);
/*
 * One step of a chained block: a layer with its input, output and residual
 * (NULL unless the layer was created with one).  Consecutive steps share
 * buffers through channel slices, so a C3k2-style block (1x1 conv, chunk,
 * bottleneck 3x3 pair with shortcut, cat, 1x1 conv) runs as its convolutions
 * alone, with no cat, chunk or add kernel in between.
 */
typedef struct cbs_step {
    const cbs_layer *layer;
    const void *in;
    void *out;
    const void *residual;
    const void *in2; /* the second input (NULL unless the layer was created with one) */
} cbs_step;

/* Enqueue steps[0..n-1] in order on one stream; stops at the first failure. */
cbs_status cbs_run_steps(const cbs_step *steps, int32_t n, void *stream);

/* Capture the same steps into a HIP graph, as cbs_graph_create does for a list. */
cbs_status cbs_graph_create_steps(const cbs_step *steps, int32_t n, void *stream, cbs_graph **out);

/* Enqueue one replay of a captured list on `stream`. */
cbs_status cbs_graph_launch(const cbs_graph *graph, void *stream);
/* Release a captured list.  NULL is a no-op. */
void cbs_graph_destroy(cbs_graph *graph);

/*
 * Grouped launch.  A small layer leaves most of the GPU idle, and every launch
 * pays a fixed few-microsecond cost that serialised small kernels add up
 * (vision-rs "YOLO26N Inference Optimisation", "Key observations" 1 and 4).
 * A group runs up to CBS_GROUP_MAX independent layers -- none reads another's
 * output, as with the three scales of a detection head -- as one kernel whose
 * grid is the members' grids end to end, so the small members fill the CUs
 * the large one leaves idle.
 *
 * cbs_group_create: layers[0..n-1], 1 <= n <= CBS_GROUP_MAX, must run the same
 * kernel variant on the same device: the same dtype; for int8 and uint8 the
 * same input chunking (C_in_pad, the input channel stride and offset all
 * multiples of 16, or not); and all with, or all without, an option of the
 * general epilogue (identity activation, byte output).  No member may have a
 * residual.  config is a register-direct configuration id (one whose
 * cbs_config_name starts with "c") or an LDS-staged one ("L.", "LS.", "R.",
 * "RS."), or -1 to let a cost model choose among the register-direct ones.
 * With a register-direct configuration each member gets its own
 * cross-workgroup split-K factor (1 to 4), which evens out the K depth of the
 * members' workgroups; the group allocates its own split-K workspace here, so
 * one group runs from one stream at a time.  LDS-staged tiles have no split-K.  The group
 * keeps pointers to the layers, which must outlive it; their own
 * configurations are not changed.  Errors: CBS_EINVAL (NULL out or layers, n
 * out of range, a NULL layer), CBS_EUNSUPPORTED (mixed variants or devices, a
 * residual, a halo-tile configuration, or one that does not fit every
 * member), CBS_ENOMEM, CBS_EDEVICE.
 *
 * cbs_group_run: enqueue the group on `stream`; member i reads ins[i] and
 * writes outs[i], with the layouts of cbs_run_layer.  No output may overlap
 * another member's input or output.  It enqueues one kernel and nothing else
 * (no allocation, copy or synchronisation), so it can be captured into a HIP
 * graph with the caller's own stream capture.  Errors: CBS_EINVAL (NULL
 * group or buffers), CBS_ELAUNCH.
 */
#define CBS_GROUP_MAX 4
cbs_status cbs_group_create(cbs_layer *const *layers, int32_t n, int32_t config, cbs_group **out);
cbs_status cbs_group_run(const cbs_group *group, const void *const *ins, void *const *outs, void *stream);
/* The configuration id the group runs with (-1 for NULL). */
int32_t cbs_group_config(const cbs_group *group);
/* Release a group and its workspace (not its layers).  NULL is a no-op. */
void cbs_group_destroy(cbs_group *group);

/* Fill *info with the layer's shapes, buffer sizes, work and configuration. */
cbs_status cbs_layer_info(const cbs_layer *layer, cbs_layer_info_t *info);

/*
 * Override the kernel configuration chosen at create: config in
 * [0, cbs_num_configs()), splitk >= 1 workgroups along K (0 keeps the
 * default for that config).  Returns CBS_EUNSUPPORTED when the configuration
 * cannot run this layer (the layer is then unchanged).  Used by tests, which
 * force every configuration on every shape, and by the offline tile sweep.
 * A cross-workgroup split-K needs a workspace of partial tiles; the layer
 * keeps the largest it has allocated (it never shrinks).  While a graph holds
 * the layer (cbs_graph_create*), a configuration that needs more returns
 * CBS_EINVAL and the layer is unchanged.
 */
cbs_status cbs_layer_set_config(cbs_layer *layer, int32_t config, int32_t splitk);
int32_t cbs_num_configs(void);

/*
 * Create-time tuning: the vision-rs page's improvement #1 in its intended
 * form ("Improvements" #1: benchmark candidate tiles per unique layer shape,
 * since one fixed tile spans 5 to 556 us across call sites).  Times every
 * kernel configuration that can run this layer (split-K 1, plus 2, 3 and 4 for
 * register-direct configurations whose grid is below 256 workgroups), each as
 * a captured graph of `iters` back-to-back launches (0 = 20) replayed with HIP
 * events (the best of three replays after a warm-up one), on a private stream
 * after waiting for `stream`, on the caller's buffers, and keeps the fastest
 * (while a graph holds the layer, only configurations whose split-K workspace
 * fits the current one).  Graph replay is how a captured list runs its
 * kernels; an eager launch costs the GPU a few microseconds of its own, which
 * would hide the differences between configurations of small layers.  The choice is
 * cached in the process per device, shape, dtype, epilogue and channel
 * strides: a later call for the same key takes it without timing, unless
 * flags has CBS_TUNE_FORCE.  Blocks until the timing is done, may allocate
 * (split-K workspaces), writes `out` as a run does; not for use under graph
 * capture.  The compiled-in tile table (an offline sweep of the same kind)
 * stays the default at create; this call replaces it for one layer.
 * *config_out / *splitk_out (may be NULL) receive the choice.  Errors:
 * CBS_EINVAL (null layer or buffer, residual mismatch, a layer created with a
 * second input, bad iters or flags), CBS_ELAUNCH / CBS_EDEVICE (the layer
 * keeps its previous configuration).
 */
#define CBS_TUNE_FORCE 1
cbs_status cbs_layer_autotune(cbs_layer *layer, const void *in, void *out, const void *residual,
                              int32_t iters, int32_t flags, void *stream, int32_t *config_out,
                              int32_t *splitk_out);
/* Forget every cached tuning result (all devices). */
void cbs_autotune_clear_cache(void);
/*
 * Name of configuration i, or NULL when i is out of range.  Static storage.
 * The prefix names the kernel family and the shapes it can run:
 *   "c..."         operands straight to registers (any layer; cross-workgroup
 *                  split-K allowed);
 *   "L.", "LS."    LDS-staged tiles filled through registers, "R.", "RS."
 *                  filled by direct-to-LDS loads into a ring of stages (any
 *                  layer; "S" = pixel-major activation loads);
 *   "H."           input window and all weights in LDS (3x3 layers with at
 *                  most 64 output channels whose window and weights fit the
 *                  device's workgroup LDS);
 *   "P."           the same on column pairs (3x3 stride 1, at most 8 output
 *                  channels);
 *   "W."           weights held in registers, runs of 16-pixel blocks per
 *                  workgroup (1x1 stride 1 without padding; fp32: C_in
 *                  rounded up to a multiple of 4 spanning 1, 2, 3, 4, 6, 8,
 *                  12, 16 or 24 steps of 16 channels, 24 steps on the
 *                  16-channel "W.c16" tiles only, at most 16 on "W.c32", at
 *                  most 8 on "W.c80"; int8 and uint8: 16-channel aligned
 *                  input spanning 1, 2, 3, 4 or 6 steps of 64 channels; the
 *                  last step partial only at 1-3 steps);
 *   "G."           the same with the 3x3 window gathered per pixel (fp32 3x3,
 *                  any stride and padding, C_in rounded up to a multiple of 4
 *                  equal to 16 or 32).
 * Only "c..." tiles take a split-K above 1.
 */
const char *cbs_config_name(int32_t config);

/* Message for the calling thread's last failure ("" if none).  Thread-local storage. */
const char *cbs_last_error(void);

/*
 * Graph-entry layout change: NCHW fp32 [n][c][h][w] -> NHWC fp32
 * [n][h][w][c_pad] with lanes c..c_pad-1 set to 0.  c_pad >= c, c_pad % 4 == 0.
 */
cbs_status cbs_pack_nhwc_f32(const float *nchw, float *nhwc, int32_t n, int32_t c, int32_t h,
                             int32_t w, int32_t c_pad, void *stream);

/*
 * Graph-entry layout change with per-tensor INT8 quantisation:
 * q = clamp(rne(fp32(x / s_x)), -127, 127), NCHW fp32 -> NHWC int8
 * [n][h][w][c_pad], padded lanes 0.  s_x > 0, c_pad >= c, c_pad % 4 == 0.
 */
cbs_status cbs_quantize_nhwc_i8(const float *nchw, int8_t *nhwc, float s_x, int32_t n, int32_t c,
                                int32_t h, int32_t w, int32_t c_pad, void *stream);

/*
 * The same with asymmetric uint8 quantisation (edge-optimization README,
 * "Design notes"): q = clamp(rne(fp32(x / s_x)) + z, 0, 255), padded lanes get
 * z (a real zero).  s_x > 0, 0 <= z <= 255, c_pad >= c, c_pad % 4 == 0.
 */
cbs_status cbs_quantize_nhwc_u8(const float *nchw, uint8_t *nhwc, float s_x, int32_t z, int32_t n, int32_t c,
                                int32_t h, int32_t w, int32_t c_pad, void *stream);

/*
 * Test hook (CBS_I8 and CBS_U8 layers): run the integer part of the layer and
 * store the raw int32 accumulators (for CBS_U8 the zero-point corrected sum), NHWC [N][OH][out_row_pitch][C_out_pad], instead
 * of the fp32 epilogue.  Same guard-pixel rule as cbs_run_layer.
 */
cbs_status cbs_run_layer_raw_acc(const cbs_layer *layer, const void *in, int32_t *acc, void *stream);

/*
 * Test hook: copy the layer's host-side quantised weights (CBS_I8, CBS_U8) as
 * OIHW int8 [C_out][C_in][k][k] and the per-channel scales s_w (double
 * [C_out]).  Either pointer may be NULL.  CBS_EINVAL for a CBS_F32 layer.
 */
cbs_status cbs_get_qweights(const cbs_layer *layer, int8_t *q_oihw, double *s_w);

/*
 * Test hook: copy the folded weights W' (OIHW, as the fp32 values the kernel
 * uses for CBS_F32) and the folded bias b' (fp32 [C_out]).  Either may be NULL.
 */
cbs_status cbs_get_folded(const cbs_layer *layer, float *w_oihw, float *bias);

#ifdef __cplusplus
}
#endif

#endif /* CBS_H_ */
