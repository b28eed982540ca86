// conv_configs.h -- kernel configurations of libcbs (shared by the kernel
// translation units and the configuration table).  Each X-macro entry is one
// tile shape; its id is its index in the table and in the tile sweep.
#pragma once

// Register-direct conv_igemm: id, CB, PB (16-channel / 16-pixel blocks per
// wave), WCO, WPX, WK (waves along channels, pixels, K), PF (prefetch depth).
#define CBS_CONFIG_LIST(X)                    \
  X(0, 1, 4, 1, 4, 1, 4, "c16p256")           \
  X(1, 2, 2, 1, 4, 1, 4, "c32p128")           \
  X(2, 2, 2, 2, 2, 1, 4, "c64p64")            \
  X(3, 4, 2, 1, 4, 1, 2, "c64p128")           \
  X(4, 4, 2, 2, 2, 1, 2, "c128p64")           \
  X(5, 4, 1, 1, 1, 4, 4, "c64p16k4")          \
  X(6, 2, 1, 1, 1, 4, 4, "c32p16k4")          \
  X(7, 1, 2, 1, 2, 2, 4, "c16p64k2")          \
  X(8, 2, 2, 2, 1, 2, 4, "c64p32k2")          \
  X(9, 1, 1, 1, 1, 4, 4, "c16p16k4")          \
  X(10, 2, 1, 1, 1, 8, 4, "c32p16k8")         \
  X(11, 2, 2, 1, 1, 4, 4, "c32p32k4")

// LDS-staged conv_lds: id, MB, NB (16-blocks per wave), WM, WN (waves), KS, name.
#define CBS_LDS_CONFIG_LIST(X)               \
  X(12, 4, 2, 2, 2, 2, "L.p128c64")          \
  X(13, 2, 2, 2, 2, 2, "L.p64c64")           \
  X(14, 2, 4, 2, 2, 2, "L.p64c128")          \
  X(15, 2, 2, 2, 1, 2, "L.p64c32")           \
  X(16, 4, 4, 2, 2, 2, "L.p128c128")

// Halo-tile conv_halo: id, TH, TW (output tile), name.
#define CBS_HALO_CONFIG_LIST(X)              \
  X(17, 4, 64, "H.t4x64")                    \
  X(18, 8, 32, "H.t8x32")                    \
  X(19, 4, 32, "H.t4x32")                    \
  X(20, 2, 64, "H.t2x64")

// More register-direct conv_igemm tiles (ids continue after the halo list, so
// earlier ids stay valid): 64- and 32-channel x 32-pixel wave tiles and 8-way
// K splits, for the batch-1 3x3 layers, where every pixel tile re-reads all
// weights and a wider pixel tile halves that traffic; and 8-step prefetch
// rings for tiles that run one wave per SIMD, whose loop is bound by the
// latency of the loads in flight.
#define CBS_CONFIG_LIST_EXT(X)                \
  X(21, 4, 2, 1, 1, 4, 4, "c64p32k4")         \
  X(22, 4, 2, 1, 1, 8, 4, "c64p32k8")         \
  X(23, 2, 2, 1, 1, 8, 4, "c32p32k8")         \
  X(24, 4, 1, 1, 1, 8, 4, "c64p16k8")         \
  X(25, 2, 1, 1, 1, 4, 8, "c32p16k4f8")       \
  X(26, 4, 1, 1, 1, 4, 8, "c64p16k4f8")

// One more LDS-staged tile with a deeper K stage (4 fragment steps per stage
// instead of 2).  Deeper stages were measured for the int8 batch-16 3x3
// layers, where a 2-step stage of a 64 x 64 tile is only 128 cycles of MFMA
// work per wave: 4- and 8-step stages (the latter in 128 KB of LDS) take the
// same time per K step, so those layers are bound by operand throughput, not
// by the wait at each stage.  Only the 4-step 64 x 64 tile wins on some shapes
// (batch-1 and int8 1x1 layers, by up to 4%).
#define CBS_LDS_CONFIG_LIST_EXT(X)           \
  X(27, 2, 2, 2, 2, 4, "L.p64c64k4")

// LDS-staged tiles filled by direct-to-LDS loads through a ring of NS stage
// buffers (NS - 1 stages in flight): id, MB, NB, WM, WN, KS, NS, name.
#define CBS_LDS_RING_CONFIG_LIST(X)             \
  X(28, 2, 2, 2, 2, 2, 3, "R.p64c64k2s3")       \
  X(29, 2, 2, 2, 2, 2, 4, "R.p64c64k2s4")       \
  X(30, 2, 2, 2, 2, 1, 4, "R.p64c64k1s4")       \
  X(31, 2, 4, 2, 2, 1, 4, "R.p64c128k1s4")      \
  X(32, 4, 2, 2, 2, 1, 4, "R.p128c64k1s4")      \
  X(33, 2, 2, 2, 1, 2, 4, "R.p64c32k2s4")       \
  X(34, 2, 2, 2, 2, 1, 8, "R.p64c64k1s8")       \
  X(35, 4, 4, 2, 2, 1, 4, "R.p128c128k1s4")     \
  X(36, 4, 2, 2, 2, 1, 5, "R.p128c64k1s5")      \
  X(37, 2, 2, 2, 1, 1, 8, "R.p64c32k1s8")

// Column-pair halo tiles (3x3, stride 1, at most 8 output channels): one
// MFMA row block holds 8 output channels of two horizontally adjacent output
// pixels, whose 3 x 4 input window is one K row, so the 16-row block carries
// no channel padding: id, TH, TW (output tile of TH x TW pixel pairs), name.
#define CBS_HALO_PAIR_CONFIG_LIST(X)         \
  X(38, 4, 32, "P.t4x32")                    \
  X(39, 8, 16, "P.t8x16")                    \
  X(40, 2, 32, "P.t2x32")                    \
  X(41, 4, 16, "P.t4x16")                    \
  X(42, 8, 32, "P.t8x32")

// LDS-staged tiles whose activation loads go pixel by pixel (four lanes per
// pixel, swizzled LDS slots; see conv_lds), filled by the direct-to-LDS ring
// (RS, NS >= 2) or through registers (LS, NS = 0); "w8": eight waves, two per
// SIMD, share each stage: id, MB, NB, WM, WN, KS, NS, name.
#define CBS_LDS_RING_SWZ_CONFIG_LIST(X)         \
  X(43, 2, 2, 2, 2, 1, 4, "RS.p64c64k1s4")      \
  X(44, 2, 2, 2, 2, 2, 4, "RS.p64c64k2s4")      \
  X(45, 2, 4, 2, 2, 1, 4, "RS.p64c128k1s4")     \
  X(46, 4, 2, 2, 2, 1, 4, "RS.p128c64k1s4")     \
  X(47, 2, 2, 2, 1, 1, 8, "RS.p64c32k1s8")      \
  X(48, 4, 4, 2, 2, 1, 4, "RS.p128c128k1s4")    \
  X(49, 2, 2, 2, 1, 2, 0, "LS.p64c32")          \
  X(50, 2, 2, 2, 2, 2, 0, "LS.p64c64")          \
  X(51, 2, 4, 2, 2, 2, 0, "LS.p64c128")         \
  X(52, 4, 2, 2, 2, 2, 0, "LS.p128c64")         \
  X(53, 2, 1, 2, 4, 2, 4, "RS.p64c64w8")        \
  X(54, 2, 2, 4, 2, 2, 2, "RS.p128c64w8")       \
  X(55, 2, 2, 2, 4, 2, 2, "RS.p64c128w8")       \
  X(56, 2, 1, 2, 4, 2, 0, "LS.p64c64w8")

// conv_ws (fp32 1x1 stride 1): id, 16-channel blocks per wave, waves per
// workgroup along channels, waves per workgroup along pixels (on the same
// channel blocks, interleaving the run's pixel blocks), workgroups per CU.
#define CBS_WS_CONFIG_LIST(X)                \
  X(57, 2, 4, 1, 1, "W.c32x4")               \
  X(58, 2, 4, 1, 2, "W.c32x4o2")             \
  X(59, 1, 4, 1, 1, "W.c16x4")

// Weight-stationary tiles with the window gather (fp32 3x3 layers with 16
// or 32 padded input channels, 9 or 18 K steps): id, 16-channel blocks per
// wave, waves per workgroup (all on the same channel blocks, interleaving the
// run's pixel blocks), workgroups per CU.
#define CBS_WSG_CONFIG_LIST(X)               \
  X(60, 2, 4, 1, "G.c32x4")                  \
  X(61, 2, 4, 2, "G.c32x4o2")                \
  X(62, 1, 4, 2, "G.c16x4o2")                \
  X(63, 1, 4, 3, "G.c16x4o3")

// More conv_ws tiles, with the waves of a workgroup along pixels: layers with
// 16-32 output channels or 80 (the detection head's class branch), whose
// channel blocks one wave holds.  Same fields as CBS_WS_CONFIG_LIST.
#define CBS_WS_CONFIG_LIST_EXT(X)            \
  X(64, 1, 1, 4, 2, "W.c16p4o2")             \
  X(65, 1, 1, 4, 4, "W.c16p4o4")             \
  X(66, 2, 1, 4, 2, "W.c32p4o2")             \
  X(67, 5, 1, 4, 1, "W.c80p4")               \
  X(68, 5, 1, 4, 2, "W.c80p4o2")
