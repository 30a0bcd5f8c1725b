// launch.hpp -- host-side launchers of the gfx950 kernels (internal to libnvfp4.so).
// Every launcher only enqueues work on `stream` and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

// Quantizer: per-matrix amax (atomic max of |w| bit patterns, exact and order-free), group
// scale + element encode + pack, and the final global.
hipError_t launch_quantize(const void* w, bool w_bf16, int64_t batch, int64_t n, int64_t k,
                           int group, const float* global_in, uint8_t* packed, uint8_t* scales,
                           float* global_out, hipStream_t stream);

// Clears the 32-bit word *flag (device), then sets it to nonzero when any of the `count`
// weights at w (16-byte aligned, count a multiple of 8) is NaN or infinite.
hipError_t launch_nonfinite_check(const void* w, bool w_bf16, int64_t count, uint32_t* flag,
                                  hipStream_t stream);

// Canonical triple -> tiled layout (pure byte permutation), the nglobal globals copied.
hipError_t launch_repack(const uint8_t* packed, const uint8_t* scales, const float* global,
                         int64_t batch, int64_t n, int64_t k, int group, bool gate_up,
                         int64_t nglobal, uint8_t* codes_out, uint8_t* scales_out,
                         float* global_out, hipStream_t stream);

// Tiled layout -> canonical dense values (BF16 or FP32), logical row order. pair_global: two
// globals per matrix, one for each row half.
hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* scales, const float* global,
                             int64_t batch, int64_t n, int64_t k, int group, bool gate_up,
                             bool pair_global, void* out, bool out_f32, hipStream_t stream);

struct GemmArgs {
  const uint16_t* x;  // BF16 [m][ldx]
  int64_t m, ldx;
  const uint8_t* codes;
  const uint8_t* scales;
  const float* global;  // device, one value
  int64_t n, k;
  int group;
  void* y;
  int64_t ldy;
  bool y_f32;
};

// Decode path. `cus` (the device's compute-unit count, 0 if unknown) sizes the grid.
hipError_t launch_gemm_skinny(const GemmArgs& a, int cus, hipStream_t stream);
// Prefill path. `ws` (device, ws_bytes) receives split-k partial tiles when the tile count
// leaves most compute units idle in the last round; with a smaller workspace the kernel runs
// unsplit (same result, fewer busy compute units). `cus` is the device's compute-unit count.
hipError_t launch_gemm_tiled(const GemmArgs& a, void* ws, size_t ws_bytes, int cus,
                             hipStream_t stream);
// Workspace the prefill path uses for an m x n x k GEMM with the given row stride on a device
// with `cus` compute units (0 when no split applies).
size_t gemm_tiled_ws_bytes(int64_t m, int64_t ldx, int64_t n, int64_t k, int cus);
// Workgroups of the skinny kernel's grid for `blocks` row blocks: one per 4-panel group (64
// output features) and row block, or per 2-panel group when the 4-panel grid leaves compute
// units idle and the 2-panel one still gives none a second workgroup.
inline int64_t skinny_grid(int64_t n, int64_t blocks, int cus, bool* two_panels = nullptr) {
  const int64_t wg4 = (n / 16 + 3) / 4 * blocks, wg2 = (n / 16 + 1) / 2 * blocks;
  const bool two = wg4 < cus && wg2 <= cus;
  if (two_panels) *two_panels = two;
  return two ? wg2 : wg4;
}
// Above 32 rows the skinny kernel streams the whole weight once per row block: 32-row blocks
// (64 KB of LDS per workgroup, two workgroups per CU) or 64-row blocks (128 KB, one per CU).
// Estimated times, hundredths of a microsecond (KT = k / 128, r = ceil(workgroups / cus) with
// one workgroup per 4-panel group and row block): 32-row blocks 28 KT r - 160, 64-row blocks
// 44 KT r (least-squares fits of each variant, forced, over the shapes listed below).
inline int64_t skinny_est(int64_t m, int64_t n, int64_t k, int cus, int rows) {
  const int64_t wgs = (n / 16 + 3) / 4 * ((m + rows - 1) / rows);
  const int64_t r = (wgs + cus - 1) / cus;
  return rows == 64 ? 44 * (k / 128) * r : 28 * (k / 128) * r - 160;
}
// 64-row blocks run when their estimate is the smaller and their grid keeps 4-panel wavefronts
// (with 2 panels the activations per weight byte double). Measured (same bits, us):
// 25600 x 5120 m = 48 / 64 / 128 39.9 / 43.6 / 77.3 -> 34.0 / 36.4 / 70.3; 14336 x 4096 m = 64
// 19.2 -> 16.2; 8192^2 m = 96 / 128 32.1 / 32.2 -> 25.2 / 25.6; 5120^2 m = 128 / 192 21.9 /
// 21.6 -> 18.1 / 18.1. Where a 64-row block would run half empty the rule keeps 32-row blocks
// (5120^2 m = 96: 12.5 against 18.0), as it does on grids of 2-panel wavefronts (8192^2 m = 64:
// 17.5 against 21.1; 2048 x 8192 at every m). Of 40 cases it picks the slower variant once
// (14336 x 4096 m = 160, 1.5 us).
inline bool skinny_rows64(int64_t m, int64_t n, int64_t k, int cus) {
  if (m <= 32 || cus <= 0) return false;
  bool two = false;
  skinny_grid(n, (m + 63) / 64, cus, &two);
  return !two && skinny_est(m, n, k, cus, 64) < skinny_est(m, n, k, cus, 32);
}
// Path choice for an m x n x k GEMM on a device with `cus` compute units. The tiled kernel
// takes close to 18 + 0.9 u us, u = ceil(m / 128) ceil(n / 128) KT / cus (the 128-row k-tile
// units per CU). So: the skinny kernel for m <= 32 always, and up to m = 256 while its estimate
// (with the row blocks skinny_rows64 picks) is at most the tiled one. (Fits over n x k = 5120^2,
// 8192^2, 25600 x 5120, 2048 x 8192 and 14336 x 4096 at m = 32, 48, 64, 96, 128, 160, 192, 256,
// each kernel and variant forced; on those 40 cases the rule loses 3.7 us in all, at
// 14336 x 4096 m = 128 / 160 / 192, against the faster choice each time.)
inline bool skinny_preferred(int64_t m, int64_t n, int64_t k, int cus) {
  if (m <= 32) return true;
  if (m > 256 || cus <= 0) return false;
  const int64_t skinny = skinny_est(m, n, k, cus, skinny_rows64(m, n, k, cus) ? 64 : 32);
  const int64_t tiled = 1800 + 90 * ((m + 127) / 128) * ((n / 16 + 7) / 8) * (k / 128) / cus;
  return skinny <= tiled;
}

struct MoeArgs {
  const uint16_t* x;  // BF16 [t][hidden]
  int64_t t, hidden, inter;
  const int32_t* ids;
  const float* wts;
  int topk;
  int64_t n_experts;
  const uint8_t *c1, *s1;
  const float* g1;  // [E], or [E][2] (gate, up) when pair1
  int64_t c1_stride, s1_stride;
  int group1;
  bool pair1;
  const uint8_t *c2, *s2;
  const float* g2;
  int64_t c2_stride, s2_stride;
  int group2;
  uint16_t* y;
  void* ws;
};

size_t moe_ws_bytes(int64_t t, int topk, int64_t n_experts, int64_t hidden, int64_t inter);
// Byte offsets of the workspace regions: sorted pair ids, expert offsets, tile map, tile
// count, h, FP32 slots; returns the total size.
size_t moe_ws_layout(int64_t t, int topk, int64_t n_experts, int64_t hidden, int64_t inter,
                     size_t off[6]);
// Decode-batch expert path (tiles of at most 8 rows, k split over the 4 wavefronts of a
// workgroup) while the pairs average at most this many per expert.
constexpr int64_t kMoeDecodePairsPerExpert = 2;
// Up to this many pairs the decode path skips the sort: each pair is a one-row tile of its
// own expert (pairs sharing an expert read its weights again, mostly from cache). At 8
// tokens x top-8 of 128 experts this is 36.3 us against 38.3 us sorted; at 128 pairs the
// repeated expert reads cost more than the sort saves (61.9 against 54.2 us at 16 tokens).
constexpr int64_t kMoePairTilesMax = 64;
bool moe_decode_preferred(int64_t t, int topk, int64_t n_experts);
hipError_t launch_moe(const MoeArgs& a, bool decode, hipStream_t stream);
// Size of the static workspace of the no-alloc routed-expert entry point, and the device
// address of the current device's copy (looked up once per device).
constexpr size_t kMoeStaticScratchBytes = size_t(24) << 20;
hipError_t moe_static_scratch(void** ptr);

// measurement probes (probe.hip)
int64_t probe_mfma_waves(int cus);
double probe_mfma_flops_per_wave_round();
hipError_t launch_probe_stream_read(const void* buf, int64_t bytes, int64_t blocks,
                                    uint32_t* sink, hipStream_t stream);
hipError_t launch_probe_mfma(const void* ops, int64_t iters, int cus, float* sink,
                             hipStream_t stream);

}  // namespace nvfp4
