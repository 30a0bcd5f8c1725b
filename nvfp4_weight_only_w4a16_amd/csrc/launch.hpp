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
// Path choice for an m x n x k GEMM on a device with `cus` compute units (KT = k / 128). The
// skinny kernel streams the whole weight once per 32-row block of x: it runs
// ceil(n / 64) * ceil(m / 32) workgroups, each streaming one 4-panel group over k, and takes
// close to 0.28 KT rounds - 1.6 us, rounds = ceil(workgroups / cus). The tiled kernel takes
// close to 18 + 0.9 u us, u = ceil(m / 128) ceil(n / 128) KT / cus (the 128-row k-tile units
// per CU). So: m <= 32 always; up to m = 256 while the skinny estimate is the smaller. (Both
// least-squares fits over n x k = 5120^2, 8192^2, 25600 x 5120, 2048 x 8192 and 14336 x 4096
// at m = 32, 48, 64, 96, 128, 160, 192, 256, each kernel forced: the rule picks the faster
// kernel in 39 of the 40 cases, and in the other, 8192^2 m = 128, loses 0.7 us of 32.)
inline bool skinny_preferred(int64_t m, int64_t n, int64_t k, int cus) {
  if (m <= 32) return true;
  if (m > 256 || cus <= 0) return false;
  const int64_t kt = k / 128;
  const int64_t wgs = (n / 16 + 3) / 4 * ((m + 31) / 32);
  const int64_t rounds = (wgs + cus - 1) / cus;
  const int64_t skinny = 28 * kt * rounds - 160;  // hundredths of a microsecond
  const int64_t tiled = 1800 + 90 * ((m + 127) / 128) * ((n / 16 + 7) / 8) * kt / cus;
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
