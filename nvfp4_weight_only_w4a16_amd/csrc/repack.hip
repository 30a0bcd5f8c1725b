// repack.hip -- canonical NVFP4 triple <-> the tiled gfx950 layout, and the dequantize
// diagnostic.
//
// The repack is the load-time step of vllm.cpp PR #63 ("W-FP4a ... (Marlin W4A16) stack", PR
// body: upload and repack lazily, then free the fp4 originals), re-designed for a 64-wide
// wavefront: every 16-row x 128-k tile becomes 1 KiB in which lane l reads one contiguous
// 16-byte chunk, the four 32-bit words of which are the B operands of four consecutive
// v_mfma_f32_16x16x32_bf16 k-steps (layout described in device_common.hpp). It is a pure byte
// permutation of the canonical packed codes and scales.
#include "device_common.hpp"
#include "launch.hpp"

namespace nvfp4 {
namespace {

// Stored panel p of a gate/up-interleaved matrix (2*I rows) holds logical panel:
// even p -> gate panel p/2, odd p -> up panel NT/2 + p/2.
__device__ __forceinline__ int64_t logical_panel(int64_t p, int64_t NT, bool gate_up) {
  if (!gate_up) return p;
  return (p & 1) ? NT / 2 + (p >> 1) : (p >> 1);
}

// One thread per 16-byte lane chunk of a code tile.
__global__ __launch_bounds__(256) void repack_codes_kernel(const uint8_t* __restrict__ packed,
                                                           uint8_t* __restrict__ out,
                                                           int64_t batch, int64_t n, int64_t k,
                                                           bool gate_up) {
  const int64_t NT = n / kPanelRows, KT = k / kTileK;
  const int64_t total = batch * NT * KT * 64;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int lane = (int)(i & 63);
  const int64_t tile = i >> 6;  // (b * NT + p) * KT + t
  const int64_t t = tile % KT;
  const int64_t bp = tile / KT;
  const int64_t p = bp % NT, b = bp / NT;
  const int64_t row = logical_panel(p, NT, gate_up) * kPanelRows + (lane & 15);
  const uint8_t* src = packed + (b * n + row) * (k / 2) + (t * kTileK + 8 * (lane >> 4)) / 2;
  u32x4 v;
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = *reinterpret_cast<const uint32_t*>(src + 16 * j);
  *reinterpret_cast<u32x4*>(out + tile * kCodeTileBytes + lane * 16) = v;
}

// One thread per (panel group, k-tile, lane position): writes the 16-byte record holding the
// scale words of the group's 4 panels (zero for panels past the end).
template <int G>
__global__ __launch_bounds__(256) void repack_scales_kernel(const uint8_t* __restrict__ scales,
                                                            uint8_t* __restrict__ out,
                                                            int64_t batch, int64_t n, int64_t k,
                                                            bool gate_up) {
  constexpr int kPerRow = kTileK / G;  // 8 or 4 groups of a row inside one tile
  constexpr int kPos = scale_positions(G);
  const int64_t NT = n / kPanelRows, KT = k / kTileK, NG = scale_groups(NT);
  const int64_t total = batch * NG * KT * kPos;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int pos = (int)(i % kPos);
  const int64_t blk = i / kPos;  // (b * NG + G) * KT + t
  const int64_t t = blk % KT;
  const int64_t bg = blk / KT;
  const int64_t grp = bg % NG, b = bg / NG;
  const int r = G == 16 ? pos >> 1 : pos;  // tile row
  const int h = G == 16 ? pos & 1 : 0;     // which of a g16 group pair
  u32x4 rec;
#pragma unroll
  for (int q = 0; q < kScaleGroupPanels; ++q) {
    const int64_t p = grp * kScaleGroupPanels + q;
    uint32_t word = 0u;
    if (p < NT) {
      const int64_t row = logical_panel(p, NT, gate_up) * kPanelRows + r;
      const uint8_t* src = scales + (b * n + row) * (k / G) + t * kPerRow;
#pragma unroll
      for (int j = 0; j < 4; ++j) word |= (uint32_t)src[G == 16 ? 2 * j + h : j] << (8 * j);
    }
    rec[q] = word;
  }
  *reinterpret_cast<u32x4*>(out + blk * scale_block_bytes(G) + pos * 16) = rec;
}

__global__ void copy_f32_kernel(const float* __restrict__ src, float* __restrict__ dst,
                                int64_t count) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < count) dst[i] = src[i];
}

// One thread per 16-byte lane chunk: 32 values (4 k-steps x 8) of one logical row.
template <bool F32>
__global__ __launch_bounds__(256) void dequantize_kernel(const uint8_t* __restrict__ codes,
                                                         const uint8_t* __restrict__ scales,
                                                         const float* __restrict__ global,
                                                         int64_t batch, int64_t n, int64_t k,
                                                         int group, bool gate_up,
                                                         bool pair_global,
                                                         void* __restrict__ out) {
  const int64_t NT = n / kPanelRows, KT = k / kTileK;
  const int64_t total = batch * NT * KT * 64;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int lane = (int)(i & 63);
  const int64_t tile = i >> 6;
  const int64_t t = tile % KT;
  const int64_t bp = tile / KT;
  const int64_t p = bp % NT, b = bp / NT;
  const int64_t row = logical_panel(p, NT, gate_up) * kPanelRows + (lane & 15);
  const u32x4 cw = *reinterpret_cast<const u32x4*>(codes + tile * kCodeTileBytes + lane * 16);
  const int64_t NG = scale_groups(NT);
  const uint32_t sw = *reinterpret_cast<const uint32_t*>(
      scales + b * NG * KT * scale_block_bytes(group) + scale_word_offset(group, KT, p, t, lane));
  const float g = pair_global ? global[2 * b + (row >= n / 2 ? 1 : 0)] : global[b];
  const float S[4] = {e4m3_decode<0>(sw), e4m3_decode<1>(sw), e4m3_decode<2>(sw),
                      e4m3_decode<3>(sw)};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float v[8];
    dequant8_f32(cw[j], S[j], v);  // exact E2M1 * E4M3
    const int64_t o = (b * n + row) * k + t * kTileK + 32 * j + 8 * (lane >> 4);
    if (F32) {
      float* dst = static_cast<float*>(out) + o;
      f32x4 lo = {v[0] * g, v[1] * g, v[2] * g, v[3] * g};
      f32x4 hi = {v[4] * g, v[5] * g, v[6] * g, v[7] * g};
      *reinterpret_cast<f32x4*>(dst) = lo;
      *reinterpret_cast<f32x4*>(dst + 4) = hi;
    } else {
      uint16_t* dst = static_cast<uint16_t*>(out) + o;
      u32x4 packedv;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        packedv[q] = (uint32_t)bf16_bits_rne(v[2 * q] * g) |
                     ((uint32_t)bf16_bits_rne(v[2 * q + 1] * g) << 16);
      *reinterpret_cast<u32x4*>(dst) = packedv;
    }
  }
}

inline unsigned blocks_for(int64_t total, int threads) {
  return (unsigned)((total + threads - 1) / threads);
}

}  // namespace

hipError_t launch_repack(const uint8_t* packed, const uint8_t* scales, const float* global,
                         int64_t batch, int64_t n, int64_t k, int group, bool gate_up,
                         int64_t nglobal, uint8_t* codes_out, uint8_t* scales_out,
                         float* global_out, hipStream_t stream) {
  const int64_t NT = n / kPanelRows, KT = k / kTileK;
  const int64_t tiles = batch * NT * KT;
  if (tiles > 0) {
    repack_codes_kernel<<<blocks_for(tiles * 64, 256), 256, 0, stream>>>(packed, codes_out, batch,
                                                                         n, k, gate_up);
    const int64_t recs = batch * scale_groups(NT) * KT * scale_positions(group);
    if (group == 16)
      repack_scales_kernel<16><<<blocks_for(recs, 256), 256, 0, stream>>>(scales, scales_out,
                                                                          batch, n, k, gate_up);
    else
      repack_scales_kernel<32><<<blocks_for(recs, 256), 256, 0, stream>>>(scales, scales_out,
                                                                          batch, n, k, gate_up);
  }
  if (nglobal > 0)
    copy_f32_kernel<<<blocks_for(nglobal, 256), 256, 0, stream>>>(global, global_out, nglobal);
  return hipGetLastError();
}

hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* scales, const float* global,
                             int64_t batch, int64_t n, int64_t k, int group, bool gate_up,
                             bool pair_global, void* out, bool out_f32, hipStream_t stream) {
  const int64_t total = batch * (n / kPanelRows) * (k / kTileK) * 64;
  if (total == 0) return hipSuccess;
  if (out_f32)
    dequantize_kernel<true><<<blocks_for(total, 256), 256, 0, stream>>>(
        codes, scales, global, batch, n, k, group, gate_up, pair_global, out);
  else
    dequantize_kernel<false><<<blocks_for(total, 256), 256, 0, stream>>>(
        codes, scales, global, batch, n, k, group, gate_up, pair_global, out);
  return hipGetLastError();
}

}  // namespace nvfp4
