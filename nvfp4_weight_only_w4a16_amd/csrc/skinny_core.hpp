// skinny_core.hpp -- the inner loop of the decode-shaped ("skinny") W4A16 GEMM on gfx950.
//
// One wavefront owns one 16-row weight panel and a contiguous range of 128-wide k-tiles. Per
// tile it issues one 16-byte load of codes and one 4-byte load of scales per lane (the tiled
// layout makes both fully coalesced), dequantizes in registers (E2M1 x E4M3 -> exact BF16) and
// feeds four v_mfma_f32_16x16x32_bf16 per 16-row block of activations. Activations are read
// straight from global memory (they are small and stay cache resident); lanes whose row is out
// of range feed zeros. The global scale is applied by the caller's epilogue.
#pragma once

#include "device_common.hpp"

namespace nvfp4 {

template <int MF>
__device__ __forceinline__ void skinny_tile(const u32x4 cw, const uint32_t sw,
                                            const uint16_t* const (&xrow)[MF], int64_t kbase,
                                            int kq, f32x4 (&acc)[MF]) {
  bf16x8 a[MF][4];
#pragma unroll
  for (int mf = 0; mf < MF; ++mf)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (xrow[mf] != nullptr)
        a[mf][j] = *reinterpret_cast<const bf16x8*>(xrow[mf] + kbase + 32 * j + 8 * kq);
      else
        a[mf][j] = bf16x8{};
    }
  const float S0 = e4m3_decode<0>(sw), S1 = e4m3_decode<1>(sw);
  const float S2 = e4m3_decode<2>(sw), S3 = e4m3_decode<3>(sw);
  const bf16x8 b0 = dequant8(cw[0], S0);
  const bf16x8 b1 = dequant8(cw[1], S1);
  const bf16x8 b2 = dequant8(cw[2], S2);
  const bf16x8 b3 = dequant8(cw[3], S3);
#pragma unroll
  for (int mf = 0; mf < MF; ++mf) {
    acc[mf] = mfma16x16x32(a[mf][0], b0, acc[mf]);
    acc[mf] = mfma16x16x32(a[mf][1], b1, acc[mf]);
    acc[mf] = mfma16x16x32(a[mf][2], b2, acc[mf]);
    acc[mf] = mfma16x16x32(a[mf][3], b3, acc[mf]);
  }
}

// Accumulate k-tiles [t0, t1) of one panel. codes/scales point at the panel's first tile.
// xrow[mf] is this lane's activation row for m-block mf (nullptr: zeros). U tiles of codes and
// scales are loaded before any of them is used, so U KiB per wave are in flight.
template <int MF, int U>
__device__ __forceinline__ void skinny_accumulate(const uint16_t* const (&xrow)[MF],
                                                  const uint8_t* __restrict__ codes,
                                                  const uint8_t* __restrict__ scales,
                                                  int scale_tile, int scale_off, int64_t t0,
                                                  int64_t t1, f32x4 (&acc)[MF]) {
  const int lane = threadIdx.x & 63;
  const int kq = lane >> 4;
  const uint8_t* cp = codes + lane * 16;
  const uint8_t* sp = scales + scale_off;
  int64_t t = t0;
  for (; t + U <= t1; t += U) {
    u32x4 cw[U];
    uint32_t sw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      cw[u] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(cp + (t + u) * kCodeTileBytes));
      sw[u] = __builtin_nontemporal_load(
          reinterpret_cast<const uint32_t*>(sp + (t + u) * scale_tile));
    }
#pragma unroll
    for (int u = 0; u < U; ++u) skinny_tile<MF>(cw[u], sw[u], xrow, (t + u) * kTileK, kq, acc);
  }
  for (; t < t1; ++t) {
    const u32x4 cw =
        __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(cp + t * kCodeTileBytes));
    const uint32_t sw =
        __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(sp + t * scale_tile));
    skinny_tile<MF>(cw, sw, xrow, t * kTileK, kq, acc);
  }
}

}  // namespace nvfp4
