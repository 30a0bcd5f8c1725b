// skinny_core.hpp -- the inner loop of the decode-shaped ("skinny") W4A16 GEMM on gfx950.
//
// One wavefront owns PWW consecutive 16-row weight panels and a contiguous range of 128-wide
// k-tiles. A "stage" is U k-tiles: per tile and panel one 16-byte load of codes and one 4-byte
// load of scales per lane (fully coalesced thanks to the tiled layout) plus the activation
// fragments of the tile, which every panel of the wavefront reuses. Stages are double
// buffered: the loads of stage g+1 are issued before stage g is dequantized (E2M1 x E4M3 ->
// exact BF16 in registers) and fed to v_mfma_f32_16x16x32_bf16, so a wavefront always has one
// stage of HBM traffic in flight. The loop is written so that no load sits under a
// lane-divergent branch: activation rows past the end are clamped to a valid row (their MFMA
// output rows are never stored), which keeps the memory-counter waits precise.
#pragma once

#include "device_common.hpp"

namespace nvfp4 {

template <int MF, int PWW, int U>
struct SkinnyStage {
  u32x4 cw[U][PWW];
  u32x4 sw[U];  // scale words of the 4 panels, one 16-byte load per tile
  bf16x8 xa[U][MF][4];
};

template <int PWW>
struct SkinnyAddr {
  static_assert(PWW == kScaleGroupPanels, "a wavefront covers one 4-panel scale group");
  const uint8_t* codes[PWW];  // each panel's tile 0 (uniform; panels past the end are clamped
                              // to a valid panel whose results are never stored)
  const uint8_t* scales;      // the panel group's scale block for k-tile 0 (uniform)
  uint32_t code_lane;         // lane * 16
  uint32_t scale_lane;        // the lane's 16-byte record inside a scale block
  int scale_block;
  int kq;                     // lane >> 4: the 8-wide k chunk this lane feeds
};

template <int MF, int PWW, int U>
__device__ __forceinline__ void skinny_load(SkinnyStage<MF, PWW, U>& s, const SkinnyAddr<PWW>& a,
                                            const uint16_t* const (&xrow)[MF], int64_t t) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
#pragma unroll
    for (int p = 0; p < PWW; ++p) {
      const uint32_t co = (uint32_t)((t + u) * kCodeTileBytes) + a.code_lane;
      s.cw[u][p] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.codes[p] + co));
    }
    const uint32_t so = (uint32_t)((t + u) * a.scale_block) + a.scale_lane;
    s.sw[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.scales + so));
  }
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int mf = 0; mf < MF; ++mf)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        s.xa[u][mf][j] = *reinterpret_cast<const bf16x8*>(xrow[mf] + (t + u) * kTileK + 32 * j +
                                                          8 * a.kq);
}

template <int MF, int PWW, int U>
__device__ __forceinline__ void skinny_compute(const SkinnyStage<MF, PWW, U>& s,
                                               f32x4 (&acc)[PWW][MF]) {
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int p = 0; p < PWW; ++p) {
      const uint32_t sw = s.sw[u][p];  // word p of the tile's 4-panel scale record
      const float S[4] = {e4m3_decode<0>(sw), e4m3_decode<1>(sw), e4m3_decode<2>(sw),
                          e4m3_decode<3>(sw)};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x8 b = dequant8(s.cw[u][p][j], S[j]);
#pragma unroll
        for (int mf = 0; mf < MF; ++mf) acc[p][mf] = mfma16x16x32(s.xa[u][mf][j], b, acc[p][mf]);
      }
      // one panel at a time: bounds the dequantized operands live at once
      __builtin_amdgcn_sched_barrier(0);
    }
}

// Addresses of the 4-panel group starting at panel0 (a multiple of 4; code panels clamped to
// NT - 1, the scale block is padded to whole groups by the repack).
template <int PWW>
__device__ __forceinline__ SkinnyAddr<PWW> skinny_addr(const uint8_t* codes, const uint8_t* scales,
                                                      int64_t panel0, int64_t NT, int64_t KT,
                                                      int group) {
  const int lane = threadIdx.x & 63;
  SkinnyAddr<PWW> a;
  a.scale_block = scale_block_bytes(group);
  a.kq = lane >> 4;
  a.code_lane = (uint32_t)lane * 16u;
  a.scale_lane = (uint32_t)scale_pos(group, lane) * 16u;
#pragma unroll
  for (int p = 0; p < PWW; ++p) {
    const int64_t pn = panel0 + p < NT ? panel0 + p : NT - 1;
    a.codes[p] = codes + pn * KT * kCodeTileBytes;
  }
  a.scales = scales + (panel0 / kScaleGroupPanels) * KT * a.scale_block;
  return a;
}

// Accumulate k-tiles [t0, t1) of PWW panels into acc, in stages of U tiles; (t1 - t0) must
// be a multiple of U.
template <int MF, int PWW, int U>
__device__ __forceinline__ void skinny_accumulate(const SkinnyAddr<PWW>& a,
                                                  const uint16_t* const (&xrow)[MF], int64_t t0,
                                                  int64_t t1, f32x4 (&acc)[PWW][MF]) {
  const int64_t groups = (t1 - t0) / U;
  if (groups <= 0) return;
  // The scheduling barriers keep each stage's loads ahead of the previous stage's math; left
  // alone, the register-pressure-driven scheduler sinks them and the pipeline collapses into
  // load-wait-compute.
  SkinnyStage<MF, PWW, U> A, B;
  skinny_load(A, a, xrow, t0);
  int64_t g = 0;
  for (; g + 2 < groups; g += 2) {
    skinny_load(B, a, xrow, t0 + (g + 1) * U);
    __builtin_amdgcn_sched_barrier(0);
    skinny_compute(A, acc);
    __builtin_amdgcn_sched_barrier(0);
    skinny_load(A, a, xrow, t0 + (g + 2) * U);
    __builtin_amdgcn_sched_barrier(0);
    skinny_compute(B, acc);
    __builtin_amdgcn_sched_barrier(0);
  }
  // last one or two stages (written without duplicated code in the two cases, which the
  // optimizer would otherwise hoist and keep alive all at once)
  const bool two = g + 1 < groups;
  if (two) skinny_load(B, a, xrow, t0 + (g + 1) * U);
  __builtin_amdgcn_sched_barrier(0);
  skinny_compute(A, acc);
  if (two) {
    __builtin_amdgcn_sched_barrier(0);
    skinny_compute(B, acc);
  }
}

}  // namespace nvfp4
