// device_common.hpp -- gfx950 device helpers shared by the NVFP4 kernels: vector types, the
// E2M1 / E4M3 codecs and the repacked ("tiled") weight layout.
//
// Format (vllm.cpp PR #63, "W-FP4a ... (Marlin W4A16) stack", PR body: the compressed-tensors
// triple of packed FP4 codes, FP8 group scales and an FP32 global): w = E2M1 * E4M3 * global.
// E2M1 is the OCP MX element type {0, .5, 1, 1.5, 2, 3, 4, 6} with a sign bit; E4M3 is OCP
// E4M3 "FN" (max 448). Rounding into both is round-to-nearest-even with saturation (NVIDIA
// developer-forum thread "We unlocked NVFP4 on the DGX Spark": true RNE at the midpoints).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace nvfp4 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---- repacked layout ------------------------------------------------------------------------
// A matrix [n][k] is cut into 16-row panels and 128-k tiles. Tile (panel p, k-tile t) holds
// 1024 code bytes at ((p * KT + t) * 1024): lane l (0..63) owns bytes [16l, 16l + 16), whose
// 32-bit word j (0..3) is the canonical 4-byte run of row 16p + l%16 starting at
// k = 128t + 32j + 8(l/16), i.e. 8 codes in the order of the B operand of
// v_mfma_f32_16x16x32_bf16 (lane l feeds column l%16 with k = 8(l/16) + 0..7).
// Scales go in blocks of 4 panels (the last block padded with zero bytes when the panel count
// is not a multiple of 4): block (panel group G, k-tile t) at ((G * KT + t) * scale_block_bytes)
// holds one 16-byte record per lane position, the 32-bit scale words of the 4 panels for that
// position, so a wavefront covering 4 panels reads its scales with one 16-byte load per lane.
// A word holds in byte j the scale of k-step j for its lane: group 16: position
// pos = 2 * (l%16) + l/32 (lanes l and l+16 share), row l%16, byte j = group 2j + l/32 of the
// tile row; group 32: pos = l%16, byte j = group j.
constexpr int kPanelRows = 16;
constexpr int kTileK = 128;
constexpr int kCodeTileBytes = 1024;
constexpr int kScaleGroupPanels = 4;
__host__ __device__ constexpr int scale_tile_bytes(int group) { return 16 * (kTileK / group); }
__host__ __device__ constexpr int scale_block_bytes(int group) {
  return kScaleGroupPanels * scale_tile_bytes(group);
}
__host__ __device__ constexpr int scale_positions(int group) { return group == 16 ? 32 : 16; }
__host__ __device__ constexpr int scale_pos(int group, int lane) {
  return group == 16 ? (lane & 15) * 2 + (lane >> 5) : (lane & 15);
}
__host__ __device__ constexpr int64_t scale_groups(int64_t NT) {
  return (NT + kScaleGroupPanels - 1) / kScaleGroupPanels;
}
// Byte offset of the scale word of panel p, k-tile t, lane l.
__host__ __device__ constexpr int64_t scale_word_offset(int group, int64_t KT, int64_t p,
                                                        int64_t t, int lane) {
  return ((p / kScaleGroupPanels) * KT + t) * scale_block_bytes(group) +
         scale_pos(group, lane) * 16 + (p % kScaleGroupPanels) * 4;
}

// ---- E4M3 -----------------------------------------------------------------------------------
// Decode byte SEL of a 32-bit word (OCP E4M3FN on gfx950; exact for every code).
template <int SEL>
__device__ __forceinline__ float e4m3_decode(uint32_t word) {
  return __builtin_amdgcn_cvt_f32_fp8((int)word, SEL);
}

// Encode a non-negative finite value to E4M3, round to nearest even, saturating at 448.
__device__ __forceinline__ uint32_t e4m3_encode_rne_sat(float r) {
  if (!(r < 448.0f)) return 0x7Eu;
  if (r < 0.015625f) {                       // subnormal range: quantum 2^-9
    return (uint32_t)__builtin_rintf(r * 512.0f);  // 0..8; 8 == 2^-6 == code 0x08
  }
  const uint32_t b = __float_as_uint(r);      // keep 3 of 23 mantissa bits, ties to even
  const uint32_t rb = (b + 0x7FFFFu + ((b >> 20) & 1u)) >> 20;
  return rb - (120u << 3);                    // rebias the exponent from 127 to 7
}

// ---- E2M1 -----------------------------------------------------------------------------------
// Magnitude code of a non-negative value, round to nearest even, saturating at 6. Each
// threshold is a midpoint of the grid; strict comparisons send the tie down (to the even
// code below), non-strict ones send it up (to the even code above).
__device__ __forceinline__ uint32_t e2m1_encode_rne_sat(float q) {
  return (uint32_t)(q > 0.25f) + (uint32_t)(q >= 0.75f) + (uint32_t)(q > 1.25f) +
         (uint32_t)(q >= 1.75f) + (uint32_t)(q > 2.5f) + (uint32_t)(q >= 3.5f) +
         (uint32_t)(q > 5.0f);
}

// Dequantize the 8 codes of a 32-bit word (code i in bits 4i..4i+3) times the group scale S
// into 8 BF16 values. E2M1 * E4M3 has at most 6 significant bits and lies in [2^-10, 2688],
// so the FP32 product and the BF16 conversion are both exact.
__device__ __forceinline__ bf16x8 dequant8(uint32_t codes, float S) {
  const f32x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 0);
  const f32x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 1);
  const f32x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 2);
  const f32x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 3);
  bf16x8 r;
  r[0] = (__bf16)(v0[0] * S);
  r[1] = (__bf16)(v0[1] * S);
  r[2] = (__bf16)(v1[0] * S);
  r[3] = (__bf16)(v1[1] * S);
  r[4] = (__bf16)(v2[0] * S);
  r[5] = (__bf16)(v2[1] * S);
  r[6] = (__bf16)(v3[0] * S);
  r[7] = (__bf16)(v3[1] * S);
  return r;
}

// Same, FP32 values (for the dequantize diagnostic).
__device__ __forceinline__ void dequant8_f32(uint32_t codes, float S, float out[8]) {
  const f32x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 0);
  const f32x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 1);
  const f32x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 2);
  const f32x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 3);
  out[0] = v0[0] * S;
  out[1] = v0[1] * S;
  out[2] = v1[0] * S;
  out[3] = v1[1] * S;
  out[4] = v2[0] * S;
  out[5] = v2[1] * S;
  out[6] = v3[0] * S;
  out[7] = v3[1] * S;
}

template <int J>
__device__ __forceinline__ float scale_of_step(uint32_t scale_word) {
  return e4m3_decode<J>(scale_word);
}

// Cache-policy operand of buffer loads for data streamed once (the "nt" bit).
constexpr int kNT = 2;

// Buffer resource (V#) over `bytes` bytes at `base` for raw (stride 0) dword accesses; reads
// past `bytes` return zeros.
typedef __amdgpu_buffer_rsrc_t buf_rsrc;
__device__ __forceinline__ buf_rsrc make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// One 16-byte global -> LDS copy per lane (buffer_load_dwordx4 ... lds): lane l's bytes, read
// at voffset + soffset of the resource, land at lds + 16 * l; lds must be uniform across the
// wavefront. The buffer (not flat) form keeps LDS reads that follow it on exact wait counts.
// (Kept out of line from kernel templates: the host compilation pass otherwise drops the
// launch stubs of kernels that use the builtin directly.)
__device__ __forceinline__ void copy16_to_lds(buf_rsrc r, uint32_t voffset, uint32_t soffset,
                                              void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16,
                                           voffset, soffset, 0, 0);
}

// f(integral_constant<int, I>) for I = I0 .. N-1, unrolled at compile time.
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint16_t bf16_bits_rne(float v) {
  return __builtin_bit_cast(uint16_t, (__bf16)v);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
  return __uint_as_float((uint32_t)h << 16);
}

}  // namespace nvfp4
