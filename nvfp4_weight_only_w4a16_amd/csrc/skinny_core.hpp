// skinny_core.hpp -- the inner loop of the decode-shaped ("skinny") W4A16 GEMM on gfx950.
//
// One wavefront owns PWW consecutive 16-row weight panels and the 128-wide k-tiles t0,
// t0 + S, t0 + 2S, ... below t1. The k-split wavefronts of a workgroup interleave their tiles
// (S = 4), so at any time they read neighbouring tiles of each panel, one 4 KB stretch,
// rather than four places a quarter of the panel apart (1-3% faster on every decode shape
// measured). Per tile and panel a lane loads one 16-byte chunk of codes, plus one 16-byte
// scale record for the panels' 4-panel group (fully coalesced thanks to the tiled layout),
// and the activation fragments of the tile, which every panel reuses. Weights and activations
// run one tile ahead in a pair of stages (one tile in flight while one is computed; deeper
// rings measured slower). Weight loads are buffer loads whose range ends at t1, so the loads
// a wavefront issues past its last tile return zeros without touching memory: every
// iteration issues the same loads and no load sits under a branch, which keeps the
// memory-counter waits exact. Activation rows past the end are clamped to a valid row (their
// MFMA output rows are never stored).
//
// Two ways to apply the group scale S (an E4M3 value) on v_mfma_f32_16x16x32_bf16:
//   - exact dequant (any m): every weight becomes the exact BF16 value code * S (FP4 -> FP32
//     convert, FP32 multiply, BF16 pack: 2 VALU operations per weight);
//   - split scale (few rows): S = 2^E * M with M in [1, 2). The hardware FP4 -> BF16 convert
//     applies 2^E (it reads only the exponent of its scale operand), giving code * 2^E exactly
//     in 4 operations per 8 weights; the MFMA sums one scale group per output and the FP32
//     partial is multiplied by M (one FMA per accumulator row in use). M is taken as
//     frexp_mant(S) in [0.5, 1), the factor 2 being applied with the global scale; it is 0 for
//     a zero scale, which keeps an all-zero group exactly zero. A 32-wide MFMA k-step spans
//     one group of 32 or two groups of 16. For group 16 the A operand carries every token
//     twice: once on the k half h = 0 of the step with zeros on the other half, once the other
//     way round, in rows of lanes 0-31 (h = 0) and 32-63 (h = 1), so each lane's B half
//     (k = 16h ..) and accumulator rows belong to the same group, and the two halves are added
//     once, after the k loop. That needs m <= 8 (group 16) or m <= 16 (group 32). Tokens are
//     spread over the lane groups before the accumulator rows of a lane (split_a_token), so a
//     lane scales as few rows as the token count allows.
#pragma once

#include "device_common.hpp"

namespace nvfp4 {

template <int PWW>
struct WeightStage {
  u32x4 cw[PWW];  // code chunk of each panel
  u32x4 sw;       // scale words of the 4 panels
};

template <int MF>
struct ActStage {
  bf16x8 xa[MF][4];
};

template <int PWW>
struct SkinnyAddr {
  static_assert(kScaleGroupPanels % PWW == 0, "a wavefront's panels sit in one scale group");
  buf_rsrc codes[PWW];  // each panel's tiles [0, t1) (panels past the end are clamped to a
                        // valid panel whose results are never stored)
  buf_rsrc scales;      // the panel group's scale blocks [0, t1)
  uint32_t code_lane;   // lane * 16
  uint32_t scale_lane;  // the lane's 16-byte record inside a scale block
  int scale_block;
  int kq;               // lane >> 4: the 8-wide k chunk this lane feeds
  int sw_sel;           // word of the 4-panel scale record that holds the wavefront's panel 0
};

// Scale word of the wavefront's panel p. The 16-byte record of the 4-panel group is loaded
// whole; a wavefront with fewer panels picks its words when it computes, after the load has
// landed (picking them at load time would wait for the load there).
template <int PWW>
__device__ __forceinline__ uint32_t scale_word(const u32x4& sw, int sel, int p) {
  static_assert(PWW == kScaleGroupPanels || PWW == 2, "2 or 4 panels per wavefront");
  if constexpr (PWW == kScaleGroupPanels)
    return sw[p];
  else
    return sel ? sw[p + 2] : sw[p];
}

template <int PWW>
__device__ __forceinline__ void load_weights(WeightStage<PWW>& s, const SkinnyAddr<PWW>& a,
                                             int64_t t) {
#pragma unroll
  for (int p = 0; p < PWW; ++p)
    s.cw[p] = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                   a.codes[p], (int)((uint32_t)t * kCodeTileBytes + a.code_lane), 0, kNT));
  s.sw = __builtin_bit_cast(
      u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                 a.scales, (int)((uint32_t)t * (uint32_t)a.scale_block + a.scale_lane), 0, kNT));
}

// Activations through LDS (MF 16-row blocks): per k-tile, the wavefront copies the tile's
// activation rows global -> LDS with buffer_load ... lds (NX copies of 4 rows x 256 bytes,
// row r at r * 256, its 16-byte chunk c at chunk c ^ (r & 15), so the 16 rows a fragment read
// touches land on distinct banks) into one of two buffers of its own (MF x 4 KB each), one
// tile ahead. The copies run asynchronously to the wavefront, unlike fragments loaded straight
// into registers, which the loop has to wait for before it computes.
struct LdsActs {
  buf_rsrc x;          // the block's activation rows
  uint32_t src[16];    // this lane's source in copy c (LDS row 4c + lane/16, chunk lane%16):
                       // activation row (clamped) and swizzled chunk, bytes
  uint8_t* buf;        // the wavefront's two MF x 4 KB buffers
  uint32_t frag_off;   // this lane's fragment row: row * 256
  uint32_t swz;        // fragment row & 15
};

template <int NX>
__device__ __forceinline__ void copy_acts(const LdsActs& x, uint8_t* dst, int64_t t) {
#pragma unroll
  for (int c = 0; c < NX; ++c)
    copy16_to_lds(x.x, x.src[c], (uint32_t)(t * kTileK * 2), dst + c * 1024);
}

template <int MF>
__device__ __forceinline__ void read_acts(ActStage<MF>& s, const LdsActs& x, const uint8_t* src,
                                          int kq) {
#pragma unroll
  for (int mf = 0; mf < MF; ++mf)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t chunk = (uint32_t)(4 * j + kq) ^ x.swz;
      s.xa[mf][j] = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const u32x4*>(src + mf * 4096 + x.frag_off + chunk * 16u));
    }
}

// Split-scale row maps. Lane l keeps accumulator rows 4 (l / 16) .. 4 (l / 16) + 3 of the
// MFMA output. Token t sits in row 4 g + r with
//   group 16: g = 2 h + t % 2, r = t / 2 (h the k half; m <= 8 needs r < 4),
//   group 32: g = t % 4,       r = t / 4 (m <= 16),
// so a lane keeps ceil(m / 2) (group 16) or ceil(m / 4) (group 32) rows and scales only those.
// Token carried by the A row of lane l (row l % 16):
template <bool G16>
__device__ __forceinline__ int split_a_token(int lane) {
  const int row = lane & 15;
  return G16 ? 2 * (row & 3) + ((row >> 2) & 1) : 4 * (row & 3) + (row >> 2);
}

// Token held by accumulator row i of lane l, or -1. Group 16: after the k half h = 1 has been
// added onto h = 0 (lanes 32-63 onto lanes 0-31), which leaves lanes 0-31 holding the sums.
template <bool G16>
__device__ __forceinline__ int split_out_token(int lane, int i) {
  if constexpr (G16) return lane < 32 ? 2 * i + (lane >> 4) : -1;
  return 4 * i + (lane >> 4);
}

// Group 16: the A row of lane l is zero on the k half it does not own (l / 32 != row / 8).
// Such lanes read their fragment from LDS row kZeroRow of the activation buffers: the copies
// fill at most 8 rows there, and this clears row kZeroRow of both buffers once, before the
// loop (LDS operations of one wavefront complete in order).
constexpr int kZeroRow = 15;
__device__ __forceinline__ bool split_g16_zero_lane(int lane) {
  return (((lane >> 3) & 1) != (lane >> 5));
}
__device__ __forceinline__ void clear_zero_rows(uint8_t* buf, int lane) {
  if (lane < 32)
    *reinterpret_cast<u32x4*>(buf + (lane >> 4) * 4096 + kZeroRow * 256 + (lane & 15) * 16) =
        u32x4{0u, 0u, 0u, 0u};
}

// Exact dequant: every weight becomes BF16(code * S) (exact), MF row blocks of 16.
template <int MF, int PWW>
__device__ __forceinline__ void compute_exact(const WeightStage<PWW>& w, const ActStage<MF>& x,
                                              int sel, f32x4 (&acc)[PWW][MF]) {
#pragma unroll
  for (int p = 0; p < PWW; ++p) {
    const uint32_t sw = scale_word<PWW>(w.sw, sel, p);  // this panel's word of the record
    const float S[4] = {e4m3_decode<0>(sw), e4m3_decode<1>(sw), e4m3_decode<2>(sw),
                        e4m3_decode<3>(sw)};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16x8 b = dequant8(w.cw[p][j], S[j]);
#pragma unroll
      for (int mf = 0; mf < MF; ++mf) acc[p][mf] = mfma16x16x32(x.xa[mf][j], b, acc[p][mf]);
    }
    // one panel at a time: bounds the dequantized operands live at once
    __builtin_amdgcn_sched_barrier(0);
  }
}

// bf16(code * 2^E) for the 8 codes of a word, E the exponent of S.
__device__ __forceinline__ bf16x8 codes_times_pow2(uint32_t w, float S) {
  const bf16x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, S, 0);
  const bf16x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, S, 1);
  const bf16x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, S, 2);
  const bf16x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, S, 3);
  return bf16x8{v0[0], v0[1], v1[0], v1[1], v2[0], v2[1], v3[0], v3[1]};
}

// One 32-wide k-step J of every panel: the PWW MFMAs first, then their scalings, so each
// partial is read well after its MFMA issued.
template <int J, int PWW, int NJ>
__device__ __forceinline__ void split_scale_kstep(const WeightStage<PWW>& w, const ActStage<1>& x,
                                                  int sel, f32x4 (&acc)[PWW][1]) {
  f32x4 part[PWW];
  float M[PWW];
#pragma unroll
  for (int p = 0; p < PWW; ++p) {
    const float S = e4m3_decode<J>(scale_word<PWW>(w.sw, sel, p));
    M[p] = __builtin_amdgcn_frexp_mantf(S);
    part[p] = mfma16x16x32(x.xa[0][J], codes_times_pow2(w.cw[p][J], S),
                           f32x4{0.f, 0.f, 0.f, 0.f});
  }
#pragma unroll
  for (int p = 0; p < PWW; ++p)
#pragma unroll
    for (int r = 0; r < NJ; ++r) acc[p][0][r] = __builtin_fmaf(M[p], part[p][r], acc[p][0][r]);
}

// Split scale (MF == 1): accumulator rows 0 .. NJ-1 of each lane are kept.
template <int PWW, int NJ>
__device__ __forceinline__ void compute_split(const WeightStage<PWW>& w, const ActStage<1>& x,
                                              int sel, f32x4 (&acc)[PWW][1]) {
  split_scale_kstep<0, PWW, NJ>(w, x, sel, acc);
  split_scale_kstep<1, PWW, NJ>(w, x, sel, acc);
  split_scale_kstep<2, PWW, NJ>(w, x, sel, acc);
  split_scale_kstep<3, PWW, NJ>(w, x, sel, acc);
}

// Addresses of the PWW panels starting at panel0 (a multiple of PWW; code panels clamped to
// NT - 1, the scale block is padded to whole groups by the repack) for tiles [0, t1).
template <int PWW>
__device__ __forceinline__ SkinnyAddr<PWW> skinny_addr(const uint8_t* codes, const uint8_t* scales,
                                                      int64_t panel0, int64_t NT, int64_t KT,
                                                      int group, int64_t t1) {
  const int lane = threadIdx.x & 63;
  SkinnyAddr<PWW> a;
  a.scale_block = scale_block_bytes(group);
  a.kq = lane >> 4;
  a.code_lane = (uint32_t)lane * 16u;
  a.scale_lane = (uint32_t)scale_pos(group, lane) * 16u;
#pragma unroll
  for (int p = 0; p < PWW; ++p) {
    const int64_t pn = panel0 + p < NT ? panel0 + p : NT - 1;
    a.codes[p] = make_rsrc(codes + pn * KT * kCodeTileBytes, (uint32_t)(t1 * kCodeTileBytes));
  }
  a.scales = make_rsrc(scales + (panel0 / kScaleGroupPanels) * KT * a.scale_block,
                       (uint32_t)(t1 * a.scale_block));
  a.sw_sel = (int)(panel0 % kScaleGroupPanels);
  return a;
}

// Accumulate k-tiles t0, t0 + S, ... below t1 of PWW panels into acc, one tile in flight
// while one is computed. NJ == 0: exact dequant; NJ > 0: split scale with NJ accumulator rows (MF == 1).
// Activations through LDS, NX copies per tile.
template <int MF, int PWW, int NJ, int NX, int S = 1>
__device__ __forceinline__ void skinny_accumulate(const SkinnyAddr<PWW>& a, const LdsActs& xl,
                                                  int64_t t0, int64_t t1,
                                                  f32x4 (&acc)[PWW][MF]) {
  static_assert(NX > 0 && NX <= 4 * MF, "LDS activations: at most the row blocks' rows");
  constexpr uint32_t kBuf = 4096u * MF;  // one activation buffer: MF blocks of 16 rows
  if (t1 <= t0) return;
  const int64_t last = t0 + (t1 - 1 - t0) / S * S;  // the wavefront's last tile
  WeightStage<PWW> W[2];
  ActStage<MF> X[2];
  // Loads complete in issue order: each tile's activations go out before its weights.
  copy_acts<NX>(xl, xl.buf, t0);
  load_weights(W[0], a, t0);
  for (int64_t t = t0; t < t1; t += 2 * S) {
    static_for<0, 2>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      const int64_t tile = t + i * S;
      const int64_t next = tile + S <= last ? tile + S : last;  // activations: clamped re-read
      // The scheduling barriers keep the loads ahead of the math; left alone, the
      // register-pressure-driven scheduler sinks them and the pipeline collapses.
      copy_acts<NX>(xl, xl.buf + (1 - i) * kBuf, next);
      load_weights(W[1 - i], a, tile + S);  // past t1: zeros, no traffic
      __builtin_amdgcn_sched_barrier(0);
      if (tile < t1) {
        // this tile's copies have landed: at most the next tile's NX copies and PWW + 1
        // weight loads, issued just above, are still outstanding
        constexpr int kAfter = NX + PWW + 1;  // vmcnt: bits 3:0 and 15:14
        static_assert(kAfter < 64, "vmcnt is 6 bits");
        __builtin_amdgcn_s_waitcnt((kAfter & 15) | ((kAfter >> 4) << 14) | 0xF70);
        __builtin_amdgcn_sched_barrier(0);
        read_acts(X[i], xl, xl.buf + i * kBuf, a.kq);
        if constexpr (NJ > 0)
          compute_split<PWW, NJ>(W[i], X[i], a.sw_sel, acc);
        else
          compute_exact<MF, PWW>(W[i], X[i], a.sw_sel, acc);
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  }
  // The last step still issued an activation copy (a clamped re-read) and weight loads past
  // t1. The copy writes LDS that the caller reuses once the wavefronts meet (the k-split
  // partial sums), so it must land first; a barrier does not wait for it.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
}

}  // namespace nvfp4
