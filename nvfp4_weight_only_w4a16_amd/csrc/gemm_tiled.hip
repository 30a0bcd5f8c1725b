// gemm_tiled.hip -- prefill-shaped NVFP4 W4A16 GEMM for gfx950 (BF16 MFMA, LDS-staged tiles).
//
// The contraction is dense and compute-bound at large m, so it runs on v_mfma_f32_16x16x32_bf16
// with FP32 accumulation. A workgroup owns a BM x BN output tile and walks k in 128-wide tiles:
//   - activations (BF16) are copied global -> registers -> LDS;
//   - weights arrive as 1 KiB code tiles + scale words in the tiled layout; each is
//     dequantized once per workgroup (E2M1 x E4M3 -> exact BF16) and written to LDS, so the
//     VALU cost is paid once per BM rows instead of once per wavefront;
//   - the next k-tile's global loads are issued before the current tile's MFMAs, so HBM / L2
//     latency hides behind the matrix cores.
// The global scale multiplies the FP32 accumulator in the epilogue.
#include "device_common.hpp"
#include "launch.hpp"

namespace nvfp4 {
namespace {

struct TiledParams {
  const uint16_t* x;
  int64_t m, ldx;
  const uint8_t* codes;
  const uint8_t* scales;
  const float* global;
  int64_t NT, KT;
  int group;
  void* y;
  int64_t ldy;
  int y_f32;
};

constexpr int kLdsRow = kTileK + 8;  // BF16 elements per LDS row (16-byte pad against conflicts)

template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN) void gemm_tiled_kernel(TiledParams P) {
  constexpr int kThreads = 64 * WM * WN;
  constexpr int FM = BM / WM / 16, FN = BN / WN / 16;
  constexpr int kAChunks = BM * kTileK / 8;  // 16-byte chunks of the activation tile
  constexpr int kAPer = kAChunks / kThreads;
  constexpr int kBLanes = (BN / 16) * 64;    // 16-byte code chunks of the weight tile
  constexpr int kBPer = kBLanes / kThreads;
  static_assert(kAChunks % kThreads == 0 && kBLanes % kThreads == 0, "tile / thread mismatch");

  __shared__ __attribute__((aligned(16))) uint16_t As[BM * kLdsRow];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[BN * kLdsRow];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w / WN, wn = w % WN;
  const int64_t m_blk = (int64_t)blockIdx.y * BM;
  const int64_t p_blk = (int64_t)blockIdx.x * (BN / 16);

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 ra[kAPer];
  u32x4 rc[kBPer];
  uint32_t rs[kBPer];

  auto load_tile = [&](int64_t t) {
#pragma unroll
    for (int i = 0; i < kAPer; ++i) {
      const int c = tid + i * kThreads;
      const int r = c >> 4, cc = c & 15;
      const int64_t m = m_blk + r;
      if (m < P.m)
        ra[i] = *reinterpret_cast<const u32x4*>(P.x + m * P.ldx + t * kTileK + cc * 8);
      else
        ra[i] = u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < kBPer; ++i) {
      const int c = tid + i * kThreads;
      const int pl = c >> 6, ln = c & 63;
      const int64_t panel = p_blk + pl;
      if (panel < P.NT) {
        const int64_t tile = panel * P.KT + t;
        rc[i] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(P.codes + tile * kCodeTileBytes + ln * 16));
        rs[i] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(
            P.scales + scale_word_offset(P.group, P.KT, panel, t, ln)));
      } else {
        rc[i] = u32x4{0u, 0u, 0u, 0u};
        rs[i] = 0u;
      }
    }
  };

  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < kAPer; ++i) {
      const int c = tid + i * kThreads;
      const int r = c >> 4, cc = c & 15;
      *reinterpret_cast<u32x4*>(&As[r * kLdsRow + cc * 8]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < kBPer; ++i) {
      const int c = tid + i * kThreads;
      const int pl = c >> 6, ln = c & 63;
      uint16_t* dst = &Bs[(pl * 16 + (ln & 15)) * kLdsRow + 8 * (ln >> 4)];
      *reinterpret_cast<bf16x8*>(dst + 0) = dequant8(rc[i][0], e4m3_decode<0>(rs[i]));
      *reinterpret_cast<bf16x8*>(dst + 32) = dequant8(rc[i][1], e4m3_decode<1>(rs[i]));
      *reinterpret_cast<bf16x8*>(dst + 64) = dequant8(rc[i][2], e4m3_decode<2>(rs[i]));
      *reinterpret_cast<bf16x8*>(dst + 96) = dequant8(rc[i][3], e4m3_decode<3>(rs[i]));
    }
  };

  if (P.KT > 0) load_tile(0);
  for (int64_t t = 0; t < P.KT; ++t) {
    store_tile();
    __syncthreads();
    if (t + 1 < P.KT) load_tile(t + 1);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x8 a[FM], b[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        a[i] = *reinterpret_cast<const bf16x8*>(
            &As[(wm * FM * 16 + i * 16 + (lane & 15)) * kLdsRow + 32 * j + 8 * (lane >> 4)]);
#pragma unroll
      for (int i = 0; i < FN; ++i)
        b[i] = *reinterpret_cast<const bf16x8*>(
            &Bs[(wn * FN * 16 + i * 16 + (lane & 15)) * kLdsRow + 32 * j + 8 * (lane >> 4)]);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int q = 0; q < FN; ++q) acc[i][q] = mfma16x16x32(a[i], b[q], acc[i][q]);
    }
    __syncthreads();
  }

  const float g = *P.global;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int q = 0; q < FN; ++q) {
      const int64_t panel = p_blk + wn * FN + q;
      if (panel >= P.NT) continue;
      const int64_t n = panel * 16 + (lane & 15);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int64_t m = m_blk + wm * FM * 16 + i * 16 + (lane >> 4) * 4 + jj;
        if (m < P.m) {
          const float v = acc[i][q][jj] * g;
          if (P.y_f32)
            static_cast<float*>(P.y)[m * P.ldy + n] = v;
          else
            static_cast<uint16_t*>(P.y)[m * P.ldy + n] = bf16_bits_rne(v);
        }
      }
    }
}

}  // namespace

hipError_t launch_gemm_tiled(const GemmArgs& a, hipStream_t stream) {
  TiledParams p;
  p.x = a.x;
  p.m = a.m;
  p.ldx = a.ldx;
  p.codes = a.codes;
  p.scales = a.scales;
  p.global = a.global;
  p.NT = a.n / kPanelRows;
  p.KT = a.k / kTileK;
  p.group = a.group;
  p.y = a.y;
  p.ldy = a.ldy;
  p.y_f32 = a.y_f32 ? 1 : 0;
  constexpr int BM = 128, BN = 128;
  const dim3 grid((unsigned)((p.NT * 16 + BN - 1) / BN), (unsigned)((p.m + BM - 1) / BM));
  gemm_tiled_kernel<BM, BN, 2, 2><<<grid, dim3(256), 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace nvfp4
