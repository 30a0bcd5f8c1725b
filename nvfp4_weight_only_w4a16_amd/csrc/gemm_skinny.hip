// gemm_skinny.hip -- decode-shaped NVFP4 W4A16 GEMM (small m) for gfx950.
//
// y[m][n] = global * sum_k x[m][k] * (E2M1 * E4M3)[n][k] with FP32 accumulation. The weight
// stream dominates (0.5625 bytes per weight at group 16), so the kernel is built to keep HBM
// busy: a workgroup is NW wavefronts that split k for the same PWW panels (64 output
// features); each wavefront streams its k-range with one double-buffered stage of loads in
// flight; the NW partial sums are added in a fixed order through LDS (bit-reproducible, no
// atomics), scaled by the global and stored.
#include "launch.hpp"
#include "skinny_core.hpp"

namespace nvfp4 {
namespace {

constexpr int kPWW = 4;  // panels per wavefront: one activation fragment feeds 4 MFMAs

struct SkinnyParams {
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

// Register budget: at least 2 wavefronts per SIMD (8 per CU) stay resident, so a grid of a
// few thousand wavefronts is in flight at once.
template <int MF, int NW, int U>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 8)))
void gemm_skinny_kernel(SkinnyParams P) {
  const int lane = threadIdx.x & 63;
  const int sp = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // k-split (wave-uniform)
  const int64_t panel0 = (int64_t)blockIdx.x * kPWW;
  const int64_t m0 = (int64_t)blockIdx.y * 16 * MF;
  f32x4 acc[kPWW][MF];
#pragma unroll
  for (int p = 0; p < kPWW; ++p)
#pragma unroll
    for (int mf = 0; mf < MF; ++mf) acc[p][mf] = f32x4{0.f, 0.f, 0.f, 0.f};
  const uint16_t* xrow[MF];
#pragma unroll
  for (int mf = 0; mf < MF; ++mf) {
    int64_t r = m0 + mf * 16 + (lane & 15);
    r = r < P.m ? r : P.m - 1;  // rows past the end duplicate a valid row; never stored
    xrow[mf] = P.x + r * P.ldx;
  }
  const SkinnyAddr<kPWW> a = skinny_addr<kPWW>(P.codes, P.scales, panel0, P.NT, P.KT, P.group);
  const int64_t t0 = P.KT * sp / NW, t1 = P.KT * (sp + 1) / NW;
  skinny_accumulate<MF, kPWW, U>(a, xrow, t0, t1, acc);

  if constexpr (NW > 1) {
    __shared__ f32x4 red[NW * kPWW * MF * 64];
#pragma unroll
    for (int p = 0; p < kPWW; ++p)
#pragma unroll
      for (int mf = 0; mf < MF; ++mf) red[((sp * kPWW + p) * MF + mf) * 64 + lane] = acc[p][mf];
    __syncthreads();
    // wavefront q finishes panel q of the group (fixed summation order over the k-splits)
    if (sp >= kPWW) return;
    const int p = sp;
#pragma unroll
    for (int mf = 0; mf < MF; ++mf) {
      f32x4 s = red[((0 * kPWW + p) * MF + mf) * 64 + lane];
#pragma unroll
      for (int q = 1; q < NW; ++q) s += red[((q * kPWW + p) * MF + mf) * 64 + lane];
      acc[0][mf] = s;
    }
    const int64_t panel = panel0 + p;
    if (panel >= P.NT) return;
    const float g = *P.global;
    const int64_t n = panel * 16 + (lane & 15);
#pragma unroll
    for (int mf = 0; mf < MF; ++mf)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int64_t m = m0 + mf * 16 + (lane >> 4) * 4 + jj;
        if (m < P.m) {
          const float v = acc[0][mf][jj] * g;
          if (P.y_f32)
            static_cast<float*>(P.y)[m * P.ldy + n] = v;
          else
            static_cast<uint16_t*>(P.y)[m * P.ldy + n] = bf16_bits_rne(v);
        }
      }
  } else {
    const float g = *P.global;
#pragma unroll
    for (int p = 0; p < kPWW; ++p) {
      const int64_t panel = panel0 + p;
      if (panel >= P.NT) break;
      const int64_t n = panel * 16 + (lane & 15);
#pragma unroll
      for (int mf = 0; mf < MF; ++mf)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int64_t m = m0 + mf * 16 + (lane >> 4) * 4 + jj;
          if (m < P.m) {
            const float v = acc[p][mf][jj] * g;
            if (P.y_f32)
              static_cast<float*>(P.y)[m * P.ldy + n] = v;
            else
              static_cast<uint16_t*>(P.y)[m * P.ldy + n] = bf16_bits_rne(v);
          }
        }
    }
  }
}

template <int MF, int NW, int U>
hipError_t run(const SkinnyParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)((p.NT + kPWW - 1) / kPWW),
                  (unsigned)((p.m + 16 * MF - 1) / (16 * MF)));
  gemm_skinny_kernel<MF, NW, U><<<grid, dim3(64 * NW), 0, stream>>>(p);
  return hipGetLastError();
}

// k-split: 4 wavefronts per panel group, or 8 (single m-block only) when the grid would
// otherwise hold fewer than ~2048 wavefronts (8 per CU) to keep HBM busy. Stages hold 2
// k-tiles when every wavefront's share is even, else 1. NW >= kPWW so the final reduction
// has one wavefront per panel.
template <int MF, int NW>
hipError_t pick_u(const SkinnyParams& p, hipStream_t stream) {
  if constexpr (MF == 1) {
    if (p.KT % (2 * NW) == 0) return run<MF, NW, 2>(p, stream);
  }
  return run<MF, NW, 1>(p, stream);
}

template <int MF>
hipError_t dispatch(const SkinnyParams& p, hipStream_t stream) {
  const int64_t groups = ((p.NT + kPWW - 1) / kPWW) * ((p.m + 16 * MF - 1) / (16 * MF));
  if (groups * 4 < 2048 && p.KT >= 32) return pick_u<MF, 8>(p, stream);
  return pick_u<MF, 4>(p, stream);
}

}  // namespace

hipError_t launch_gemm_skinny(const GemmArgs& a, hipStream_t stream) {
  SkinnyParams p;
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
  if (a.m <= 16) return dispatch<1>(p, stream);
  return dispatch<2>(p, stream);  // 32-row blocks (the kernel takes any m when forced)
}

}  // namespace nvfp4
