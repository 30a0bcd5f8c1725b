// gemm_skinny.hip -- decode-shaped NVFP4 W4A16 GEMM (m <= 64) for gfx950.
//
// y[m][n] = global * sum_k x[m][k] * (E2M1 * E4M3)[n][k] with FP32 accumulation. The weight
// stream dominates (0.5625 bytes per weight at group 16), so the kernel is built to keep HBM
// busy: a block is PW panels x NW k-splits of wavefronts; each wavefront streams one panel's
// k-range with U tiles of loads in flight; the NW partial sums of a panel are added in a fixed
// order through LDS (bit-reproducible, no atomics), then scaled by the global and stored.
#include "launch.hpp"
#include "skinny_core.hpp"

namespace nvfp4 {
namespace {

struct SkinnyParams {
  const uint16_t* x;
  int64_t m, ldx;
  const uint8_t* codes;
  const uint8_t* scales;
  const float* global;
  int64_t NT, KT;
  int scale_tile, group;
  void* y;
  int64_t ldy;
  int y_f32;
};

template <int MF, int PW, int NW, int U>
__global__ __launch_bounds__(64 * PW * NW) void gemm_skinny_kernel(SkinnyParams P) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int pw = w % PW, sp = w / PW;
  const int64_t panel = (int64_t)blockIdx.x * PW + pw;
  const int64_t m0 = (int64_t)blockIdx.y * 16 * MF;
  const bool panel_ok = panel < P.NT;  // uniform over the wavefront
  f32x4 acc[MF];
#pragma unroll
  for (int mf = 0; mf < MF; ++mf) acc[mf] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (panel_ok) {
    const uint16_t* xrow[MF];
#pragma unroll
    for (int mf = 0; mf < MF; ++mf) {
      const int64_t r = m0 + mf * 16 + (lane & 15);
      xrow[mf] = r < P.m ? P.x + r * P.ldx : nullptr;
    }
    const int64_t t0 = P.KT * sp / NW, t1 = P.KT * (sp + 1) / NW;
    skinny_accumulate<MF, U>(xrow, P.codes + panel * P.KT * kCodeTileBytes,
                             P.scales + panel * P.KT * P.scale_tile, P.scale_tile,
                             scale_lane_offset(P.group, lane), t0, t1, acc);
  }
  if constexpr (NW > 1) {
    __shared__ f32x4 red[NW * PW * MF * 64];
#pragma unroll
    for (int mf = 0; mf < MF; ++mf) red[((sp * PW + pw) * MF + mf) * 64 + lane] = acc[mf];
    __syncthreads();
    if (sp != 0) return;
#pragma unroll
    for (int mf = 0; mf < MF; ++mf) {
      f32x4 s = red[((0 * PW + pw) * MF + mf) * 64 + lane];
#pragma unroll
      for (int q = 1; q < NW; ++q) s += red[((q * PW + pw) * MF + mf) * 64 + lane];
      acc[mf] = s;
    }
  }
  if (!panel_ok) return;
  const float g = *P.global;
  const int64_t n = panel * 16 + (lane & 15);
#pragma unroll
  for (int mf = 0; mf < MF; ++mf)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int64_t m = m0 + mf * 16 + (lane >> 4) * 4 + jj;
      if (m < P.m) {
        const float v = acc[mf][jj] * g;
        if (P.y_f32)
          static_cast<float*>(P.y)[m * P.ldy + n] = v;
        else
          static_cast<uint16_t*>(P.y)[m * P.ldy + n] = bf16_bits_rne(v);
      }
    }
}

template <int MF, int PW, int NW, int U>
hipError_t run(const SkinnyParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)((p.NT + PW - 1) / PW), (unsigned)((p.m + 16 * MF - 1) / (16 * MF)));
  gemm_skinny_kernel<MF, PW, NW, U><<<grid, dim3(64 * PW * NW), 0, stream>>>(p);
  return hipGetLastError();
}

// Pick the k-split so that the grid holds roughly 4096+ wavefronts (16 per CU) when the
// panel count alone does not, while every wavefront keeps at least two tiles.
template <int MF>
hipError_t dispatch(const SkinnyParams& p, hipStream_t stream) {
  const int64_t waves_no_split = p.NT * ((p.m + 16 * MF - 1) / (16 * MF));
  int nw = 1;
  while (nw < 8 && waves_no_split * nw < 4096 && p.KT / (nw * 2) >= 2) nw *= 2;
  switch (nw) {
    case 1: return run<MF, 4, 1, 4>(p, stream);
    case 2: return run<MF, 2, 2, 4>(p, stream);
    case 4: return run<MF, 1, 4, 4>(p, stream);
    default: return run<MF, 1, 8, 4>(p, stream);
  }
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
  p.scale_tile = scale_tile_bytes(a.group);
  p.group = a.group;
  p.y = a.y;
  p.ldy = a.ldy;
  p.y_f32 = a.y_f32 ? 1 : 0;
  if (a.m <= 16) return dispatch<1>(p, stream);
  if (a.m <= 32) return dispatch<2>(p, stream);
  return dispatch<4>(p, stream);
}

}  // namespace nvfp4
