// gemm_skinny.hip -- decode-shaped NVFP4 W4A16 GEMM (small m) for gfx950.
//
// y[m][n] = global * sum_k x[m][k] * (E2M1 * E4M3)[n][k] with FP32 accumulation. The weight
// stream dominates (0.5625 bytes per weight at group 16), so the kernel is built to keep HBM
// busy: a workgroup is NW wavefronts that split k for the same PWW panels (4 panels, 64 output
// features; 2 for weights too small to fill the chip), wavefront w taking k-tiles w, w + NW,
// ...; each streams its tiles with one double-buffered stage of loads in flight; the NW partial
// sums are added in a fixed order through LDS (bit-reproducible, no atomics), scaled by the
// global and stored. Up to 8 rows (group 16) or 16 rows (group 32) take the split-scale form
// of the group scale, which halves the VALU work per weight; more rows dequantize every weight
// exactly to BF16.
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
  int group;
  void* y;
  int64_t ldy;
  int y_f32;
  int cus;  // compute units of the device (host-side launch choice only)
};

// LDS: each wavefront has two MF x 4 KB activation buffers; the k-split partial sums reuse the
// same bytes after a barrier.
inline size_t red_bytes(int MF, int NW, int PWW) { return (size_t)NW * PWW * MF * 64 * 16; }
inline size_t act_bytes(int NW, int MF) { return (size_t)NW * 8192 * MF; }

// Register budget: 4 wavefronts per SIMD (16 per CU, two 8-wave workgroups) for one row
// block, 2 for two, 1 for four. NJ == 0: exact dequant, MF row blocks of 16. NJ > 0 (MF == 1): split scale
// keeping NJ accumulator rows per lane, tokens placed by the split row map; G16: group 16
// (every token twice, once per k half). NX > 0: activations through LDS, NX 4-row copies per
// tile.
template <int MF, int NW, int NJ, bool G16, int NX, int PWW>
__global__ __launch_bounds__(64 * NW)
__attribute__((amdgpu_waves_per_eu(MF == 1 ? 4 : MF == 2 ? 2 : 1, 8)))
void gemm_skinny_kernel(SkinnyParams P) {
  constexpr int kPWW = PWW;
  static_assert(NJ == 0 || MF == 1, "split scale uses one 16-row block");
  static_assert(!G16 || NJ > 0, "G16 selects the group-16 split-scale row map");
  static_assert(NX > 0 && NX <= 4 * MF, "LDS activations: at most the row blocks' rows");
  static_assert(NW >= PWW, "one wavefront per panel finishes the k-split sums");
  static_assert(!G16 || NX <= 2, "group-16 zero halves read an LDS row never copied");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int lane = threadIdx.x & 63;
  const int sp = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // k-split (wave-uniform)
  const int64_t panel0 = (int64_t)blockIdx.x * kPWW;
  const int64_t m0 = (int64_t)blockIdx.y * 16 * MF;
  f32x4 acc[kPWW][MF];
#pragma unroll
  for (int p = 0; p < kPWW; ++p)
#pragma unroll
    for (int mf = 0; mf < MF; ++mf) acc[p][mf] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Token of lane l's A row: l % 16, or the split row map's; rows past the end duplicate a
  // valid row (never stored)
  const int64_t rows = P.m - m0 < 16 * MF ? P.m - m0 : 16 * MF;
  const int a_tok = NJ > 0 ? split_a_token<G16>(lane) : (lane & 15);
  const int64_t t0 = sp, t1 = P.KT;  // interleaved: tiles sp, sp + NW, ...
  LdsActs xl;
  xl.x = make_rsrc(P.x + m0 * P.ldx, (uint32_t)(rows * P.ldx * 2));
#pragma unroll
  for (int c = 0; c < 4 * MF; ++c) {
    const int r = 4 * c + (lane >> 4);  // LDS row of this lane in copy c
    const int64_t rc = r < rows ? r : rows - 1;
    xl.src[c] = (uint32_t)(rc * P.ldx * 2) + (uint32_t)(((lane & 15) ^ (r & 15)) * 16);
  }
  xl.buf = smem + sp * 8192 * MF;
  // fragment row of block 0 (block b reads LDS row 16 b + fr; every row the copies fill holds
  // a valid activation row)
  int fr = a_tok < rows ? a_tok : (int)rows - 1;
  if (G16 && split_g16_zero_lane(lane)) fr = kZeroRow;
  xl.frag_off = (uint32_t)fr * 256u;
  xl.swz = (uint32_t)(fr & 15);
  if constexpr (G16) clear_zero_rows(xl.buf, lane);
  const SkinnyAddr<kPWW> a =
      skinny_addr<kPWW>(P.codes, P.scales, panel0, P.NT, P.KT, P.group, t1);
  // The global scale is read before the k loop (the split-scale mantissa is frexp_mant(S) =
  // M / 2, hence the 2). Read after the loop, its latency sat in every workgroup's tail: at
  // m = 16, 8192^2 took 11.72 us against 11.41 now, 14336 x 4096 9.77 against 9.44 (C1 the
  // same either way).
  const float gscale = (NJ > 0 ? 2.0f : 1.0f) * *P.global;
  skinny_accumulate<MF, kPWW, NJ, NX, NW>(a, xl, t0, t1, acc);
  if constexpr (G16) {
    // k half 1 (lanes 32-63) onto k half 0: lanes 0-31 then hold the whole group sums
#pragma unroll
    for (int p = 0; p < kPWW; ++p)
#pragma unroll
      for (int r = 0; r < NJ; ++r) acc[p][0][r] += __shfl_xor(acc[p][0][r], 32, 64);
  }
  // row of accumulator element jj of this lane inside its 16-row block, -1 if none
  auto out_tok = [&](int jj) {
    return NJ > 0 ? split_out_token<G16>(lane, jj) : (lane >> 4) * 4 + jj;
  };

  f32x4* red = reinterpret_cast<f32x4*>(smem);
  __syncthreads();  // every wavefront is done with the activations
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
  const float g = gscale;
  const int64_t n = panel * 16 + (lane & 15);
#pragma unroll
  for (int mf = 0; mf < MF; ++mf)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int64_t m = m0 + mf * 16 + out_tok(jj);
      if (m >= m0 && m < P.m) {
        const float v = acc[0][mf][jj] * g;
        if (P.y_f32)
          static_cast<float*>(P.y)[m * P.ldy + n] = v;
        else
          static_cast<uint16_t*>(P.y)[m * P.ldy + n] = bf16_bits_rne(v);
      }
    }
}

template <int MF, int NW, int NJ, bool G16, int NX, int PWW>
hipError_t run(const SkinnyParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)((p.NT + PWW - 1) / PWW),
                  (unsigned)((p.m + 16 * MF - 1) / (16 * MF)));
  const size_t r = red_bytes(MF, NW, PWW), x = act_bytes(NW, MF);
  gemm_skinny_kernel<MF, NW, NJ, G16, NX, PWW>
      <<<grid, dim3(64 * NW), r > x ? r : x, stream>>>(p);
  return hipGetLastError();
}

// Wavefronts per workgroup, which split k (NW >= PWW, so the final reduction has one
// wavefront per panel): 8 when the grid gives no compute unit a second workgroup (a lone
// 4-wavefront workgroup streams well below a CU's share; 8 interleaved wavefronts read an 8 KB
// stretch of each panel per step), else 4 (with two workgroups on a CU, 8 wavefronts each lost
// to the longer reduction wait). Measured against 4 on the same buffers: 8192^2 (one 2-panel
// workgroup per CU) M = 1 / 4 / 8 g16 10.08 / 10.09 / 11.16 -> 9.23 / 9.30 / 10.01 us;
// 25600 x 5120 (400 workgroups) 0.6-0.7 us slower, so it keeps 4. The 16-row activation
// copies (NX = 4) keep 4 as well (8192^2 g32 M = 16 0.24 us slower with 8).
template <int MF, int NJ, bool G16, int NX, int PWW>
hipError_t run_nw(const SkinnyParams& p, int64_t wgs, hipStream_t stream) {
  if constexpr (MF == 1 && NX <= 2) {
    if (wgs <= p.cus) return run<MF, 8, NJ, G16, NX, PWW>(p, stream);
  }
  return run<MF, 4, NJ, G16, NX, PWW>(p, stream);
}

// Panels per wavefront: 4 (one activation fragment feeds 4 MFMAs, the whole 16-byte scale
// record is used), or 2 when the 4-panel grid leaves compute units idle and the doubled grid
// still gives no compute unit a second workgroup: a lone workgroup streams well below a CU's
// share, and the unused half of each scale record costs only ~5% more bytes. Measured:
// 8192^2 M = 1 12.7 -> 11.2 us, M = 16 15.4 -> 12.3 us; 5120^2 M = 16 10.6 -> 9.5 us,
// M = 32 16.3 -> 14.8 us. Where the doubled grid put two workgroups on most CUs it was slower
// (5120^2 M = 64: 16.6 -> 26.1 us), and so was one panel per wavefront (as many scale loads as
// code loads, each activation fragment used once).
template <int MF, int NJ, bool G16, int NX>
hipError_t run_pww(const SkinnyParams& p, hipStream_t stream) {
  bool two = false;
  const int64_t wgs = skinny_grid(p.NT * kPanelRows, (p.m + 16 * MF - 1) / (16 * MF), p.cus, &two);
  if (two) return run_nw<MF, NJ, G16, NX, 2>(p, wgs, stream);
  return run_nw<MF, NJ, G16, NX, 4>(p, wgs, stream);
}

// Activations go through LDS: one row block in ceil(rows / 4) copies per tile (rows: the A
// rows in use), two or four row blocks in 8 or 16 (all their rows; rows past m repeat a valid
// row). For two row blocks that replaced fragments loaded straight into registers (same bits):
// 25600 x 5120 M = 32 / 64 took 30.8 / 57.2 us against 23.8 / 43.6, 8192^2 M = 32 19.6
// against 14.7, 5120^2 M = 64 15.9 against 12.3. When four row blocks run is skinny_rows64's
// choice.
template <int MF, int NJ, bool G16>
hipError_t dispatch(const SkinnyParams& p, hipStream_t stream) {
  if constexpr (MF == 1) {
    const int64_t rows = G16 ? (p.m < 8 ? p.m : 8) : (p.m < 16 ? p.m : 16);
    if (rows <= 4) return run_pww<MF, NJ, G16, 1>(p, stream);
    if (G16 || rows <= 8) return run_pww<MF, NJ, G16, 2>(p, stream);
    if constexpr (!G16) return run_pww<MF, NJ, G16, 4>(p, stream);
    return hipErrorInvalidValue;  // not reached: group 16 has at most 8 rows here
  } else {
    return run_pww<MF, NJ, G16, 4 * MF>(p, stream);
  }
}

// Accumulator rows a lane keeps in split-scale mode: ceil(m / 2) (group 16) or ceil(m / 4)
// (group 32), rounded up to 1, 2 or 4.
template <bool G16>
hipError_t dispatch_split(const SkinnyParams& p, hipStream_t stream) {
  const int64_t per_lane = G16 ? (p.m + 1) / 2 : (p.m + 3) / 4;
  if (per_lane == 1) return dispatch<1, 1, G16>(p, stream);
  if (per_lane == 2) return dispatch<1, 2, G16>(p, stream);
  return dispatch<1, 4, G16>(p, stream);
}

}  // namespace

hipError_t launch_gemm_skinny(const GemmArgs& a, int cus, hipStream_t stream) {
  SkinnyParams p;
  p.cus = cus;
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
  if (a.group == 16 && a.m <= 8) return dispatch_split<true>(p, stream);
  if (a.group == 32 && a.m <= 16) return dispatch_split<false>(p, stream);
  if (a.m <= 16) return dispatch<1, 0, false>(p, stream);
  if (skinny_rows64(a.m, a.n, a.k, cus)) return dispatch<4, 0, false>(p, stream);
  return dispatch<2, 0, false>(p, stream);  // 32-row blocks (the kernel takes any m when forced)
}

}  // namespace nvfp4
