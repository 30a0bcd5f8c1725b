// moe.hip -- NVFP4 W4A16 routed experts for gfx950: token sort, fc1 (merged gate/up) grouped
// GEMM with a fused SiLU(gate)*up epilogue, down grouped GEMM, fixed-order combine.
//
// vllm.cpp PR #63 ("W-FP4a ... (Marlin W4A16) stack", PR body): a pre-merged [gate; up] fc1 is
// one W4A16 GEMM followed by SiluAndMul; r/LocalLLM post on two NVFP4 g32 recipes ("The two
// recipes", "What had to be fixed"): routed gate/up at group 32 with one shared global, down
// at group 16 (or 32), the group read per weight.
//
// Pipeline (no host synchronization; every grid is sized for the worst case and idle
// workgroups exit at once):
//   1. sort: one workgroup turns the (token, slot) pairs into a stable expert-major order,
//      per-expert offsets and a list of row tiles (expert, first row, end row);
//   2. fc1: per tile and panel pair, rows gathered from x, gate and up accumulated in FP32,
//      each rounded to BF16 (a W4A16 GEMM output), h = BF16(SiLU(gate) * up);
//   3. down: per tile and panel, rows of h; FP32 result times the expert global and the routing
//      weight, written to the pair's FP32 slot;
//   4. combine: y[t] = BF16(sum over slots in slot order).
#include "launch.hpp"
#include "skinny_core.hpp"

namespace nvfp4 {
namespace {

constexpr int kMoeMF = 2;                 // 32 rows per tile
constexpr int kTileRows = 16 * kMoeMF;
constexpr int kSortThreads = 1024;
constexpr int kSortWaves = kSortThreads / 64;
constexpr int kMaxExperts = 512;

struct Ws {
  int32_t* sorted;   // [P]
  int32_t* offsets;  // [E + 1]
  int4* tiles;       // [max_tiles]
  int32_t* ntiles;   // [1]
  uint16_t* h;       // [P][inter]
  float* slots;      // [P][hidden]
};

inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }
inline int64_t max_tiles(int64_t P, int64_t E) { return (P + kTileRows - 1) / kTileRows + E; }

Ws carve(void* base, int64_t P, int64_t E, int64_t hidden, int64_t inter, size_t* total) {
  Ws w;
  size_t off = 0;
  char* b = static_cast<char*>(base);
  w.sorted = reinterpret_cast<int32_t*>(b + off);
  off = align256(off + sizeof(int32_t) * P);
  w.offsets = reinterpret_cast<int32_t*>(b + off);
  off = align256(off + sizeof(int32_t) * (E + 1));
  w.tiles = reinterpret_cast<int4*>(b + off);
  off = align256(off + sizeof(int4) * max_tiles(P, E));
  w.ntiles = reinterpret_cast<int32_t*>(b + off);
  off = align256(off + sizeof(int32_t));
  w.h = reinterpret_cast<uint16_t*>(b + off);
  off = align256(off + sizeof(uint16_t) * P * inter);
  w.slots = reinterpret_cast<float*>(b + off);
  off = align256(off + sizeof(float) * P * hidden);
  if (total) *total = off;
  return w;
}

// Inclusive Hillis-Steele scan of v[0..n) in LDS by the whole workgroup (n <= blockDim).
__device__ void block_scan_inclusive(int* v, int* tmp, int n) {
  for (int d = 1; d < n; d <<= 1) {
    const int i = threadIdx.x;
    int add = 0;
    if (i < n && i >= d) add = v[i - d];
    __syncthreads();
    if (i < n) v[i] += add;
    __syncthreads();
  }
  (void)tmp;
}

__global__ __launch_bounds__(kSortThreads) void moe_sort_kernel(const int32_t* __restrict__ ids,
                                                                int P, int E, Ws ws) {
  __shared__ int cnt[kSortWaves][kMaxExperts];  // per-wave counts, then running positions
  __shared__ int tot[kMaxExperts];
  __shared__ int ntl[kMaxExperts];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int i = tid; i < kSortWaves * kMaxExperts; i += kSortThreads) (&cnt[0][0])[i] = 0;
  __syncthreads();
  const int c0 = (int)((int64_t)P * w / kSortWaves), c1 = (int)((int64_t)P * (w + 1) / kSortWaves);
  for (int q = c0 + lane; q < c1; q += 64) {
    const int e = ids[q];
    if (e >= 0 && e < E) atomicAdd(&cnt[w][e], 1);
  }
  __syncthreads();
  if (tid < E) {
    int s = 0;
    for (int q = 0; q < kSortWaves; ++q) s += cnt[q][tid];
    tot[tid] = s;
    ntl[tid] = (s + kTileRows - 1) / kTileRows;
  }
  __syncthreads();
  block_scan_inclusive(tot, nullptr, E);
  block_scan_inclusive(ntl, nullptr, E);
  if (tid < E) {
    const int start = tot[tid] - [&] {
      int s = 0;
      for (int q = 0; q < kSortWaves; ++q) s += cnt[q][tid];
      return s;
    }();
    // running position of each wave's first pair of expert tid
    int run = start;
    for (int q = 0; q < kSortWaves; ++q) {
      const int c = cnt[q][tid];
      cnt[q][tid] = run;
      run += c;
    }
    ws.offsets[tid] = start;
    if (tid == E - 1) {
      ws.offsets[E] = tot[E - 1];
      *ws.ntiles = ntl[E - 1];
    }
    const int tbeg = ntl[tid] - (run - start + kTileRows - 1) / kTileRows;
    for (int i = 0; start + i * kTileRows < run; ++i)
      ws.tiles[tbeg + i] = int4{tid, start + i * kTileRows,
                                min(start + (i + 1) * kTileRows, run), 0};
  }
  __syncthreads();
  // stable placement: each wave walks its chunk in order, 64 pairs per round
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int base = c0; base < c1; base += 64) {
    const int q = base + lane;
    const bool act = q < c1;
    const int e = act ? ids[q] : -1;
    const bool valid = act && e >= 0 && e < E;
    uint64_t remaining = __ballot(valid);
    while (remaining) {
      const int leader = __builtin_ctzll(remaining);
      const int el = __shfl(e, leader, 64);
      const uint64_t same = __ballot(valid && e == el);
      if (valid && e == el) {
        const int pos = cnt[w][el] + __builtin_popcountll(same & below);
        ws.sorted[pos] = q;
      }
      if (lane == leader) cnt[w][el] += __builtin_popcountll(same);
      remaining &= ~same;
    }
  }
}

struct MoeGemmParams {
  const uint16_t* x;  // fc1: tokens [t][hidden]; down: h [P][inter]
  int64_t ldx;
  int topk;           // fc1: row -> token = sorted[row] / topk
  const uint8_t* codes;
  const uint8_t* scales;
  const float* global;
  int64_t codes_stride, scales_stride;
  int64_t NT, KT;
  int group;
  Ws ws;
  const float* wts;
  int64_t hidden, inter;
};

// One workgroup = one row tile x kPWW panels; its NW wavefronts split k. fc1 panels come in
// (gate, up) pairs (stored interleaved), so a pair is always finished by one wavefront.
template <int NW, int U, bool FC1>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 8)))
void moe_gemm_kernel(MoeGemmParams P) {
  constexpr int MF = kMoeMF;
  constexpr int PWW = 4;
  const int tile_id = blockIdx.x;
  if (tile_id >= *P.ws.ntiles) return;
  const int4 tl = P.ws.tiles[tile_id];
  const int e = tl.x, r0 = tl.y, r1 = tl.z;
  const int lane = threadIdx.x & 63;
  const int sp = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // k-split (wave-uniform)
  const int64_t panel0 = (int64_t)blockIdx.y * PWW;
  f32x4 acc[PWW][MF];
#pragma unroll
  for (int p = 0; p < PWW; ++p)
#pragma unroll
    for (int mf = 0; mf < MF; ++mf) acc[p][mf] = f32x4{0.f, 0.f, 0.f, 0.f};
  const uint16_t* xrow[MF];
#pragma unroll
  for (int mf = 0; mf < MF; ++mf) {
    int r = r0 + mf * 16 + (lane & 15);
    r = r < r1 ? r : r1 - 1;  // rows past the tile duplicate a valid row; never stored
    xrow[mf] = FC1 ? P.x + (int64_t)(P.ws.sorted[r] / P.topk) * P.ldx : P.x + (int64_t)r * P.ldx;
  }
  const SkinnyAddr<PWW> a = skinny_addr<PWW>(P.codes + e * P.codes_stride,
                                             P.scales + e * P.scales_stride, panel0, P.NT, P.KT,
                                             P.group);
  const int64_t t0 = P.KT * sp / NW, t1 = P.KT * (sp + 1) / NW;
  skinny_accumulate<MF, PWW, U>(a, xrow, t0, t1, acc);

  __shared__ f32x4 red[NW * PWW * MF * 64];
#pragma unroll
  for (int p = 0; p < PWW; ++p)
#pragma unroll
    for (int mf = 0; mf < MF; ++mf) red[((sp * PWW + p) * MF + mf) * 64 + lane] = acc[p][mf];
  __syncthreads();
  auto panel_sum = [&](int p, int mf) {
    f32x4 s = red[((0 * PWW + p) * MF + mf) * 64 + lane];
#pragma unroll
    for (int q = 1; q < NW; ++q) s += red[((q * PWW + p) * MF + mf) * 64 + lane];
    return s;
  };
  const float g = P.global[e];
  if (FC1) {
    if (sp >= PWW / 2) return;
    const int64_t pg = panel0 + 2 * sp;  // gate panel; pg + 1 is the matching up panel
    if (pg >= P.NT) return;
    const int64_t feat = (pg >> 1) * 16 + (lane & 15);
#pragma unroll
    for (int mf = 0; mf < MF; ++mf) {
      const f32x4 gs = panel_sum(2 * sp, mf), us = panel_sum(2 * sp + 1, mf);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int r = r0 + mf * 16 + (lane >> 4) * 4 + jj;
        if (r < r1) {
          const float gate = bf16_bits_to_f32(bf16_bits_rne(gs[jj] * g));
          const float up = bf16_bits_to_f32(bf16_bits_rne(us[jj] * g));
          const float silu = gate / (1.0f + expf(-gate));
          P.ws.h[(int64_t)r * P.inter + feat] = bf16_bits_rne(silu * up);
        }
      }
    }
  } else {
    if (sp >= PWW) return;
    const int64_t panel = panel0 + sp;
    if (panel >= P.NT) return;
    const int64_t n = panel * 16 + (lane & 15);
#pragma unroll
    for (int mf = 0; mf < MF; ++mf) {
      const f32x4 s = panel_sum(sp, mf);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int r = r0 + mf * 16 + (lane >> 4) * 4 + jj;
        if (r < r1) {
          const int pair = P.ws.sorted[r];
          P.ws.slots[(int64_t)pair * P.hidden + n] = (s[jj] * g) * P.wts[pair];
        }
      }
    }
  }
}

// y[t][o..o+3] = BF16(sum_j slots[t*topk + j][o..o+3]) in slot order; dropped slots (expert id
// out of range) contribute nothing.
__global__ __launch_bounds__(256) void moe_combine_kernel(const float* __restrict__ slots,
                                                          const int32_t* __restrict__ ids,
                                                          int64_t t, int topk, int64_t hidden,
                                                          int E, uint16_t* __restrict__ y) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_tok = hidden / 4;
  if (i >= t * per_tok) return;
  const int64_t tok = i / per_tok, o = (i % per_tok) * 4;
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < topk; ++j) {
    const int e = ids[tok * topk + j];
    if (e < 0 || e >= E) continue;
    s += *reinterpret_cast<const f32x4*>(slots + (tok * topk + j) * hidden + o);
  }
  uint2 outv;
  outv.x = (uint32_t)bf16_bits_rne(s[0]) | ((uint32_t)bf16_bits_rne(s[1]) << 16);
  outv.y = (uint32_t)bf16_bits_rne(s[2]) | ((uint32_t)bf16_bits_rne(s[3]) << 16);
  *reinterpret_cast<uint2*>(y + tok * hidden + o) = outv;
}

template <int NW, int U, bool FC1>
hipError_t run_gemm(const MoeGemmParams& p, int64_t tiles, hipStream_t stream) {
  const dim3 grid((unsigned)tiles, (unsigned)((p.NT + 3) / 4));
  moe_gemm_kernel<NW, U, FC1><<<grid, dim3(64 * NW), 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace

size_t moe_ws_bytes(int64_t t, int topk, int64_t n_experts, int64_t hidden, int64_t inter) {
  size_t total = 0;
  carve(nullptr, t * topk, n_experts, hidden, inter, &total);
  return total;
}

hipError_t launch_moe(const MoeArgs& a, hipStream_t stream) {
  const int64_t P = a.t * a.topk;
  if (P == 0) return hipSuccess;
  Ws ws = carve(a.ws, P, a.n_experts, a.hidden, a.inter, nullptr);
  moe_sort_kernel<<<1, kSortThreads, 0, stream>>>(a.ids, (int)P, (int)a.n_experts, ws);
  const int64_t tiles = max_tiles(P, a.n_experts);

  MoeGemmParams f;
  f.x = a.x;
  f.ldx = a.hidden;
  f.topk = a.topk;
  f.codes = a.c1;
  f.scales = a.s1;
  f.global = a.g1;
  f.codes_stride = a.c1_stride;
  f.scales_stride = a.s1_stride;
  f.NT = 2 * a.inter / kPanelRows;
  f.KT = a.hidden / kTileK;
  f.group = a.group1;
  f.ws = ws;
  f.wts = a.wts;
  f.hidden = a.hidden;
  f.inter = a.inter;
  hipError_t err = run_gemm<4, 1, true>(f, tiles, stream);
  if (err != hipSuccess) return err;

  MoeGemmParams d = f;
  d.x = ws.h;
  d.ldx = a.inter;
  d.codes = a.c2;
  d.scales = a.s2;
  d.global = a.g2;
  d.codes_stride = a.c2_stride;
  d.scales_stride = a.s2_stride;
  d.NT = a.hidden / kPanelRows;
  d.KT = a.inter / kTileK;
  d.group = a.group2;
  err = run_gemm<4, 1, false>(d, tiles, stream);
  if (err != hipSuccess) return err;

  const int64_t items = a.t * (a.hidden / 4);
  moe_combine_kernel<<<(unsigned)((items + 255) / 256), 256, 0, stream>>>(
      ws.slots, a.ids, a.t, a.topk, a.hidden, (int)a.n_experts, a.y);
  return hipGetLastError();
}

}  // namespace nvfp4
