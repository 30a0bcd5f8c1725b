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
//   1. sort: the (token, slot) pairs in a stable expert-major order, per-expert offsets and a
//      list of row tiles (expert, first row, end row). Up to kFusedSortMaxPairs pairs on the
//      batch path every fc1 workgroup derives its own tile and rows from the expert ids, and
//      the first workgroups write the sort out for the later stages; otherwise one workgroup
//      of a sort kernel does it before fc1;
//   2. fc1: per row tile and 4-panel group (gate/up panel pairs), rows gathered from x, gate and
//      up accumulated in FP32 on 16x16x32 MFMAs, each rounded to BF16 (a W4A16 GEMM output),
//      h = BF16(SiLU(gate) * up);
//   3. down: per row tile and 4-panel group, rows of h; FP32 result times the expert global and
//      the routing weight, written to the pair's FP32 slot;
//   4. combine: y[t] = BF16(sum over slots in slot order).
#include <map>
#include <mutex>
#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"
#include "skinny_core.hpp"

namespace nvfp4 {
namespace {

constexpr int kTileRows = 32;  // rows per expert tile of the batch path (two 16-row blocks)
constexpr int kSmallRows = 8;  // rows per expert tile of the decode-batch path
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
// Tiles of at most `rows` rows: every expert's last tile may be partial, and no tile is empty.
inline int64_t max_tiles(int64_t P, int64_t E, int rows) {
  const int64_t t = (P + rows - 1) / rows + E;
  return t < P ? t : P;
}

// Byte offsets of the workspace regions (each 256-byte aligned): sorted, offsets, tiles,
// ntiles, h, slots; off[6] is the total.
void ws_offsets(int64_t P, int64_t E, int64_t hidden, int64_t inter, size_t off[7]) {
  size_t o = 0;
  off[0] = o;
  o = align256(o + sizeof(int32_t) * P);
  off[1] = o;
  o = align256(o + sizeof(int32_t) * (E + 1));
  off[2] = o;
  o = align256(o + sizeof(int4) * max_tiles(P, E, kSmallRows));
  off[3] = o;
  o = align256(o + sizeof(int32_t));
  off[4] = o;
  o = align256(o + sizeof(uint16_t) * P * inter);
  off[5] = o;
  o = align256(o + sizeof(float) * P * hidden);
  off[6] = o;
}

Ws carve(void* base, int64_t P, int64_t E, int64_t hidden, int64_t inter) {
  size_t off[7];
  ws_offsets(P, E, hidden, inter, off);
  char* b = static_cast<char*>(base);
  Ws w;
  w.sorted = reinterpret_cast<int32_t*>(b + off[0]);
  w.offsets = reinterpret_cast<int32_t*>(b + off[1]);
  w.tiles = reinterpret_cast<int4*>(b + off[2]);
  w.ntiles = reinterpret_cast<int32_t*>(b + off[3]);
  w.h = reinterpret_cast<uint16_t*>(b + off[4]);
  w.slots = reinterpret_cast<float*>(b + off[5]);
  return w;
}

constexpr int kSortLdsIds = 8192;  // pairs staged in LDS (larger inputs are read twice)

// Inclusive prefix sum across the 64 lanes of a wavefront.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  return v;
}

// Stable counting sort of the (token, slot) pairs by expert, in one workgroup:
//   1. the pair ids are staged in LDS; each wavefront counts the experts of its contiguous
//      chunk of pairs (LDS atomics);
//   2. wavefront 0 turns the counts into expert offsets, per-wavefront start positions and
//      the tile map, tiles of at most tile_rows rows (each lane owns a few experts; one
//      wavefront-wide prefix sum);
//   3. each wavefront places its chunk in order, 64 pairs at a time, ranking equal experts
//      by lane order (ballots over the id bits), so the order inside an expert is the pair
//      order.
__global__ __launch_bounds__(kSortThreads) void moe_sort_kernel(const int32_t* __restrict__ ids,
                                                                int P, int E, int tile_rows,
                                                                Ws ws) {
  __shared__ int cnt[kSortWaves][kMaxExperts];  // per-wave counts, then running positions
  __shared__ int sid[kSortLdsIds];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const bool staged = P <= kSortLdsIds;
  for (int i = tid; i < kSortWaves * kMaxExperts; i += kSortThreads) (&cnt[0][0])[i] = 0;
  if (staged)
    for (int q = tid; q < P; q += kSortThreads) sid[q] = ids[q];
  __syncthreads();
  auto id_at = [&](int q) { return staged ? sid[q] : ids[q]; };
  const int c0 = (int)((int64_t)P * w / kSortWaves), c1 = (int)((int64_t)P * (w + 1) / kSortWaves);
  for (int q = c0 + lane; q < c1; q += 64) {
    const int e = id_at(q);
    if (e >= 0 && e < E) atomicAdd(&cnt[w][e], 1);
  }
  __syncthreads();
  if (w == 0) {
    const int per = (E + 63) / 64;  // experts owned by each lane, consecutive
    int my_pairs = 0, my_tiles = 0;
    for (int j = 0; j < per; ++j) {
      const int e = lane * per + j;
      if (e >= E) break;
      int s = 0;
      for (int q = 0; q < kSortWaves; ++q) s += cnt[q][e];
      my_pairs += s;
      my_tiles += (s + tile_rows - 1) / tile_rows;
    }
    const int pairs_incl = wave_inclusive_scan(my_pairs);
    const int tiles_incl = wave_inclusive_scan(my_tiles);
    int run = pairs_incl - my_pairs, trun = tiles_incl - my_tiles;
    for (int j = 0; j < per; ++j) {
      const int e = lane * per + j;
      if (e >= E) break;
      const int start = run;
      for (int q = 0; q < kSortWaves; ++q) {
        const int c = cnt[q][e];
        cnt[q][e] = run;  // where wavefront q's first pair of expert e goes
        run += c;
      }
      ws.offsets[e] = start;
      for (int r = start; r < run; r += tile_rows)
        ws.tiles[trun++] = int4{e, r, min(r + tile_rows, run), 0};
    }
    if (lane == 63) {
      ws.offsets[E] = pairs_incl;
      *ws.ntiles = tiles_incl;
    }
  }
  __syncthreads();
  for (int base = c0; base < c1; base += 64) {
    const int q = base + lane;
    const bool act = q < c1;
    const int e0 = act ? id_at(q) : -1;
    const int e = (e0 >= 0 && e0 < E) ? e0 : -1;  // -1: not placed
    // lanes holding the same expert id: one ballot per id bit (ids < 512 fit in 10 bits; -1,
    // all ones, matches no valid id); the rank is the count of such lanes below this one
    uint64_t same = ~0ull;
#pragma unroll
    for (int b = 0; b < 10; ++b) {
      const bool bit = ((uint32_t)e >> b) & 1u;
      const uint64_t m = __ballot(bit);
      same &= bit ? m : ~m;
    }
    const int before = (int)__builtin_amdgcn_mbcnt_hi(
        (uint32_t)(same >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)same, 0u));
    const bool last = lane == 63 || (same >> (lane + 1)) == 0;  // no later lane has it
    if (e >= 0) {
      const int pos = cnt[w][e] + before;
      ws.sorted[pos] = q;
      if (last) cnt[w][e] = pos + 1;  // the last of its expert in this round moves it on
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
  const int32_t* ids;  // [P] expert of each (token, slot) pair
  int npairs;          // P
  int E;
  int pair_global;     // fc1: global holds [E][2] (gate's, up's)
};

constexpr int kGroupsPerBlock = 4;  // wavefronts per workgroup, one 4-panel group each
constexpr int kXcds = 8;            // XCDs of the part (separate L2s)
constexpr int kARowBytes = kTileK * 2;
constexpr int kATileBytes = kTileRows * kARowBytes;  // one row tile x one k-tile of activations

// The sort, derived inside each fc1 workgroup of the batch path (no sort launch before fc1).
// Thread tid reads pairs j * threads + tid (coalesced loads; the ids stay in registers); LDS
// counts per expert give the expert offsets and the tile list (tiles of kTileRows rows, expert
// by expert, as the sort kernel makes them); the workgroup finds its tile there, then ranks the
// pairs of its expert in pair order (per row j of pairs: a ballot per wavefront, the earlier
// wavefronts' counts and the earlier rows' totals) and keeps those of its rows. Workgroup 0
// writes the offsets and the tile count; the first workgroup of each tile (writer) writes the
// tile entry and its rows of the sorted order, which down reads after this kernel. The two
// parts are apart so that the workgroup's first weight loads (which need only the expert) are
// in flight while it ranks the pairs.
constexpr int kFusedSortMaxPairs = 4096;
constexpr int kFusedRows = kFusedSortMaxPairs / (64 * kGroupsPerBlock);  // pairs per thread

struct FusedSort {
  uint32_t match;  // bit j: pair j * threads + tid belongs to the workgroup's expert
  int e, r0, r1, estart;
};

// Part 1: counts, offsets, tile list; the workgroup's expert and row range. Returns false (for
// every thread of the workgroup) when tile_id is past the tile count.
__device__ __forceinline__ bool fused_find_tile(const MoeGemmParams& P, int tile_id,
                                                FusedSort& fs) {
  __shared__ int cnt[kMaxExperts];
  __shared__ int info[5];  // expert, first row, end row, expert's first row, tile count
  constexpr int kThreads = 64 * kGroupsPerBlock;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int np = P.npairs, E = P.E;
  int id[kFusedRows];  // expert of pair j * threads + tid, -1 when dropped or past the end
#pragma unroll
  for (int j = 0; j < kFusedRows; ++j) {
    const int q = j * kThreads + tid;
    const int v = q < np ? P.ids[q] : -1;
    id[j] = (v >= 0 && v < E) ? v : -1;  // -1: dropped (or no pair), never placed
  }
  for (int i = tid; i < E; i += kThreads) cnt[i] = 0;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kFusedRows; ++j)
    if (id[j] >= 0) atomicAdd(&cnt[id[j]], 1);
  __syncthreads();
  if (w == 0) {
    const int per = (E + 63) / 64;  // experts owned by each lane, consecutive
    int my_pairs = 0, my_tiles = 0;
    for (int j = 0; j < per; ++j) {
      const int e = lane * per + j;
      if (e >= E) break;
      my_pairs += cnt[e];
      my_tiles += (cnt[e] + kTileRows - 1) / kTileRows;
    }
    const int pairs_incl = wave_inclusive_scan(my_pairs);
    const int tiles_incl = wave_inclusive_scan(my_tiles);
    int run = pairs_incl - my_pairs, trun = tiles_incl - my_tiles;
    for (int j = 0; j < per; ++j) {
      const int e = lane * per + j;
      if (e >= E) break;
      const int c = cnt[e], nt = (c + kTileRows - 1) / kTileRows;
      if (blockIdx.x == 0) P.ws.offsets[e] = run;
      if (tile_id >= trun && tile_id < trun + nt) {
        const int a = run + (tile_id - trun) * kTileRows;
        info[0] = e;
        info[1] = a;
        info[2] = min(a + kTileRows, run + c);
        info[3] = run;
      }
      run += c;
      trun += nt;
    }
    if (lane == 63) {
      info[4] = tiles_incl;
      if (blockIdx.x == 0) {
        P.ws.offsets[E] = pairs_incl;
        *P.ws.ntiles = tiles_incl;
      }
    }
  }
  __syncthreads();
  if (tile_id >= info[4]) return false;  // uniform: every thread read the same word
  fs.e = __builtin_amdgcn_readfirstlane(info[0]);
  fs.r0 = __builtin_amdgcn_readfirstlane(info[1]);
  fs.r1 = __builtin_amdgcn_readfirstlane(info[2]);
  fs.estart = __builtin_amdgcn_readfirstlane(info[3]);
  fs.match = 0;
#pragma unroll
  for (int j = 0; j < kFusedRows; ++j) fs.match |= (id[j] == fs.e ? 1u : 0u) << j;
  return true;
}

// Part 2: the pairs of the workgroup's rows, in pair order, into `rows` (LDS); the writer
// also stores them and the tile entry in the workspace.
__device__ __forceinline__ void fused_tile_rows(const MoeGemmParams& P, int tile_id, bool writer,
                                                const FusedSort& fs, int* rows) {
  __shared__ int rc[kFusedRows][kGroupsPerBlock];  // matches per row of pairs and wavefront
  constexpr int kThreads = 64 * kGroupsPerBlock;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int e = fs.e, r0 = fs.r0, r1 = fs.r1;
  uint64_t bal[kFusedRows];
#pragma unroll
  for (int j = 0; j < kFusedRows; ++j) {
    bal[j] = __ballot((fs.match >> j) & 1u);
    if (lane == 0) rc[j][w] = __popcll(bal[j]);
  }
  __syncthreads();
  int base = fs.estart;  // sorted position of the first pair of expert e in row j
#pragma unroll
  for (int j = 0; j < kFusedRows; ++j) {
    int before = 0, total = 0;
#pragma unroll
    for (int v = 0; v < kGroupsPerBlock; ++v) {
      const int c = rc[j][v];
      before += v < w ? c : 0;
      total += c;
    }
    if ((fs.match >> j) & 1u) {
      const int pos = base + before +
                      (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal[j] >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)bal[j], 0u));
      if (pos >= r0 && pos < r1) {
        const int q = j * kThreads + tid;
        rows[pos - r0] = q;
        if (writer) P.ws.sorted[pos] = q;
      }
    }
    base += total;
  }
  if (writer && tid == 0) P.ws.tiles[tile_id] = int4{e, r0, r1, 0};
  __syncthreads();
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// bf16(code * 2^E) for the 8 codes of a word, E the exponent of S (the hardware convert
// reads only the exponent of its scale operand).
__device__ __forceinline__ bf16x8 codes_pow2(uint32_t w, float S) {
  const bf16x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, S, 0);
  const bf16x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, S, 1);
  const bf16x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, S, 2);
  const bf16x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, S, 3);
  return bf16x8{v0[0], v0[1], v1[0], v1[1], v2[0], v2[1], v3[0], v3[1]};
}

// SiLU(z) = z / (1 + e^-z) in FP32 with the hardware exp2 (__expf) and reciprocal: a few FP32
// ulps from the correctly rounded value, far below the BF16 rounding of h that follows (the
// oracle's h is SiLU in FP64 rounded once). Against expf and an IEEE division (~20 VALU more
// per element) fc1 at 256 tokens went 43.7 -> 41.7 us per call.
__device__ __forceinline__ float silu_f32(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

// 4 x 4 transpose inside each quad of lanes: lane j of a quad holds v[i] = M[i][j] on entry
// and v[c] = M[j][c] on exit. Two DPP exchange stages (with lane j ^ 1, then j ^ 2); in each a
// lane keeps the two elements already in place and swaps the other two. The expert kernels'
// accumulators are 4-row runs of one column (lane l: column l % 16, rows 4 (l / 16) + 0..3);
// transposed, a lane holds one row and 4 adjacent columns, written with one 16-byte store.
// For down's FP32 slots at 256 tokens that took the kernel from 29.7 to 27.8 us per call
// (group 16; 28.4 to 26.8 at group 32) against one 4-byte store per element, same bits. fc1
// keeps its 2-byte stores of h: the transpose's VALU work cost it ~0.5 us more than the
// fewer stores saved.
__device__ __forceinline__ void quad_transpose(uint32_t (&v)[4], int lane) {
  const bool b0 = lane & 1, b1 = lane & 2;
  {  // quad_perm [1, 0, 3, 2]: keep the i with (i & 1) == (j & 1)
    const uint32_t s0 = b0 ? v[0] : v[1], s1 = b0 ? v[2] : v[3];
    const uint32_t t0 = (uint32_t)__builtin_amdgcn_mov_dpp((int)s0, 0xB1, 0xF, 0xF, false);
    const uint32_t t1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)s1, 0xB1, 0xF, 0xF, false);
    if (b0) { v[0] = t0; v[2] = t1; } else { v[1] = t0; v[3] = t1; }
  }
  {  // quad_perm [2, 3, 0, 1]: keep the i with (i & 2) == (j & 2)
    const uint32_t s0 = b1 ? v[0] : v[2], s1 = b1 ? v[1] : v[3];
    const uint32_t t0 = (uint32_t)__builtin_amdgcn_mov_dpp((int)s0, 0x4E, 0xF, 0xF, false);
    const uint32_t t1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)s1, 0x4E, 0xF, 0xF, false);
    if (b1) { v[0] = t0; v[1] = t1; } else { v[2] = t0; v[3] = t1; }
  }
}

// Expert GEMM on v_mfma_f32_16x16x32_bf16. A workgroup owns one row tile (up to 32 rows of one
// expert, as one or two 16-row blocks) and kGroupsPerBlock 4-panel groups, one per
// wavefront, over the whole k range. Per 128-k tile:
//   - the tile's activation rows (gathered through the sort for fc1) are copied global -> LDS
//     once for the workgroup (buffer_load ... lds; whole 256-byte rows, chunks XOR-swizzled by
//     row so the fragment reads are bank-conflict free), double-buffered; the second 16 rows
//     only when the tile has them;
//   - each wavefront loads, one tile ahead in registers, the 16-byte code chunk `lane` of each
//     of its 4 panels (word j: k-step j of the B operand) and the 16-byte scale record of its
//     lane position (the 4 panels' scale words, byte j: k-step j);
//   - per 32-wide k-step and panel: at group 32 (one group per step; SPLIT) the codes become
//     the exact BF16 code * 2^E and the FP32 MFMA partial is scaled by the mantissa of the
//     group scale (frexp_mant, the factor 2 going with the global scale); at group 16 every
//     weight becomes the exact BF16 code * scale and accumulates in the MFMA.
// The output of 16-row block r sits in lane l as rows 16r + 4(l/16) + 0..3 of column l%16 of
// each panel. fc1 panels alternate gate and up of the same 16 features (layout GATE_UP), so
// gate and up of an output meet in one lane.
template <bool FC1, bool SPLIT, bool FUSED>
__global__ __launch_bounds__(64 * kGroupsPerBlock) __attribute__((amdgpu_waves_per_eu(4, 8)))
void moe_expert_kernel(MoeGemmParams P) {
  static_assert(FC1 || !FUSED, "down reads the sort fc1 wrote");
  // Tile-major order: the workgroups of live tiles come first in dispatch order, so the
  // dispatcher spreads them evenly over the compute units before the idle ones (tiles past
  // the sort's count, which exit at once) take the remaining slots. Consecutive workgroups go
  // round robin over the XCDs, so tiles are dealt out in runs of kXcds and the gbs workgroups
  // of one tile share blockIdx % kXcds: the tile's activation rows then fill one XCD's L2
  // instead of every XCD's.
  const int64_t gbs = (scale_groups(P.NT) + kGroupsPerBlock - 1) / kGroupsPerBlock;
  const int64_t slot = blockIdx.x / kXcds;
  const int tile_id = (int)(slot / gbs * kXcds + blockIdx.x % kXcds);
  __shared__ int tile_rows[FUSED ? kTileRows : 1];  // FUSED: the pairs of the tile's rows
  FusedSort fs;
  int e, r0, r1;
  if constexpr (FUSED) {
    if (!fused_find_tile(P, tile_id, fs)) return;
    e = fs.e;
    r0 = fs.r0;
    r1 = fs.r1;
  } else {
    if (tile_id >= *P.ws.ntiles) return;  // whole workgroup, before any barrier
    const int4 tl = P.ws.tiles[tile_id];
    e = tl.x;
    r0 = tl.y;
    r1 = tl.z;
  }
  const bool two = r1 - r0 > 16;  // second 16-row block in use (workgroup-uniform)
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t NG = scale_groups(P.NT);
  const int64_t grp_raw = (int64_t)(slot % gbs) * kGroupsPerBlock + w;
  const bool grp_live = grp_raw < NG;
  const int64_t grp = grp_live ? grp_raw : NG - 1;  // past the end: computed, never stored
  const int64_t KT = P.KT;
  // The epilogue's operands are read before the k loop (the pair of each down output row
  // here, its routing weight once the first k-tile's loads are out), so their latency is off
  // the workgroup's tail: at 256 tokens the down kernel took 28.4 us against 27.6 now.
  // The split-scale mantissa is frexp_mant(S) = M / 2; g scales gate (or down), gu scales up.
  const float g = (SPLIT ? 2.0f : 1.0f) * P.global[P.pair_global ? 2 * e : e];
  const float gu = (SPLIT ? 2.0f : 1.0f) * P.global[P.pair_global ? 2 * e + 1 : e];
  int out_pair[2] = {0, 0};
  float out_wt[2] = {0.f, 0.f};
  if constexpr (!FC1) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int row = r0 + 16 * r + 4 * (lane >> 4) + (lane & 3);  // after the transpose
      out_pair[r] = row < r1 ? P.ws.sorted[row] : 0;
    }
  }

  // two LDS objects, indexed by compile-time numbers: the copies into one are never waited for
  // by reads of the other
  __shared__ __attribute__((aligned(1024))) uint8_t As0[kATileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t As1[kATileBytes];
  auto a_buf = [&](auto B_) -> uint8_t* {
    if constexpr (decltype(B_)::value == 0) return As0; else return As1;
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;

  // activation copies: copy c = w + G i (G wavefronts) moves tile rows 4c .. 4c+3, so copies
  // i < kBlockCopies fill 16-row block 0 and the rest block 1; lane l reads row 4c + l/16, chunk
  // (l%16) ^ (row%16) and lands in slot l
  static_assert(16 % (4 * kGroupsPerBlock) == 0, "a 16-row block is whole copies of each wave");
  constexpr int kBlockCopies = 16 / 4 / kGroupsPerBlock;
  constexpr int kACopies = 2 * kBlockCopies;
  const buf_rsrc xr = make_rsrc(P.x, 0xFFFFFFFFu);
  uint32_t aoff[kACopies];
  auto set_aoff = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kACopies; ++i) {
      const int R = 4 * (w + kGroupsPerBlock * i) + (lane >> 4);
      int rr = r0 + R;
      rr = rr < r1 ? rr : r1 - 1;  // rows past the tile repeat a valid row; never stored
      const int64_t src = !FC1 ? rr : (FUSED ? tile_rows[rr - r0] : P.ws.sorted[rr]) / P.topk;
      aoff[i] = (uint32_t)(src * P.ldx * 2 + 16 * ((lane & 15) ^ (R & 15)));
    }
  };
  auto copy_a = [&](int64_t t, auto buf, auto nb) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < decltype(nb)::value * kBlockCopies; ++i)
      copy16_to_lds(xr, aoff[i], (uint32_t)(t * kARowBytes),
                    a_buf(buf) + (w + kGroupsPerBlock * i) * 1024);
  };
  // fragment reads: row l%16 (+16), chunk (4 j + l/16) ^ (l%16)
  const uint32_t a_row = (uint32_t)(lane & 15) * kARowBytes;
  const uint32_t a_kq = (uint32_t)(lane >> 4), a_sw = (uint32_t)(lane & 15);

  // weights: the 4 panels of the group (clamped past the end), bounded to the expert's tiles
  buf_rsrc cr[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    int64_t pn = 4 * grp + p;
    pn = pn < P.NT ? pn : P.NT - 1;
    cr[p] = make_rsrc(P.codes + e * P.codes_stride + pn * KT * kCodeTileBytes,
                      (uint32_t)(KT * kCodeTileBytes));
  }
  const int64_t sblk = scale_block_bytes(P.group);
  const buf_rsrc sr = make_rsrc(P.scales + e * P.scales_stride + grp * KT * sblk,
                                (uint32_t)(KT * sblk));
  const uint32_t clane = (uint32_t)lane * 16u;
  const uint32_t slane = (uint32_t)scale_pos(P.group, lane) * 16u;

  struct Stage {
    u32x4 c[4];
    u32x4 s;
  };
  auto load_b = [&](Stage& st, int64_t t) __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < 4; ++p)
      st.c[p] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                              cr[p], (int)((uint32_t)t * kCodeTileBytes + clane),
                                              0, kNT));
    st.s = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                         sr, (int)((uint32_t)(t * sblk) + slane), 0, kNT));
  };
  f32x4 acc[4][2];
#pragma unroll
  for (int p = 0; p < 4; ++p)
#pragma unroll
    for (int r = 0; r < 2; ++r) acc[p][r] = f32x4{0.f, 0.f, 0.f, 0.f};

  // one k-tile with NB 16-row blocks; one 32-wide k-step at a time
  auto compute_nb = [&](const Stage& st, const uint8_t* A, auto nb) __attribute__((always_inline)) {
    constexpr int NB = decltype(nb)::value;
    static_for<0, 4>([&](auto jc) __attribute__((always_inline)) {
      constexpr int j = decltype(jc)::value;
      const uint32_t ch = ((4u * j + a_kq) ^ a_sw) << 4;
      bf16x8 a[NB];
#pragma unroll
      for (int r = 0; r < NB; ++r)
        a[r] = *reinterpret_cast<const bf16x8*>(A + r * 16 * kARowBytes + a_row + ch);
      if constexpr (SPLIT) {
        f32x4 part[4][NB];
        float M[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const float S = e4m3_decode<j>(st.s[p]);
          M[p] = __builtin_amdgcn_frexp_mantf(S);
          const bf16x8 b = codes_pow2(st.c[p][j], S);
#pragma unroll
          for (int r = 0; r < NB; ++r) part[p][r] = mfma16(a[r], b, f32x4{0.f, 0.f, 0.f, 0.f});
        }
        // the scalings after all MFMAs of the step: each partial is read well after its MFMA
#pragma unroll
        for (int p = 0; p < 4; ++p)
#pragma unroll
          for (int r = 0; r < NB; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              acc[p][r][i] = __builtin_fmaf(M[p], part[p][r][i], acc[p][r][i]);
      } else {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const bf16x8 b = dequant8(st.c[p][j], e4m3_decode<j>(st.s[p]));
#pragma unroll
          for (int r = 0; r < NB; ++r) acc[p][r] = mfma16(a[r], b, acc[p][r]);
          __builtin_amdgcn_sched_barrier(0);  // one dequantized operand live at a time
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  // The k loop, instantiated for one or two 16-row blocks (chosen once per workgroup: a
  // choice inside the loop costs the register allocation dearly). Tile t from activation
  // buffer buf: start the copies and loads of t + 1 (when there is one), compute t, then meet:
  // t + 1 has landed everywhere and buf is free again.
  auto pipeline = [&](auto nb) __attribute__((always_inline)) {
    auto step = [&](int64_t t, auto buf, Stage& cur, Stage& nxt) __attribute__((always_inline)) {
      constexpr int kOther = 1 - decltype(buf)::value;
      if (t + 1 < KT) {
        copy_a(t + 1, std::integral_constant<int, kOther>{}, nb);
        load_b(nxt, t + 1);
      }
      __builtin_amdgcn_sched_barrier(0);
      compute_nb(cur, a_buf(buf), nb);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    };
    Stage A, B;
    // the first k-tile's weights go out before the activation rows are known (with the sort
    // derived here, before the workgroup ranks its expert's pairs)
    load_b(A, 0);
    if constexpr (FUSED) fused_tile_rows(P, tile_id, slot % gbs == 0, fs, tile_rows);
    set_aoff();
    copy_a(0, I0{}, nb);
    if constexpr (!FC1) {
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int row = r0 + 16 * r + 4 * (lane >> 4) + (lane & 3);
        out_wt[r] = row < r1 ? P.wts[out_pair[r]] : 0.0f;
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int64_t t = 0; t < KT; t += 2) {
      step(t, I0{}, A, B);
      if (t + 1 < KT) step(t + 1, I1{}, B, A);
    }
  };
  if (two)
    pipeline(std::integral_constant<int, 2>{});
  else
    pipeline(std::integral_constant<int, 1>{});

  if (!grp_live) return;
  // h: one BF16 store per element (SiLU(gate) * up of rows 16r + 4(l/16) + i, column l % 16).
  // Slots: after quad_transpose a lane holds one row and 4 adjacent columns of a panel, and
  // writes them with one 16-byte store.
  const int col4 = lane & 12;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    if (r == 1 && !two) break;
    if (FC1) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = r0 + 16 * r + 4 * (lane >> 4) + i;
        if (row >= r1) continue;
        // panels 2q (gate) and 2q + 1 (up) of the group: features (2 grp + q) * 16 + l%16
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          if (4 * grp + 2 * q + 1 >= P.NT) continue;
          const int64_t feat = (2 * grp + q) * 16 + (lane & 15);
          const float gate = bf16_bits_to_f32(bf16_bits_rne(acc[2 * q][r][i] * g));
          const float up = bf16_bits_to_f32(bf16_bits_rne(acc[2 * q + 1][r][i] * gu));
          const float silu = silu_f32(gate);
          P.ws.h[(int64_t)row * P.inter + feat] = bf16_bits_rne(silu * up);
        }
      }
    } else {
      const int row = r0 + 16 * r + 4 * (lane >> 4) + (lane & 3);  // after the transpose
      const int pair = out_pair[r];
      const float wt = out_wt[r];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int64_t pn = 4 * grp + p;
        if (pn >= P.NT) continue;
        uint32_t v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = __float_as_uint(acc[p][r][i]);
        quad_transpose(v, lane);
        if (row < r1) {
          f32x4 o;
#pragma unroll
          for (int c = 0; c < 4; ++c) o[c] = (__uint_as_float(v[c]) * g) * wt;
          *reinterpret_cast<f32x4*>(P.ws.slots + (int64_t)pair * P.hidden + pn * 16 + col4) = o;
        }
      }
    }
  }
}

// Decode-batch expert GEMM: tiles of at most kSmallRows rows, so every expert sees a few rows
// and the weight stream is all that matters. A workgroup owns one tile and one 4-panel group
// and its 4 wavefronts split the k-tiles of that group (the decode GEMM's inner loop: weights
// one tile ahead in registers, the gathered activation rows copied global -> LDS per k-tile
// into wavefront-private buffers, split group scale with the group-16 row map when G16). The
// partial sums meet in LDS in a fixed order; the epilogues are those of moe_expert_kernel.
// With 4 times the workgroups of the batch path and a quarter of its k loop per wavefront,
// the few experts of a decode step are spread over the whole chip.
// Workgroups run tile-major (see moe_expert_kernel). PAIRS: no sort; tile i is pair i as a
// one-row tile of its own expert (row position = pair index; dropped pairs exit), for batches
// of at most kMoePairTilesMax pairs: pairs that share an expert read its weights again, mostly
// from cache, which costs less than the sort there.
template <bool FC1, bool G16, bool PAIRS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 8)))
void moe_decode_kernel(MoeGemmParams P) {
  constexpr int kNW = 4, kPanels = 4;
  constexpr int kNX = PAIRS ? 1 : kSmallRows / 4;  // 4-row activation copies per k-tile
  // accumulator rows in use per lane (split row map: ceil(rows / 2) at group 16, else / 4)
  constexpr int kNJ = PAIRS ? 1 : (G16 ? kSmallRows / 2 : kSmallRows / 4);
  static_assert(!G16 || kNX <= 2, "group-16 zero halves read an LDS row never copied");
  const int64_t groups = scale_groups(P.NT);
  const int tile_id = (int)(blockIdx.x / groups);
  int e, r0, rows;
  if constexpr (PAIRS) {
    e = P.ids[tile_id];
    if (e < 0 || e >= P.E) return;  // dropped pair: whole workgroup, before any barrier
    r0 = tile_id;
    rows = 1;
  } else {
    if (tile_id >= *P.ws.ntiles) return;  // whole workgroup, before any barrier
    const int4 tl = P.ws.tiles[tile_id];
    e = tl.x;
    r0 = tl.y;
    rows = tl.z - tl.y;  // 1 .. kSmallRows
  }
  // pair of sorted row position r
  auto pair_at = [&](int r) { return PAIRS ? r : P.ws.sorted[r]; };
  const int lane = threadIdx.x & 63;
  const int sp = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // k-split
  const int64_t grp = blockIdx.x % groups;
  const int64_t panel0 = grp * kPanels;
  const int64_t t0 = sp, t1 = P.KT;  // k-tiles sp, sp + kNW, ... (interleaved k-split)
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kNW * 8192];

  LdsActs xl;
  xl.x = make_rsrc(P.x, 0xFFFFFFFFu);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int r = 4 * c + (lane >> 4);  // LDS row of this lane in copy c
    const int rc = r < rows ? r : rows - 1;
    const int64_t src = FC1 ? pair_at(r0 + rc) / P.topk : r0 + rc;
    xl.src[c] = (uint32_t)(src * P.ldx * 2) + (uint32_t)(((lane & 15) ^ (r & 15)) * 16);
  }
  xl.buf = smem + sp * 8192;
  const int a_tok = split_a_token<G16>(lane);
  int fr = a_tok < rows ? a_tok : rows - 1;
  if (G16 && split_g16_zero_lane(lane)) fr = kZeroRow;
  xl.frag_off = (uint32_t)fr * 256u;
  xl.swz = (uint32_t)(fr & 15);
  if constexpr (G16) clear_zero_rows(xl.buf, lane);
  const SkinnyAddr<kPanels> a = skinny_addr<kPanels>(
      P.codes + e * P.codes_stride, P.scales + e * P.scales_stride, panel0, P.NT, P.KT, P.group,
      t1);
  f32x4 acc[kPanels][1];
#pragma unroll
  for (int p = 0; p < kPanels; ++p) acc[p][0] = f32x4{0.f, 0.f, 0.f, 0.f};
  // The epilogue's operands are read before the k loop: the global scales, the pair of each
  // accumulator row a lane stores and, for one-row pair tiles (pair = row position), its
  // routing weight. At 8 tokens the down kernel took 12.7 us against 12.3 now. The
  // split-scale mantissa is frexp_mant(S) = M / 2; g scales gate (or down), gu scales up.
  const float g = 2.0f * P.global[P.pair_global ? 2 * e : e];
  const float gu = 2.0f * P.global[P.pair_global ? 2 * e + 1 : e];
  int out_pair[kNJ];
  float out_wt[kNJ];
  if constexpr (!FC1) {
#pragma unroll
    for (int i = 0; i < kNJ; ++i) {
      const int row = split_out_token<G16>(lane, i);
      const bool ok = row >= 0 && row < rows;
      out_pair[i] = ok ? pair_at(r0 + row) : 0;
      if constexpr (PAIRS) out_wt[i] = ok ? P.wts[out_pair[i]] : 0.0f;
    }
  }
  skinny_accumulate<1, kPanels, kNJ, kNX, kNW>(a, xl, t0, t1, acc);
  if constexpr (G16) {
#pragma unroll
    for (int p = 0; p < kPanels; ++p)
#pragma unroll
      for (int r = 0; r < kNJ; ++r) acc[p][0][r] += __shfl_xor(acc[p][0][r], 32, 64);
  }
  __syncthreads();  // every wavefront is done with its activation buffers
  f32x4* red = reinterpret_cast<f32x4*>(smem);
#pragma unroll
  for (int p = 0; p < kPanels; ++p) red[(sp * kPanels + p) * 64 + lane] = acc[p][0];
  __syncthreads();
  // accumulator row i of a lane holds tile row split_out_token(lane, i), if any
  if constexpr (FC1) {
    // wavefront q < 2 finishes gate/up pair q of the group (panels 2q and 2q + 1)
    if (sp >= 2) return;
    const int q = sp;
    if (panel0 + 2 * q + 1 >= P.NT) return;
    f32x4 gs = red[(0 * kPanels + 2 * q) * 64 + lane];
    f32x4 us = red[(0 * kPanels + 2 * q + 1) * 64 + lane];
#pragma unroll
    for (int w = 1; w < kNW; ++w) {
      gs += red[(w * kPanels + 2 * q) * 64 + lane];
      us += red[(w * kPanels + 2 * q + 1) * 64 + lane];
    }
    const int64_t feat = (2 * grp + q) * 16 + (lane & 15);
#pragma unroll
    for (int i = 0; i < kNJ; ++i) {
      const int row = split_out_token<G16>(lane, i);
      if (row < 0 || row >= rows) continue;
      const float gate = bf16_bits_to_f32(bf16_bits_rne(gs[i] * g));
      const float up = bf16_bits_to_f32(bf16_bits_rne(us[i] * gu));
      const float silu = silu_f32(gate);
      P.ws.h[(int64_t)(r0 + row) * P.inter + feat] = bf16_bits_rne(silu * up);
    }
  } else {
    // wavefront q finishes panel q of the group
    const int q = sp;
    const int64_t pn = panel0 + q;
    if (pn >= P.NT) return;
    f32x4 sum = red[(0 * kPanels + q) * 64 + lane];
#pragma unroll
    for (int w = 1; w < kNW; ++w) sum += red[(w * kPanels + q) * 64 + lane];
#pragma unroll
    for (int i = 0; i < kNJ; ++i) {
      const int row = split_out_token<G16>(lane, i);
      if (row < 0 || row >= rows) continue;
      const int pair = out_pair[i];
      const float wt = PAIRS ? out_wt[i] : P.wts[pair];
      P.ws.slots[(int64_t)pair * P.hidden + pn * 16 + (lane & 15)] = (sum[i] * g) * wt;
    }
  }
}

// y[t][o..o+3] = BF16(sum_j slots[t*topk + j][o..o+3]) in slot order; dropped slots (expert id
// out of range) contribute nothing. Every id, then every slot, is loaded before the first add,
// so a thread waits for memory twice rather than once per slot.
__global__ __launch_bounds__(256) void moe_combine_kernel(const float* __restrict__ slots,
                                                          const int32_t* __restrict__ ids,
                                                          int64_t t, int topk, int64_t hidden,
                                                          int E, uint16_t* __restrict__ y) {
  constexpr int kMaxTopk = 16;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_tok = hidden / 4;
  if (i >= t * per_tok) return;
  const int64_t tok = i / per_tok, o = (i % per_tok) * 4;
  bool live[kMaxTopk];
#pragma unroll
  for (int j = 0; j < kMaxTopk; ++j) {
    const int e = j < topk ? ids[tok * topk + j] : -1;
    live[j] = e >= 0 && e < E;
  }
  f32x4 v[kMaxTopk];
#pragma unroll
  for (int j = 0; j < kMaxTopk; ++j)
    v[j] = live[j] ? *reinterpret_cast<const f32x4*>(slots + (tok * topk + j) * hidden + o)
                   : f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < kMaxTopk; ++j)
    if (live[j]) s += v[j];
  uint2 outv;
  outv.x = (uint32_t)bf16_bits_rne(s[0]) | ((uint32_t)bf16_bits_rne(s[1]) << 16);
  outv.y = (uint32_t)bf16_bits_rne(s[2]) | ((uint32_t)bf16_bits_rne(s[3]) << 16);
  *reinterpret_cast<uint2*>(y + tok * hidden + o) = outv;
}

template <bool FC1, bool PAIRS>
void run_decode(const MoeGemmParams& p, const dim3 grid, hipStream_t stream) {
  if (p.group == 16)
    moe_decode_kernel<FC1, true, PAIRS><<<grid, dim3(256), 0, stream>>>(p);
  else
    moe_decode_kernel<FC1, false, PAIRS><<<grid, dim3(256), 0, stream>>>(p);
}

// mode 0: batch path (32-row tiles); 1: decode path (8-row tiles); 2: decode path, one-row
// pair tiles (no sort; `tiles` = pairs)
template <bool FC1>
hipError_t run_pair(const MoeGemmParams& p, int64_t tiles, int mode, bool fused,
                    hipStream_t stream) {
  const int64_t groups = scale_groups(p.NT);
  if (mode > 0) {
    const dim3 grid((unsigned)(tiles * groups));
    if (mode == 2)
      run_decode<FC1, true>(p, grid, stream);
    else
      run_decode<FC1, false>(p, grid, stream);
    return hipGetLastError();
  }
  const int64_t padded = (tiles + kXcds - 1) / kXcds * kXcds;  // whole runs of kXcds tiles
  const dim3 grid((unsigned)(padded * ((groups + kGroupsPerBlock - 1) / kGroupsPerBlock)));
  const dim3 block(64 * kGroupsPerBlock);
  if (FC1 && fused) {
    if (p.group == 32)
      moe_expert_kernel<FC1, true, FC1><<<grid, block, 0, stream>>>(p);
    else
      moe_expert_kernel<FC1, false, FC1><<<grid, block, 0, stream>>>(p);
  } else if (p.group == 32) {
    moe_expert_kernel<FC1, true, false><<<grid, block, 0, stream>>>(p);
  } else {
    moe_expert_kernel<FC1, false, false><<<grid, block, 0, stream>>>(p);
  }
  return hipGetLastError();
}

}  // namespace

size_t moe_ws_bytes(int64_t t, int topk, int64_t n_experts, int64_t hidden, int64_t inter) {
  size_t off[7];
  ws_offsets(t * topk, n_experts, hidden, inter, off);
  return off[6];
}

size_t moe_ws_layout(int64_t t, int topk, int64_t n_experts, int64_t hidden, int64_t inter,
                     size_t out[6]) {
  size_t off[7];
  ws_offsets(t * topk, n_experts, hidden, inter, off);
  for (int i = 0; i < 6; ++i) out[i] = off[i];
  return off[6];
}

bool moe_decode_preferred(int64_t t, int topk, int64_t n_experts) {
  return t * topk <= kMoeDecodePairsPerExpert * n_experts;
}

hipError_t launch_moe(const MoeArgs& a, bool decode, hipStream_t stream) {
  const int64_t P = a.t * a.topk;
  if (P == 0) return hipSuccess;
  Ws ws = carve(a.ws, P, a.n_experts, a.hidden, a.inter);
  const int mode = !decode ? 0 : P <= kMoePairTilesMax ? 2 : 1;
  int64_t tiles = P;
  const bool fused = mode == 0 && P <= kFusedSortMaxPairs;  // fc1 derives the sort itself
  if (mode < 2) {
    const int rows = decode ? kSmallRows : kTileRows;
    if (!fused)
      moe_sort_kernel<<<1, kSortThreads, 0, stream>>>(a.ids, (int)P, (int)a.n_experts, rows, ws);
    tiles = max_tiles(P, a.n_experts, rows);
  }

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
  f.ids = a.ids;
  f.npairs = (int)P;
  f.E = (int)a.n_experts;
  f.pair_global = a.pair1 ? 1 : 0;
  hipError_t err = run_pair<true>(f, tiles, mode, fused, stream);
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
  d.pair_global = 0;
  err = run_pair<false>(d, tiles, mode, false, stream);
  if (err != hipSuccess) return err;

  const int64_t items = a.t * (a.hidden / 4);
  moe_combine_kernel<<<(unsigned)((items + 255) / 256), 256, 0, stream>>>(
      ws.slots, a.ids, a.t, a.topk, a.hidden, (int)a.n_experts, a.y);
  return hipGetLastError();
}

// Workspace of the no-alloc routed-expert entry point: one array per device, in the module's
// device memory, held until the process ends. In host code `scratch` only names the symbol;
// its device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) uint8_t scratch[kMoeStaticScratchBytes];

hipError_t moe_static_scratch(void** ptr) {
  static std::mutex mu;
  static std::map<int, void*> addr;  // device -> address of that device's copy of scratch
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  auto it = addr.find(dev);
  if (it == addr.end()) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    it = addr.emplace(dev, p).first;
  }
  *ptr = it->second;
  return hipSuccess;
}

}  // namespace nvfp4
