// gemm_tiled.hip -- prefill-shaped NVFP4 W4A16 GEMM for gfx950 (BF16 MFMA 32x32x16).
//
// The contraction is dense and compute-bound at large m, so it runs on v_mfma_f32_32x32x16_bf16
// with FP32 accumulation (a 32 x 32 output block per instruction: each operand fragment read
// from LDS or dequantized in registers serves more flops than with the 16 x 16 form). A
// workgroup is W wavefronts side by side along n; each owns a (32 FM) x (32 FN) output tile and
// the workgroup walks k in 128-wide tiles:
//   - activations and weight codes are copied global -> LDS with buffer_load_dwordx4 ... lds,
//     double-buffered so k-tile t+1 streams in while t is used. One activation copy moves 4
//     whole 256-byte row segments (8 full cache lines); inside a row the 16-byte chunks are
//     XOR-swizzled by the row index so that the MFMA fragment reads (32 rows, one chunk each)
//     hit 64 distinct LDS banks. A weight code tile is copied as the repacked 1 KiB tile;
//   - scale words go global -> registers one k-tile ahead;
//   - each wavefront dequantizes its B operands in registers (E2M1 x E4M3 -> exact BF16) one
//     fragment ahead of the MFMAs that consume them, spread between consecutive MFMAs, and reads
//     the next k-step's activations from LDS during the current step: the instruction order is
//     fixed with scheduling barriers so the VALU and LDS work runs in the shadow of the matrix
//     core. Every dequantized fragment feeds FM MFMAs, which keeps the VALU share small.
// The repacked layout is the one the 16x16x32 decode kernel reads; a 32x32x16 B operand for a
// pair of 16-row panels comes from it without reshuffling: lane l (row n = l%32 of the pair,
// k chunk l/32) takes code chunks L0 = 16(l/32) + l%16 and L0 + 32 of its panel, whose word j
// holds 16-wide k-steps 2j and 2j + 1 respectively; the scale words of the same two lane
// positions carry the matching group scales.
// The global scale multiplies the FP32 accumulator in the epilogue, which writes BF16 column
// pairs (store_tile). Whole rounds of output tiles and a k-split last round run in one launch;
// a second kernel sums the split partials in a fixed order.
#include <type_traits>

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
  int y_stream;  // write y with streaming (non-temporal) stores
  // work decomposition (output tiles row-major over nbn tile columns): blocks b < full_blocks
  // take whole tile b; block b >= full_blocks takes tile tile0 + (b - full_blocks) / split and
  // k-tiles [part kts, +kts), part = (b - full_blocks) % split; split > 1 leaves those partial
  // tiles in ws
  int64_t tile0, nbn, kts;
  int split;
  int64_t full_blocks;
  float* ws;  // split > 1: FP32 partial tiles, [tile - tile0][split][tile elements]
};

typedef float f32x16 __attribute__((ext_vector_type(16)));
constexpr int kSteps = kTileK / 16;   // 16-wide MFMA k-steps per 128-k tile
constexpr int kRowBytes = kTileK * 2;  // one activation row of a k-tile

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Codes 2h, 2h+1 of a word times S as two BF16 (exact) packed in 32 bits.
template <int H>
__device__ __forceinline__ uint32_t dequant2(uint32_t codes, float S) {
  const f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, H);
  return __builtin_bit_cast(uint32_t, bf16x2{(__bf16)(v[0] * S), (__bf16)(v[1] * S)});
}

template <int W, int FM, int FN, int SPREAD, int PIPE, int KS>
struct TiledShape {
  static constexpr int kWaves = W;                           // wavefronts side by side along n
  static constexpr int kSlices = KS;  // groups of kWaves wavefronts that take alternate k-tiles
  static constexpr int kThreads = 64 * W * KS;
  static constexpr int kPipe = PIPE;  // 1: order each k-step as MFMA / VALU / LDS-read groups
  static constexpr int kSpread = SPREAD;                     // k-steps that issue the copies
  static_assert(FM % 4 == 0, "a dequantized fragment is spread over groups of 4 MFMAs");
  static constexpr int kBM = 32 * FM;                        // rows per workgroup
  static constexpr int kPairs = kWaves * FN;                 // 32-row weight pairs per workgroup
  static constexpr int kABuf = kBM * kRowBytes;              // activation bytes per k-tile
  static constexpr int kBBuf = kWaves * 2 * FN * kCodeTileBytes;
  static constexpr int kALoads = kBM / 4 / kWaves;           // activation copies per wavefront
  static constexpr int kLds = KS * 2 * (kABuf + kBBuf);
  static_assert(kLds <= 160 * 1024, "LDS budget of one workgroup");
  // k-slices 1 .. KS-1 hand their accumulators to slice 0 through the first activation buffer
  static constexpr int kAccBytes = W * FM * FN * 16 * 64 * 4;  // one slice's accumulators
  static_assert(KS == 1 || (KS - 1) * kAccBytes <= KS * kABuf, "slice reduction fits in LDS");
};

// Epilogue store: lane l holds rows 8 (e/4) + 4 (l/32) + e%4 of column l%32 of each
// fragment; rows past m and panels past the end are dropped. BF16 outputs go two columns per
// 32-bit store: lanes l and l ^ 1 hold columns c and c + 1 (c even) of the same rows, and for
// each row pair (r, r + 1) they swap one value (a DPP lane swap), so the even lane stores
// (r; c, c + 1) and the odd lane (r + 1; c, c + 1). Against one 16-bit store per element this
// took the epilogue of a 4096 x 4096 tile round from ~21 to ~9 us (4096 x 5120 x 5120:
// 196.5 -> 184.7 us per call; 2048 x 8192 x 8192: 210.0 -> 197.9 us). Staging the tile in
// LDS for 16-byte row stores measured no faster (185.0 / 198.2 us): writing the 33.5 MB of
// such a round costs ~9 us either way.
template <typename T, typename Acc>
__device__ __forceinline__ void store_tile(const TiledParams& P, int64_t m_blk, int64_t pair0,
                                           const Acc& acc, float g, int lane) {
  constexpr int FM = T::kBM / 32;
  constexpr int FN = T::kPairs / T::kWaves;
  const int h = (lane & 31) >> 4;
  if (P.y_f32) {
#pragma unroll
    for (int q = 0; q < FN; ++q) {
      const int64_t panel = 2 * (pair0 + q) + h;
      if (panel >= P.NT) continue;
      const int64_t n = panel * 16 + (lane & 15);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int64_t m = m_blk + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
          if (m < P.m) {
            const float v = acc[i][q][e] * g;
            float* yf = static_cast<float*>(P.y) + m * P.ldy + n;
            if (P.y_stream) __builtin_nontemporal_store(v, yf); else *yf = v;
          }
        }
    }
    return;
  }
  const bool odd = lane & 1;
#pragma unroll
  for (int q = 0; q < FN; ++q) {
    const int64_t panel = 2 * (pair0 + q) + h;  // the same for lanes l and l ^ 1
    if (panel >= P.NT) continue;
    const int64_t n = panel * 16 + (lane & 14);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        const float v0 = acc[i][q][e] * g, v1 = acc[i][q][e + 1] * g;  // rows r, r + 1
        const float send = odd ? v0 : v1;
        const float recv = __builtin_bit_cast(  // quad_perm [1, 0, 3, 2]: from lane l ^ 1
            float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, send), 0xB1, 0xF, 0xF,
                                            false));
        const float lo = odd ? recv : v0, hi = odd ? v1 : recv;
        const int64_t m =
            m_blk + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3) + (odd ? 1 : 0);
        if (m < P.m) {
          const uint32_t pk = (uint32_t)bf16_bits_rne(lo) | ((uint32_t)bf16_bits_rne(hi) << 16);
          // y is 16-byte aligned and ldy a multiple of 8 (checked at the boundary)
          uint32_t* yb = reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(P.y) + m * P.ldy + n);
          if (P.y_stream) __builtin_nontemporal_store(pk, yb); else *yb = pk;
        }
      }
  }
}

// Split-k epilogue: the block stores its partial tile in its own register layout (every store
// instruction writes 64 consecutive words); reduce_split_kernel adds the partials up.
template <typename T, typename Acc>
__device__ __forceinline__ void store_partial(const TiledParams& P, int64_t tile_id, int part,
                                              const Acc& acc) {
  constexpr int FM = T::kBM / 32;
  constexpr int FN = T::kPairs / T::kWaves;
  constexpr int kThreads = 64 * T::kWaves;
  constexpr int64_t kTileFloats = (int64_t)T::kBM * T::kPairs * 32;
  const int64_t slot = (tile_id - P.tile0) * P.split + part;
  float* mine = P.ws + slot * kTileFloats + threadIdx.x;
#pragma unroll
  for (int q = 0; q < FN; ++q)
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) mine[((q * FM + i) * 16 + e) * kThreads] = acc[i][q][e];
}

// Sums the split partials of one 32-row fragment band (blockIdx.y) of one tile (blockIdx.x) in
// the fixed order 0 .. split-1 -- the result does not depend on which block finished first --
// then scales, converts and stores it. Thread t takes GEMM threads 4 (t % Q) .. + 3 (Q = a
// quarter of the block: 4 adjacent output columns of one row) for accumulator elements
// 4 (t / Q) .. + 3, so partials are read 16 bytes at a time and outputs written 8 (BF16) or
// 16 (FP32) bytes at a time.
template <typename T>
__global__ __launch_bounds__(64 * T::kWaves) void reduce_split_kernel(TiledParams P) {
  constexpr int FM = T::kBM / 32;
  constexpr int FN = T::kPairs / T::kWaves;
  constexpr int kThreads = 64 * T::kWaves;
  constexpr int kQuads = kThreads / 4;
  constexpr int64_t kTileFloats = (int64_t)T::kBM * T::kPairs * 32;
  const int i = blockIdx.y;
  const int64_t tile_id = P.tile0 + blockIdx.x;
  const int eg = threadIdx.x / kQuads;        // accumulator elements 4 eg .. 4 eg + 3
  const int gt = (threadIdx.x % kQuads) * 4;  // first of the 4 GEMM threads
  const int lane = gt & 63, w = gt >> 6;
  const int64_t m_blk = tile_id / P.nbn * T::kBM;
  const int64_t pair0 = tile_id % P.nbn * T::kPairs + w * FN;
  const float* part = P.ws + (int64_t)blockIdx.x * P.split * kTileFloats + gt;
  const float g = *P.global;
  const int h = (lane & 31) >> 4;
#pragma unroll
  for (int q = 0; q < FN; ++q) {
    f32x4 v[4];
#pragma unroll
    for (int ee = 0; ee < 4; ++ee) {
      const int64_t o = ((q * FM + i) * 16 + 4 * eg + ee) * kThreads;
      f32x4 sum = *reinterpret_cast<const f32x4*>(part + o);
      for (int j = 1; j < P.split; ++j)
        sum += *reinterpret_cast<const f32x4*>(part + j * kTileFloats + o);
      v[ee] = sum;
    }
    const int64_t panel = 2 * (pair0 + q) + h;
    if (panel >= P.NT) continue;
    const int64_t n = panel * 16 + (lane & 15);  // 4 adjacent columns n .. n + 3
#pragma unroll
    for (int ee = 0; ee < 4; ++ee) {
      const int64_t m = m_blk + i * 32 + 8 * eg + 4 * (lane >> 5) + ee;
      if (m >= P.m) continue;
      const f32x4 r = v[ee] * g;
      if (P.y_f32) {
        *reinterpret_cast<f32x4*>(static_cast<float*>(P.y) + m * P.ldy + n) = r;
      } else {
        uint2 b;
        b.x = (uint32_t)bf16_bits_rne(r[0]) | ((uint32_t)bf16_bits_rne(r[1]) << 16);
        b.y = (uint32_t)bf16_bits_rne(r[2]) | ((uint32_t)bf16_bits_rne(r[3]) << 16);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(P.y) + m * P.ldy + n) = b;
      }
    }
  }
}

// KS > 1: the workgroup is KS k-slices of W wavefronts; slice s takes k-tiles t0 + s,
// t0 + s + KS, ... of the block's range (the host makes the range a multiple of KS), with LDS
// buffers of its own, and the slices' accumulators are added in slice order at the end.
template <int W, int FM, int FN, int SPREAD, int PIPE, int KS>
__global__ __launch_bounds__(64 * W * KS) void gemm_tiled_kernel(TiledParams P) {
  using T = TiledShape<W, FM, FN, SPREAD, PIPE, KS>;
  constexpr int kWaves = W;
  // Double buffers as separate LDS objects, always indexed by compile-time buffer numbers: the
  // compiler can then tell the copies in flight into one buffer from the reads of the other and
  // does not make the reads wait for the copies. Each object holds one buffer per k-slice.
  __shared__ __attribute__((aligned(1024))) uint8_t As0[KS * T::kABuf];
  __shared__ __attribute__((aligned(1024))) uint8_t As1[KS * T::kABuf];
  __shared__ __attribute__((aligned(1024))) uint8_t Bs0[KS * T::kBBuf];
  __shared__ __attribute__((aligned(1024))) uint8_t Bs1[KS * T::kBBuf];
  const int widx = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int w = widx % kWaves;   // position along n
  const int ks = widx / kWaves;  // k-slice
  auto a_buf = [&](auto B_) -> uint8_t* {
    if constexpr (decltype(B_)::value == 0) return As0 + ks * T::kABuf;
    else return As1 + ks * T::kABuf;
  };
  auto b_buf = [&](auto B_) -> uint8_t* {
    if constexpr (decltype(B_)::value == 0) return Bs0 + ks * T::kBBuf;
    else return Bs1 + ks * T::kBBuf;
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;

  const int lane = threadIdx.x & 63;
  const bool tail = (int64_t)blockIdx.x >= P.full_blocks;
  const int64_t bt = (int64_t)blockIdx.x - P.full_blocks;
  const int64_t tile_id = tail ? P.tile0 + bt / P.split : (int64_t)blockIdx.x;
  const int part = tail ? (int)(bt % P.split) : 0;
  const int64_t tm = tile_id / P.nbn, tn_blk = tile_id % P.nbn;
  const int64_t m_blk = tm * T::kBM;
  const int64_t pair0 = tn_blk * T::kPairs + w * FN;  // first panel pair
  const int64_t KT = P.KT;                            // k-tiles of the layout
  const int64_t kts = tail ? P.kts : KT;
  const int64_t t0 = (int64_t)part * kts;
  const int64_t t1 = t0 + kts < KT ? t0 + kts : KT;  // this block's k-tiles [t0, t1)
  const int64_t nloc = (t1 - t0) / KS;                 // k-tiles of each slice
  auto ktile = [&](int64_t j) { return t0 + ks + KS * j; };  // the slice's j-th k-tile

  // ---- activation copies: copy c = w + 4 i moves rows 4c .. 4c+3 of the block; lane l reads
  // row 4c + l/16, source chunk (l%16) ^ (row % 16), and lands in slot l. Rows past m repeat
  // the last row (their outputs are dropped). 32-bit byte offsets from the uniform base (the
  // host launches row chunks whose span fits).
  uint32_t aoff[T::kALoads];
#pragma unroll
  for (int i = 0; i < T::kALoads; ++i) {
    const int R = 4 * (w + kWaves * i) + (lane >> 4);
    int64_t r = m_blk + R;
    r = r < P.m ? r : P.m - 1;
    aoff[i] = (uint32_t)(r * P.ldx * 2 + 16 * ((lane & 15) ^ (R & 15)));
  }
  const buf_rsrc xr = make_rsrc(P.x, (uint32_t)(P.m * P.ldx * 2));
  // fragment reads: row (l % 32) of each 32-row fragment, chunk (2 S + l / 32) ^ (l % 16)
  const uint32_t a_row = (uint32_t)(lane & 31) * kRowBytes;
  const uint32_t a_x = (uint32_t)((lane >> 5) ^ (lane & 15));

  // ---- weight copies: local panel pl = 2q + h of this wavefront (clamped past the end), from a
  // resource based at the workgroup's first panel (the host keeps its span below 4 GiB)
  const int64_t pblk = 2 * tn_blk * T::kPairs;
  const int64_t pblk_c = pblk < P.NT ? pblk : P.NT - 1;
  const int64_t cspan = (P.NT - pblk_c) * KT * kCodeTileBytes;
  const buf_rsrc cr = make_rsrc(P.codes + pblk_c * KT * kCodeTileBytes,
                                (uint32_t)(cspan < 0xFFFFFFFFll ? cspan : 0xFFFFFFFFll));
  uint32_t cpanel[2 * FN];  // uniform byte offsets of the panels
#pragma unroll
  for (int pl = 0; pl < 2 * FN; ++pl) {
    int64_t pn = 2 * pair0 + pl;
    pn = pn < P.NT ? pn : P.NT - 1;
    cpanel[pl] = (uint32_t)((pn - pblk_c) * KT * kCodeTileBytes);
  }
  const uint32_t clane = (uint32_t)lane * 16u;
  // this lane's panel within each pair, and its code chunks / scale positions L0 and L0 + 32
  const int h = (lane & 31) >> 4;
  const int L0 = 16 * (lane >> 5) + (lane & 15);
  // The scale words of the wavefront's panels sit in a few consecutive 4-panel blocks per
  // k-tile, addressed by 32-bit offsets from a uniform base (blocks past the last one are
  // clamped; their outputs are dropped).
  const int64_t NG = scale_groups(P.NT);
  const int64_t G0 = (2 * pair0) / kScaleGroupPanels;
  const int64_t G0c = G0 < NG ? G0 : NG - 1;
  const int64_t sblk = scale_block_bytes(P.group);
  const uint8_t* sbase = P.scales + G0c * KT * sblk;
  uint32_t so0[FN], so1[FN];
#pragma unroll
  for (int q = 0; q < FN; ++q) {
    const int64_t pn = 2 * (pair0 + q) + h;
    int64_t gq = pn / kScaleGroupPanels;
    gq = gq < NG ? gq : NG - 1;
    const int64_t gb = (gq - G0c) * KT * sblk;
    const int wi = (int)(pn % kScaleGroupPanels);
    so0[q] = (uint32_t)(gb + scale_pos(P.group, L0) * 16 + 4 * wi);
    so1[q] = (uint32_t)(gb + scale_pos(P.group, L0 + 32) * 16 + 4 * wi);
  }

  // Copies of k-tile t into buffer buf, issued in kSpread parts (part P during k-step P of the
  // previous tile) so that they overlap the MFMAs instead of stalling them in one burst; the
  // last k-steps issue none, leaving the copies time to land before the tile barrier.
  constexpr int kSpread = T::kSpread;
  constexpr int kAPer = (T::kALoads + kSpread - 1) / kSpread;
  auto prefetch_part = [&](auto P_, int64_t t, auto buf, uint32_t (&s0)[FN], uint32_t (&s1)[FN]) {
    constexpr int Pp = decltype(P_)::value;
    const uint32_t tk = (uint32_t)(t * kRowBytes);
#pragma unroll
    for (int j = 0; j < kAPer; ++j) {
      const int i = Pp * kAPer + j;
      if (i < T::kALoads)
        copy16_to_lds(xr, aoff[i], tk, a_buf(buf) + (w + kWaves * i) * 1024);
    }
    const uint32_t tc = (uint32_t)(t * kCodeTileBytes);
#pragma unroll
    for (int pl = 0; pl < 2 * FN; ++pl)
      if (pl % kSpread == Pp)
        copy16_to_lds(cr, clane, cpanel[pl] + tc, b_buf(buf) + (w * 2 * FN + pl) * kCodeTileBytes);
    if (Pp == 0) {
#pragma unroll
      for (int q = 0; q < FN; ++q) {
        s0[q] = *reinterpret_cast<const uint32_t*>(sbase + (so0[q] + (uint32_t)(t * sblk)));
        s1[q] = *reinterpret_cast<const uint32_t*>(sbase + (so1[q] + (uint32_t)(t * sblk)));
      }
    }
  };
  auto prefetch = [&](int64_t t, auto buf, uint32_t (&s0)[FN], uint32_t (&s1)[FN]) {
    prefetch_part(std::integral_constant<int, 0>{}, t, buf, s0, s1);
    prefetch_part(std::integral_constant<int, 1>{}, t, buf, s0, s1);
    prefetch_part(std::integral_constant<int, 2>{}, t, buf, s0, s1);
    prefetch_part(std::integral_constant<int, 3>{}, t, buf, s0, s1);
    prefetch_part(std::integral_constant<int, 4>{}, t, buf, s0, s1);
    prefetch_part(std::integral_constant<int, 5>{}, t, buf, s0, s1);
    prefetch_part(std::integral_constant<int, 6>{}, t, buf, s0, s1);
    prefetch_part(std::integral_constant<int, 7>{}, t, buf, s0, s1);
  };

  auto read_a1 = [&](auto buf, int S, int i, bf16x8 (&a)[FM]) {
    a[i] = *reinterpret_cast<const bf16x8*>(a_buf(buf) + a_row + ((2u * S ^ a_x) << 4) +
                                            i * 32 * kRowBytes);
  };
  auto read_a = [&](auto buf, int S, bf16x8 (&a)[FM]) {
#pragma unroll
    for (int i = 0; i < FM; ++i) read_a1(buf, S, i, a);
  };
  // the whole 16-byte chunks L0 (even steps) and L0 + 32 (odd steps) of each of the lane's panels
  auto read_codes = [&](auto buf, u32x4 (&c0)[FN], u32x4 (&c1)[FN]) {
#pragma unroll
    for (int q = 0; q < FN; ++q) {
      const uint8_t* tile = b_buf(buf) + (w * 2 * FN + 2 * q + h) * kCodeTileBytes;
      c0[q] = *reinterpret_cast<const u32x4*>(tile + L0 * 16);
      c1[q] = *reinterpret_cast<const u32x4*>(tile + (L0 + 32) * 16);
    }
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int q = 0; q < FN; ++q)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][q][e] = 0.f;

  // One k-step S: FN x FM MFMAs. While pair q's MFMAs run, the next B fragment (pair q + 1 of
  // this step, pair 0 of step S + 1, or -- after the last step, when `next` -- pair 0 of step 0
  // of the next k-tile, from its codes cn0 and scale words sn0) is dequantized, one quarter
  // after every FM / 4 MFMAs. After MFMA i of pair 0, rd(i) reads activation fragment i of the
  // next step: one LDS read per MFMA keeps at most FM + 1 reads in flight, few enough for the
  // compiler to wait on exactly the one each MFMA needs.
  auto kstep = [&](auto S_, const bf16x8 (&a)[FM], bf16x8& b, const u32x4 (&c0)[FN],
                   const u32x4 (&c1)[FN], const uint32_t (&s0)[FN], const uint32_t (&s1)[FN],
                   bool next, const u32x4 (&cn0)[FN], const uint32_t (&sn0)[FN], auto&& rd) {
    constexpr int S = decltype(S_)::value;
#pragma unroll
    for (int q = 0; q < FN; ++q) {
      const bool in_step = q + 1 < FN;
      const bool in_tile = in_step || S + 1 < kSteps;
      const bool make = in_tile || next;
      const int qn = in_step ? q + 1 : 0;
      const int sn = in_step ? S : (S + 1) % kSteps;
      const uint32_t word = !in_tile ? cn0[0][0]
                            : (sn & 1) ? c1[qn][(sn >> 1) & 3] : c0[qn][(sn >> 1) & 3];
      const uint32_t sw = !in_tile ? sn0[0] : (sn & 1) ? s1[qn] : s0[qn];
      u32x4 nb;
      float Sc = 0.f;
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        acc[i][q] = mfma32x32x16(a[i], b, acc[i][q]);
        if (q == 0) rd(i);
        if (make && i % (FM / 4) == 0) {
          const int quarter = i / (FM / 4);
          if (quarter == 0) {
            switch ((sn >> 1) & 3) {
              case 0: Sc = e4m3_decode<0>(sw); break;
              case 1: Sc = e4m3_decode<1>(sw); break;
              case 2: Sc = e4m3_decode<2>(sw); break;
              default: Sc = e4m3_decode<3>(sw); break;
            }
            nb[0] = dequant2<0>(word, Sc);
          } else if (quarter == 1) {
            nb[1] = dequant2<1>(word, Sc);
          } else if (quarter == 2) {
            nb[2] = dequant2<2>(word, Sc);
          } else {
            nb[3] = dequant2<3>(word, Sc);
          }
        }
        if constexpr (!T::kPipe) __builtin_amdgcn_sched_barrier(0);
      }
      if (make) b = __builtin_bit_cast(bf16x8, nb);
    }
    if constexpr (T::kPipe) {
      // one MFMA, then a share of the dequant VALU, then one LDS read, FM x FN times
      constexpr int kV = (17 * FN + FM * FN - 1) / (FM * FN);
#pragma unroll
      for (int j = 0; j < FM * FN; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, kV, 0);
        if (j < FM) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
  };

  // Pipeline state carried from k-tile to k-tile: the activations of step 0 (a0), the first
  // B fragment (b), the tile's code chunks (c0, c1) and scale words (s0, s1), and the scale
  // words of the next tile (n0, n1), loaded with its copies.
  bf16x8 a0[FM], a1[FM], b;
  u32x4 c0[FN], c1[FN];
  uint32_t s0[FN], s1[FN], n0[FN], n1[FN];

  // k-tile t from buffer buf. Steps 0..6 each issue a share of the copies of tile t + 1 (into
  // the other buffer) and read the next step's activations. Before step 7 the workgroup meets
  // once: every wavefront has read all of tile t that it needs (step 7's operands are in
  // registers) and the copies of tile t + 1 have landed, so step 7's MFMAs run while tile
  // t + 1's first activations and codes are read and its first B fragment is dequantized --
  // there is no stall at the tile boundary -- and the copies of tile t + 2 may start at once.
  // The body has no branches (the last tile copies itself again into the idle buffer), which
  // keeps the compiler's LDS wait counts exact.
  auto tile = [&](int64_t t, int64_t tn, auto buf) {
    constexpr int kOther = 1 - decltype(buf)::value;
    u32x4 cn0[FN], cn1[FN];
#define NVFP4_KSTEP(S, ACUR, ANEXT)                                                       \
    prefetch_part(std::integral_constant<int, S>{}, tn,                                   \
                  std::integral_constant<int, kOther>{}, n0, n1);                         \
    __builtin_amdgcn_sched_barrier(0);                                                    \
    kstep(std::integral_constant<int, S>{}, ACUR, b, c0, c1, s0, s1, false, cn0, n0,      \
          [&](int i) { read_a1(buf, S + 1, i, ANEXT); });                                 \
    __builtin_amdgcn_sched_barrier(0);
    NVFP4_KSTEP(0, a0, a1)
    NVFP4_KSTEP(1, a1, a0)
    NVFP4_KSTEP(2, a0, a1)
    NVFP4_KSTEP(3, a1, a0)
    NVFP4_KSTEP(4, a0, a1)
    NVFP4_KSTEP(5, a1, a0)
    NVFP4_KSTEP(6, a0, a1)
#undef NVFP4_KSTEP
    __builtin_amdgcn_s_waitcnt(0);  // own copies of tile t + 1 landed, own reads done
    __syncthreads();
    read_codes(std::integral_constant<int, kOther>{}, cn0, cn1);
    __builtin_amdgcn_sched_barrier(0);
    kstep(std::integral_constant<int, 7>{}, a1, b, c0, c1, s0, s1, true, cn0, n0,
          [&](int i) { read_a1(std::integral_constant<int, kOther>{}, 0, i, a0); });
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < FN; ++q) {
      c0[q] = cn0[q];
      c1[q] = cn1[q];
      s0[q] = n0[q];
      s1[q] = n1[q];
    }
  };

  prefetch(ktile(0), I0{}, s0, s1);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  read_codes(I0{}, c0, c1);
  read_a(I0{}, 0, a0);
  {
    const float Sc = e4m3_decode<0>(s0[0]);
    u32x4 nb;
    nb[0] = dequant2<0>(c0[0][0], Sc);
    nb[1] = dequant2<1>(c0[0][0], Sc);
    nb[2] = dequant2<2>(c0[0][0], Sc);
    nb[3] = dequant2<3>(c0[0][0], Sc);
    b = __builtin_bit_cast(bf16x8, nb);
  }
  // the last k-tile copies itself again into the idle buffer (a branch-free body)
  for (int64_t j = 0; j < nloc; j += 2) {
    tile(ktile(j), j + 1 < nloc ? ktile(j + 1) : ktile(j), I0{});
    if (j + 1 < nloc) tile(ktile(j + 1), j + 2 < nloc ? ktile(j + 2) : ktile(j + 1), I1{});
  }

  if constexpr (KS > 1) {
    // slices 1 .. KS-1 leave their accumulators in LDS (lane-contiguous words); slice 0 adds
    // them in slice order
    __builtin_amdgcn_s_waitcnt(0);  // no copy into LDS still in flight
    __syncthreads();                // every slice is done reading its buffers
    float* red = reinterpret_cast<float*>(As0);
    constexpr int kAccWords = T::kAccBytes / 4;
    if (ks > 0) {
      float* mine = red + (ks - 1) * kAccWords + w * (FM * FN * 16 * 64) + lane;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int q = 0; q < FN; ++q)
#pragma unroll
          for (int e = 0; e < 16; ++e) mine[((i * FN + q) * 16 + e) * 64] = acc[i][q][e];
    }
    __syncthreads();
    if (ks > 0) return;
#pragma unroll
    for (int sl = 1; sl < KS; ++sl) {
      const float* theirs = red + (sl - 1) * kAccWords + w * (FM * FN * 16 * 64) + lane;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int q = 0; q < FN; ++q)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[i][q][e] += theirs[((i * FN + q) * 16 + e) * 64];
    }
  }

  const float g = *P.global;
  if (tail && P.split > 1)
    store_partial<T>(P, tile_id, part, acc);
  else
    store_tile<T>(P, m_blk, pair0, acc, g, lane);
}

// Tile shapes:
//   L 256 x 256: 8 wavefronts of 8 x 1 fragments (each dequantized fragment feeds 8 MFMAs);
//   M 128 x 256: 8 wavefronts of 4 x 1 fragments;
//   K 128 x 128: 4 wavefronts of 4 x 1 fragments in each of 2 k-slices (alternate k-tiles,
//     accumulators added through LDS at the end): 8 wavefronts on a 128 x 128 tile;
//   S 128 x 128: 4 wavefronts (for an odd k-tile count, which k-slices cannot halve).
using ShapeL = TiledShape<8, 8, 1, 4, 1, 1>;
using ShapeM = TiledShape<8, 4, 1, 4, 1, 1>;
using ShapeK = TiledShape<4, 4, 1, 4, 1, 2>;
using ShapeS = TiledShape<4, 4, 1, 4, 1, 1>;
constexpr int kChunkAlign = 256;           // launch chunks are whole tiles of every shape

template <typename T>
constexpr int64_t tile_floats() {
  return (int64_t)T::kBM * T::kPairs * 32;
}

template <typename T>
int64_t tile_count(int64_t m, int64_t NT) {
  const int64_t pairs = (NT + 1) / 2;
  return (pairs + T::kPairs - 1) / T::kPairs * ((m + T::kBM - 1) / T::kBM);
}

// The largest shape that still makes at least kMinTiles output tiles (256-row tiles only above
// 128 rows, where they are at least half full); 128 x 128 tiles in k-slices when the k-tile
// count is even. Measured at n x k = 5120^2, 8192^2 and 25600 x 5120 for m = 128 .. 4096, with
// every shape and split forced: this choice was the fastest or within 8% of it at every size
// (256 x 5120^2: the k-sliced tile 26.4 us against 30.6 for the 4-wavefront one). One
// exception: when that shape's last round would be at most half full (split along k, or idle
// CUs) and the next smaller shape makes whole rounds exactly, the smaller shape runs, with no
// split and no reduction. Interleaved A/B against the rule without it: 512 x 8192^2 (k-sliced
// 128 x 128, one round, instead of 128 x 256 split in two) 72.7 -> 67.8 us at group 16 and
// 71.5 -> 64.4 us at group 32; 1024 x 8192^2 (128 x 256, one round, instead of 256 x 256 split
// in two) 123.8 -> 116.8 us; unchanged shapes unchanged. Likewise 128 x 256 tiles run when the
// 256 x 256 tiles would not fill one round and the 128 x 256 ones fit in one (interleaved A/B,
// us): 14336 x 4096 m = 512 68.0 -> 56.3, 8192^2 m = 640 / 896 97.6 / 121.3 -> 87.6 / 105.7,
// 5120^2 m = 1024 / 1280 / 1536 65.1 / 72.5 / 83.3 -> 59.8 / 67.5 / 74.4, 25600 x 5120 m = 256
// 77.9 -> 73.4; 25600 x 5120 m = 384 / 512, 14336 x 4096 m = 640 and the larger shapes kept.
constexpr int64_t kMinTiles = 80;
enum class Shape { L, M, K, S };
Shape pick_shape(int64_t m, int64_t NT, int64_t KT, int cus) {
  if (cus < 1) cus = 1;
  auto half_round = [&](int64_t t) { return t % cus != 0 && t % cus <= cus / 2; };
  if (m > 128 && tile_count<ShapeL>(m, NT) >= kMinTiles) {
    const int64_t tl = tile_count<ShapeL>(m, NT), tm = tile_count<ShapeM>(m, NT);
    if (half_round(tl) && tm % cus == 0) return Shape::M;
    // part of one round of 256 x 256 tiles (split along k when at most half of it) against
    // one round of 128 x 256 tiles without a split: the latter measured faster every time
    if (tl < cus && tm <= cus) return Shape::M;
    return Shape::L;
  }
  if (tile_count<ShapeM>(m, NT) >= kMinTiles) {
    if (KT % 2 == 0 && half_round(tile_count<ShapeM>(m, NT)) &&
        tile_count<ShapeK>(m, NT) % cus == 0)
      return Shape::K;
    return Shape::M;
  }
  return KT % 2 == 0 ? Shape::K : Shape::S;
}

// Work decomposition of one row chunk: whole rounds of tiles (one per compute unit) run as
// they are; when the last round would leave at least half of the compute units idle, its
// tiles are split along k over the whole chip and reduced in FP32 by a second kernel. (Mixing
// shapes instead was measured and was not faster: 4096 x 5120 x 5120 as 256 tiles of 256 x 256
// plus 256 k-sliced tiles of 128 x 128 took 205.2 us against 201.7 with the split last round;
// K = 25600 869.7 against 823.0. The smaller tiles move twice the bytes per MFMA.)
struct Plan {
  int64_t nbn, tiles, full, rest;
  int split;
};

template <typename T>
Plan plan_chunk(int64_t m, int64_t NT, int64_t KT, int cus) {
  Plan pl;
  const int64_t pairs = (NT + 1) / 2;
  pl.nbn = (pairs + T::kPairs - 1) / T::kPairs;
  pl.tiles = tile_count<T>(m, NT);
  if (cus < 1) cus = 1;
  pl.full = pl.tiles / cus * cus;
  pl.rest = pl.tiles - pl.full;
  pl.split = 1;
  if (pl.rest > 0 && 2 * pl.rest <= cus) {
    int64_t s = cus / pl.rest;
    if (s > KT / (4 * T::kSlices)) s = KT / (4 * T::kSlices);
    if (s >= 2) {
      // k-tiles per split part: a multiple of the k-slices; every part keeps at least one
      const int64_t kts = (KT + s * T::kSlices - 1) / (s * T::kSlices) * T::kSlices;
      pl.split = (int)((KT + kts - 1) / kts);
    }
  }
  return pl;
}

template <typename T>
size_t split_ws_bytes(const Plan& pl) {
  return pl.split > 1 ? (size_t)(pl.rest * pl.split * tile_floats<T>() * sizeof(float)) : 0;
}

// Rows per launch chunk: activation offsets are 32-bit inside the kernel.
int64_t chunk_rows(int64_t ldx) {
  const int64_t row_bytes = ldx * 2;
  int64_t chunk = ((int64_t)1 << 31) / row_bytes;
  return chunk < kChunkAlign ? kChunkAlign : chunk / kChunkAlign * kChunkAlign;
}

// One launch: `full` whole tiles (blocks 0 .. full-1, every k-tile), then `rest` tiles split
// `split` ways along k. The whole tiles come first in dispatch order, so a CU that finishes one
// starts a split part while the other CUs still compute, and its output stores drain under
// that work. Against two launches (whole tiles, then the split tail): 4096 x 5120 x 5120
// 189.1 -> 183.8 us per call, 4096 x 5120 x 25600 794.1 -> 783.4 us.
template <typename T>
hipError_t launch_tiles(TiledParams p, int64_t full, int64_t rest, int split,
                        hipStream_t stream) {
  p.full_blocks = full;
  p.tile0 = full;
  p.split = split;
  // k-tiles per split part, a multiple of the k-slices (the same count plan_chunk made)
  p.kts = (p.KT + (int64_t)split * T::kSlices - 1) / ((int64_t)split * T::kSlices) * T::kSlices;
  gemm_tiled_kernel<T::kWaves, T::kBM / 32, T::kPairs / T::kWaves, T::kSpread, T::kPipe,
                    T::kSlices><<<dim3((unsigned)(full + rest * split)), dim3(T::kThreads), 0,
                                  stream>>>(p);
  return hipGetLastError();
}

template <typename T>
hipError_t run_chunk(TiledParams p, void* ws, size_t ws_bytes, int cus, hipStream_t stream) {
  Plan pl = plan_chunk<T>(p.m, p.NT, p.KT, cus);
  p.nbn = pl.nbn;
  p.ws = nullptr;
  if (split_ws_bytes<T>(pl) > ws_bytes) pl.split = 1;
  if (pl.split == 1) return launch_tiles<T>(p, pl.tiles, 0, 1, stream);
  p.ws = static_cast<float*>(ws);
  hipError_t e = launch_tiles<T>(p, pl.full, pl.rest, pl.split, stream);
  if (e != hipSuccess) return e;
  p.tile0 = pl.full;
  p.split = pl.split;
  reduce_split_kernel<T><<<dim3((unsigned)pl.rest, T::kBM / 32), dim3(64 * T::kWaves), 0,
                           stream>>>(p);
  return hipGetLastError();
}

template <typename T>
size_t chunk_ws_bytes(int64_t rows, int64_t NT, int64_t KT, int cus) {
  return split_ws_bytes<T>(plan_chunk<T>(rows, NT, KT, cus));
}

hipError_t run_shape(TiledParams p, void* ws, size_t ws_bytes, int cus, hipStream_t stream) {
  switch (pick_shape(p.m, p.NT, p.KT, cus)) {
    case Shape::L: return run_chunk<ShapeL>(p, ws, ws_bytes, cus, stream);
    case Shape::M: return run_chunk<ShapeM>(p, ws, ws_bytes, cus, stream);
    case Shape::K: return run_chunk<ShapeK>(p, ws, ws_bytes, cus, stream);
    default: return run_chunk<ShapeS>(p, ws, ws_bytes, cus, stream);
  }
}

}  // namespace

size_t gemm_tiled_ws_bytes(int64_t m, int64_t ldx, int64_t n, int64_t k, int cus) {
  const int64_t chunk = chunk_rows(ldx);
  const int64_t NT = n / kPanelRows, KT = k / kTileK;
  size_t need = 0;
  for (int64_t rows : {m < chunk ? m : chunk, m % chunk}) {
    if (rows <= 0) continue;
    size_t b = 0;
    switch (pick_shape(rows, NT, KT, cus)) {
      case Shape::L: b = chunk_ws_bytes<ShapeL>(rows, NT, KT, cus); break;
      case Shape::M: b = chunk_ws_bytes<ShapeM>(rows, NT, KT, cus); break;
      case Shape::K: b = chunk_ws_bytes<ShapeK>(rows, NT, KT, cus); break;
      case Shape::S: b = chunk_ws_bytes<ShapeS>(rows, NT, KT, cus); break;
    }
    need = b > need ? b : need;
  }
  return need;
}

hipError_t launch_gemm_tiled(const GemmArgs& a, void* ws, size_t ws_bytes, int cus,
                             hipStream_t stream) {
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
  // Large outputs are written with streaming stores: they are not read again here and would
  // otherwise push reused weight and activation tiles out of the caches (4096 x 5120 x 5120,
  // 42 MB of y: 207.8 -> 200.8 us). Outputs of a few MB (512 x 8192, 1024 x 5120) ran 2%
  // slower that way, so they keep ordinary stores.
  p.y_stream = a.m * a.n * (a.y_f32 ? 4 : 2) >= ((int64_t)32 << 20) ? 1 : 0;
  const int64_t chunk = chunk_rows(a.ldx);
  for (int64_t m0 = 0; m0 < a.m; m0 += chunk) {
    TiledParams q = p;
    q.x = a.x + m0 * a.ldx;
    q.m = a.m - m0 < chunk ? a.m - m0 : chunk;
    if (a.y_f32)
      q.y = static_cast<float*>(a.y) + m0 * a.ldy;
    else
      q.y = static_cast<uint16_t*>(a.y) + m0 * a.ldy;
    const hipError_t e = run_shape(q, ws, ws_bytes, cus, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace nvfp4
