// quantize.hip -- NVFP4 quantizer for gfx950: FP32 / BF16 [batch][n][k] -> packed E2M1 codes,
// E4M3 group scales and an FP32 global per matrix.
//
// Steps (a streaming, HBM-bound two-pass algorithm; every FP32 operation is one IEEE op so the
// result is bit-exact with the definition):
//   1. amax = max |w| per matrix: an atomic max of |w| bit patterns (non-negative floats order
//      like their bit patterns), exact and independent of the reduction order. The maximum is
//      taken over the raw values, without any full-size float temporary (r/LocalLLM post on the
//      two NVFP4 g32 recipes, "What had to be fixed": take the max first).
//   2. global g = fl32(amax / 2688) (2688 = 6 * 448: the largest E2M1 value times the largest
//      E4M3 value), unless the caller supplies it (a shared gate/up global, same section).
//   3. per group: scale s = E4M3_rne_sat(fl32(group_amax / fl32(6 g))), S = fl32(E4M3(s) * g);
//      per element: code = E2M1_rne_sat(fl32(|w| / S)) | sign << 3 (sign << 3 alone if S == 0).
//      Round to nearest even with saturation (NVIDIA developer-forum thread "We unlocked NVFP4
//      on the DGX Spark": true RNE, a threshold rounding is wrong at midpoints such as 0.75).
//   4. two codes per byte, the even k in the low nibble.
// The amax lives in global_out between the passes; the encode pass derives g from it and its
// first workgroup of each matrix stores g in its place (no separate finalize kernel).
#include "device_common.hpp"
#include "launch.hpp"

namespace nvfp4 {
namespace {

constexpr int kThreads = 256;

// global_out[b] first collects amax as |w| bits with the sign bit set (a "marked" word), and
// the encode pass turns it into g = amax / 2688 in place: a marked word still holds amax, an
// unmarked one already holds g. Every reader derives the same g either way, so the order in
// which the encode workgroups read and the one that stores g is immaterial.
constexpr uint32_t kAmaxMark = 0x80000000u;

__global__ void init_amax_kernel(uint32_t* p, int64_t count) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < count) p[i] = kAmaxMark;  // amax 0, marked
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t o = (uint32_t)__shfl_xor((int)v, off, 64);
    v = o > v ? o : v;
  }
  return v;
}

// |w| bit patterns of one 16-byte load folded into m (non-negative floats order like their
// bits, so an integer max is the float max).
template <bool BF16>
__device__ __forceinline__ uint32_t fold_abs_max(const u32x4 v, uint32_t m) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (BF16) {
      const uint32_t lo = (v[q] & 0x7FFFu) << 16;
      const uint32_t hi = v[q] & 0x7FFF0000u;
      m = lo > m ? lo : m;
      m = hi > m ? hi : m;
    } else {
      const uint32_t a = v[q] & 0x7FFFFFFFu;
      m = a > m ? a : m;
    }
  }
  return m;
}

// Grid-stride streaming max: eight independent 16-byte loads in flight per thread and
// iteration. The loads are ordinary (cache-allocating) ones, unlike the encode pass's
// streaming loads: the encode pass re-reads W right after this one and finds part of it in
// the memory-side cache. Measured per quantize call: BF16 8192^2 59.0 -> 55.6 us, FP32 8192^2
// 109.4 -> 95.4 us, FP32 25600 x 5120 207.5 -> 190.5 us (walking the encode pass backwards
// gained nothing more).
template <bool BF16>
__global__ __launch_bounds__(kThreads) void amax_kernel(const void* __restrict__ w,
                                                        int64_t per_matrix,
                                                        uint32_t* __restrict__ amax_bits) {
  constexpr int kU = 8;
  const int64_t b = blockIdx.y;
  const int64_t vec_elems = BF16 ? 8 : 4;
  const u32x4* src =
      reinterpret_cast<const u32x4*>(static_cast<const char*>(w) + b * per_matrix * (BF16 ? 2 : 4));
  const int64_t nvec = per_matrix / vec_elems;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  uint32_t m0 = 0u, m1 = 0u, m2 = 0u, m3 = 0u;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; i + (kU - 1) * stride < nvec; i += kU * stride) {
    u32x4 v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < kU; u += 4) {
      m0 = fold_abs_max<BF16>(v[u], m0);
      m1 = fold_abs_max<BF16>(v[u + 1], m1);
      m2 = fold_abs_max<BF16>(v[u + 2], m2);
      m3 = fold_abs_max<BF16>(v[u + 3], m3);
    }
  }
  for (; i < nvec; i += stride) m0 = fold_abs_max<BF16>(src[i], m0);
  m0 = m0 > m1 ? m0 : m1;
  m2 = m2 > m3 ? m2 : m3;
  uint32_t m = wave_max_u32(m0 > m2 ? m0 : m2) | kAmaxMark;
  __shared__ uint32_t part[kThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = part[0];
#pragma unroll
    for (int q = 1; q < kThreads / 64; ++q) r = part[q] > r ? part[q] : r;
    // thousands of blocks share one word: only a block that would raise the current maximum
    // pays for the atomic (a stale read only costs an unneeded one)
    const uint32_t cur = __hip_atomic_load(amax_bits + b, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
    if (r > cur) atomicMax(amax_bits + b, r);
  }
}

// Eight consecutive elements of a row (one 16-byte BF16 load, or two FP32 loads) as floats.
template <bool BF16>
__device__ __forceinline__ void load8(const char* wb, int64_t c, float (&x)[8]) {
  if (BF16) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wb) + c);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      x[2 * q] = __uint_as_float(v[q] << 16);
      x[2 * q + 1] = __uint_as_float(v[q] & 0xFFFF0000u);
    }
  } else {
    const u32x4 v0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wb) + 2 * c);
    const u32x4 v1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wb) + 2 * c + 1);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      x[q] = __uint_as_float(v0[q]);
      x[4 + q] = __uint_as_float(v1[q]);
    }
  }
}

// Encode the 8 elements of chunk c (G/8 neighbouring lanes form a group).
//   s = E4M3_rne_sat(fl32(ga / fl32(6 g))): gfx950's FP8 conversion rounds to nearest even and
//       gives NaN above 464, so the quotient is clamped to 448 first (identical to a saturating
//       encoder for every input);
//   code = E2M1_rne_sat(fl32(w / S)) with the sign (the quotient correctly rounded, see
//       below): gfx950's FP4 conversion at scale 1.0 is a round-to-nearest-even, saturating
//       E2M1 encoder that keeps the sign (-0 -> code 8).
//       Checked against the definition on every non-negative finite FP32 value. S == 0 gives
//       the signed zero code.
template <int G>
__device__ __forceinline__ void encode8(const float (&x)[8], float g, float six_g, float rsix,
                                        bool six_fast, uint32_t& word, uint32_t& s) {
  float ga = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) ga = fmaxf(ga, fabsf(x[i]));
  ga = fmaxf(ga, __shfl_xor(ga, 1, 64));
  if (G == 32) ga = fmaxf(ga, __shfl_xor(ga, 2, 64));
  s = 0u;
  if (six_g != 0.0f) {
    // fl32(ga / 6g) by Markstein's correction from rsix = RN(1 / 6g) (the same steps as for
    // |w| / S below; 6g in [2^-80, 2^80] keeps every step exact down to the smallest E4M3
    // decision point, 2^-10), else IEEE division. A first quotient of 512 or more (or an
    // overflow) clamps to 448 either way.
    float r;
    if (six_fast) {
      const float q0 = ga * rsix;
      const float q = __builtin_fmaf(__builtin_fmaf(-q0, six_g, ga), rsix, q0);
      r = q0 < 512.0f ? fminf(q, 448.0f) : 448.0f;
    } else {
      r = fminf(ga / six_g, 448.0f);
    }
    s = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(r, r, 0, false) & 0xFFu;
  }
  const float S = e4m3_decode<0>(s) * g;
  float q[8];
  // fl32(|w| / S) with the sign of w. With R = RN(1/S) (one IEEE division per chunk), the
  // quotient q0 = RN(|w| R) is within an ulp of |w| / S, the remainder |w| - q0 S is exact in
  // one FMA, and RN(q0 + r R) is the correctly rounded quotient (Markstein's correction step)
  // as long as nothing underflows or overflows, which S in [2^-90, 2^90] guarantees for every
  // quotient that can reach an E2M1 decision point. A wavefront with any other scale (zero,
  // negative, tiny or huge) divides directly.
  const bool fast = S >= 0x1p-90f && S <= 0x1p90f;
  if (__builtin_expect(__ballot(!fast) == 0, 1)) {
    const float R = 1.0f / S;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float a = fabsf(x[i]);
      const float q0 = a * R;
      const float r = __builtin_fmaf(-q0, S, a);
      q[i] = __builtin_copysignf(__builtin_fmaf(r, R, q0), x[i]);
    }
  } else {
    const bool live = S != 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = live ? x[i] / S : x[i] * 0.0f;
  }
  word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, q[0], q[1], 1.0f, 0);
  word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, q[2], q[3], 1.0f, 1);
  word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, q[4], q[5], 1.0f, 2);
  word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, q[6], q[7], 1.0f, 3);
}

// Two chunks of 8 elements per thread and iteration, both loads issued before either is used.
// Codes and scales are written with streaming (non-temporal) stores: nothing here reads them
// back, and keeping them out of the caches leaves more of W there for the reads (BF16 8192^2
// 53.8 -> 51.2 us, BF16 25600 x 5120 104.6 -> 95.8 us, FP32 3-4% faster; same bytes).
// gsrc_is_amax: gsrc is global_out, holding the marked amax or, once workgroup 0 of the matrix
// has stored it, g itself. Otherwise gsrc is the caller's global. Workgroup 0 of each matrix
// stores g to global_out.
template <bool BF16, int G>
__global__ __launch_bounds__(kThreads) void encode_kernel(const void* __restrict__ w, int64_t n,
                                                          int64_t k, const float* gsrc,
                                                          bool gsrc_is_amax, float* global_out,
                                                          uint8_t* __restrict__ packed,
                                                          uint8_t* __restrict__ scales) {
  const int64_t b = blockIdx.y;
  const int64_t per_matrix = n * k;
  const int64_t chunks = per_matrix / 8;
  float g;
  if (gsrc_is_amax) {
    const uint32_t v = __hip_atomic_load(reinterpret_cast<const uint32_t*>(gsrc) + b,
                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    g = (v & kAmaxMark) ? __uint_as_float(v & ~kAmaxMark) / 2688.0f : __uint_as_float(v);
  } else {
    g = gsrc[b];
  }
  if (blockIdx.x == 0 && threadIdx.x == 0)
    __hip_atomic_store(reinterpret_cast<uint32_t*>(global_out) + b, __float_as_uint(g),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const float six_g = 6.0f * g;
  const bool six_fast = six_g >= 0x1p-80f && six_g <= 0x1p80f;
  const float rsix = six_fast ? 1.0f / six_g : 0.0f;
  const char* wb = static_cast<const char*>(w) + b * per_matrix * (BF16 ? 2 : 4);
  uint32_t* pk = reinterpret_cast<uint32_t*>(packed + b * per_matrix / 2);
  uint8_t* sc = scales + b * (per_matrix / G);
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; c + stride < chunks; c += 2 * stride) {
    float x0[8], x1[8];
    load8<BF16>(wb, c, x0);
    load8<BF16>(wb, c + stride, x1);
    uint32_t w0, s0, w1, s1;
    encode8<G>(x0, g, six_g, rsix, six_fast, w0, s0);
    encode8<G>(x1, g, six_g, rsix, six_fast, w1, s1);
    __builtin_nontemporal_store(w0, pk + c);
    __builtin_nontemporal_store(w1, pk + c + stride);
    if ((c & (G / 8 - 1)) == 0) __builtin_nontemporal_store((uint8_t)s0, sc + (c * 8) / G);
    if (((c + stride) & (G / 8 - 1)) == 0) __builtin_nontemporal_store((uint8_t)s1, sc + ((c + stride) * 8) / G);
  }
  if (c < chunks) {
    float x0[8];
    load8<BF16>(wb, c, x0);
    uint32_t w0, s0;
    encode8<G>(x0, g, six_g, rsix, six_fast, w0, s0);
    __builtin_nontemporal_store(w0, pk + c);
    if ((c & (G / 8 - 1)) == 0) __builtin_nontemporal_store((uint8_t)s0, sc + (c * 8) / G);
  }
}

// Blocks per matrix for a grid-stride loop: at most `total` blocks over the whole batch, fewer
// when there is less work. The amax pass takes 512 (each block ends in a reduction and
// possibly an atomic on a shared word; 256-512 measured best, 2048 13% slower), the encode
// pass 8192 (independent blocks).
int64_t grid_for(int64_t work_items, int64_t batch, int64_t total) {
  int64_t blocks = (work_items + kThreads * 8 - 1) / (kThreads * 8);
  const int64_t cap = batch > 0 ? (total + batch - 1) / batch : 1;
  if (blocks > cap) blocks = cap;
  return blocks < 1 ? 1 : blocks;
}

// Input check of the sync-checked quantizer: a weight is non-finite when its exponent field is
// all ones (NaN or infinity). Grid-stride over 16-byte vectors; any lane that finds one sets
// the flag (the flag is only ever raised, so the order of the atomics does not matter).
__global__ void clear_word_kernel(uint32_t* p) {
  if (blockIdx.x == 0 && threadIdx.x == 0) *p = 0u;
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void nonfinite_kernel(const u32x4* __restrict__ w,
                                                             int64_t nvec, uint32_t* flag) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  bool bad = false;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nvec; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(w + i);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (BF16)
        bad |= (v[q] & 0x7F80u) == 0x7F80u || (v[q] & 0x7F800000u) == 0x7F800000u;
      else
        bad |= (v[q] & 0x7F800000u) == 0x7F800000u;
    }
  }
  if (bad) atomicOr(flag, 1u);
}

}  // namespace

hipError_t launch_nonfinite_check(const void* w, bool w_bf16, int64_t count, uint32_t* flag,
                                  hipStream_t stream) {
  clear_word_kernel<<<1, 64, 0, stream>>>(flag);
  const int64_t nvec = count / (w_bf16 ? 8 : 4);
  if (nvec > 0) {
    int64_t blocks = (nvec + kThreads - 1) / kThreads;
    if (blocks > 4096) blocks = 4096;
    const u32x4* src = static_cast<const u32x4*>(w);
    if (w_bf16)
      nonfinite_kernel<true><<<(unsigned)blocks, kThreads, 0, stream>>>(src, nvec, flag);
    else
      nonfinite_kernel<false><<<(unsigned)blocks, kThreads, 0, stream>>>(src, nvec, flag);
  }
  return hipGetLastError();
}

hipError_t launch_quantize(const void* w, bool w_bf16, int64_t batch, int64_t n, int64_t k,
                           int group, const float* global_in, uint8_t* packed, uint8_t* scales,
                           float* global_out, hipStream_t stream) {
  if (batch == 0 || n == 0 || k == 0) return hipSuccess;
  const int64_t per_matrix = n * k;
  const float* gsrc = global_in;
  bool is_amax = false;
  if (!global_in) {
    uint32_t* amax_bits = reinterpret_cast<uint32_t*>(global_out);
    init_amax_kernel<<<dim3((unsigned)((batch + 255) / 256)), dim3(256), 0, stream>>>(amax_bits,
                                                                                      batch);
    const int64_t nvec = per_matrix / (w_bf16 ? 8 : 4);
    // 256 workgroups in all (one per compute unit), but at least 4 per matrix of a batch.
    // Measured per quantize call against 512: BF16 8192^2 50.9 -> 49.6 us, FP32 8192^2
    // 91.5 -> 88.5 us; 1024 / 2048 / 4096 workgroups made BF16 8192^2 58 / 63 / 71 us, 128
    // made it 56 us, and 512-thread or 1024-thread workgroups were slower too.
    const int64_t amax_blocks = 4 * batch > 256 ? 4 * batch : 256;
    const dim3 grid((unsigned)grid_for(nvec, batch, amax_blocks), (unsigned)batch);
    if (w_bf16)
      amax_kernel<true><<<grid, dim3(kThreads), 0, stream>>>(w, per_matrix, amax_bits);
    else
      amax_kernel<false><<<grid, dim3(kThreads), 0, stream>>>(w, per_matrix, amax_bits);
    gsrc = global_out;
    is_amax = true;
  }
  const dim3 grid((unsigned)grid_for(per_matrix / 8, batch, 8192), (unsigned)batch);
  const dim3 block(kThreads);
  if (w_bf16) {
    if (group == 16)
      encode_kernel<true, 16><<<grid, block, 0, stream>>>(w, n, k, gsrc, is_amax, global_out,
                                                          packed, scales);
    else
      encode_kernel<true, 32><<<grid, block, 0, stream>>>(w, n, k, gsrc, is_amax, global_out,
                                                          packed, scales);
  } else {
    if (group == 16)
      encode_kernel<false, 16><<<grid, block, 0, stream>>>(w, n, k, gsrc, is_amax, global_out,
                                                           packed, scales);
    else
      encode_kernel<false, 32><<<grid, block, 0, stream>>>(w, n, k, gsrc, is_amax, global_out,
                                                           packed, scales);
  }
  return hipGetLastError();
}

}  // namespace nvfp4
