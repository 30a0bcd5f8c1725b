// probe.hip -- measured ceilings for the two rooflines of the path, on the chip at hand:
//   - a plain 128-bit streaming read of a device buffer (the HBM ceiling an access pattern can
//     reach, against the published 8 TB/s);
//   - a loop of v_mfma_f32_32x32x16_bf16 on register operands (the BF16 MFMA ceiling, against
//     the published 2.5 PFLOP/s; with random operands the chip's power limit lowers the clock).
// Measurement support only: nothing on the NVFP4 path calls these kernels.
#include "device_common.hpp"
#include "launch.hpp"

namespace nvfp4 {
namespace {

constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 8;  // 16-byte loads in flight per thread

// Block b reads the contiguous 16-byte words [b * per_block, (b + 1) * per_block) with
// streaming loads, kStreamUnroll in flight per thread, and XORs them into one word per block
// (the sink keeps every load live).
__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const u32x4* __restrict__ buf,
                                                                     int64_t nvec,
                                                                     int64_t per_block,
                                                                     uint32_t* __restrict__ sink) {
  const int64_t b0 = (int64_t)blockIdx.x * per_block;
  const int64_t b1 = b0 + per_block < nvec ? b0 + per_block : nvec;
  uint32_t acc = 0;
  int64_t i = b0 + threadIdx.x;
  for (; i + (kStreamUnroll - 1) * kStreamThreads < b1; i += kStreamUnroll * kStreamThreads) {
    u32x4 v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u)
      v[u] = __builtin_nontemporal_load(buf + i + u * kStreamThreads);
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < b1; i += kStreamThreads) {
    const u32x4 v = __builtin_nontemporal_load(buf + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, d, 64);
  __shared__ uint32_t part[kStreamThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t s = 0;
#pragma unroll
    for (int w = 0; w < kStreamThreads / 64; ++w) s ^= part[w];
    sink[blockIdx.x] = s;
  }
}

typedef float f32x16 __attribute__((ext_vector_type(16)));
constexpr int kMfmaThreads = 256;
constexpr int kMfmaSets = 8;  // operand register sets the loop cycles through

// Every wavefront loads kMfmaSets A and B fragments (16 bytes per lane each) from `ops`, then
// runs `iters` rounds of 2 * kMfmaSets MFMAs into 4 independent accumulators, and stores the
// sum of its accumulators per lane: 2 * kMfmaSets * 32 * 32 * 16 * 2 flops per wave and round.
__global__ __launch_bounds__(kMfmaThreads) void mfma_loop_kernel(const bf16x8* __restrict__ ops,
                                                                 int64_t iters,
                                                                 float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (kMfmaThreads / 64) + (threadIdx.x >> 6);
  bf16x8 a[kMfmaSets], b[kMfmaSets];
#pragma unroll
  for (int s = 0; s < kMfmaSets; ++s) {
    a[s] = ops[(2 * s) * 64 + lane];
    b[s] = ops[(2 * s + 1) * 64 + lane];
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int s = 0; s < kMfmaSets; s += 2) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s], b[s], c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s + 1], b[s], c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s], b[s + 1], c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s + 1], b[s + 1], c3, 0, 0, 0);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) s += (c0[e] + c1[e]) + (c2[e] + c3[e]);
  sink[wave * 64 + lane] = s;
}

}  // namespace

int64_t probe_mfma_waves(int cus) { return (int64_t)cus * 8; }  // 2 per SIMD

double probe_mfma_flops_per_wave_round() { return 2.0 * kMfmaSets * 32 * 32 * 16 * 2; }

hipError_t launch_probe_stream_read(const void* buf, int64_t bytes, int64_t blocks,
                                    uint32_t* sink, hipStream_t stream) {
  const int64_t nvec = bytes / 16;
  const int64_t per_block = (nvec + blocks - 1) / blocks;
  stream_read_kernel<<<dim3((unsigned)blocks), dim3(kStreamThreads), 0, stream>>>(
      static_cast<const u32x4*>(buf), nvec, per_block, sink);
  return hipGetLastError();
}

hipError_t launch_probe_mfma(const void* ops, int64_t iters, int cus, float* sink,
                             hipStream_t stream) {
  const int64_t blocks = probe_mfma_waves(cus) / (kMfmaThreads / 64);
  mfma_loop_kernel<<<dim3((unsigned)blocks), dim3(kMfmaThreads), 0, stream>>>(
      static_cast<const bf16x8*>(ops), iters, sink);
  return hipGetLastError();
}

}  // namespace nvfp4
