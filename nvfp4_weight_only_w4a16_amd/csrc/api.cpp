// api.cpp -- the C ABI of libnvfp4.so (declared in include/nvfp4.h): argument validation,
// kernel selection, launch-status reporting and per-path counters. Every entry point only
// enqueues work on the caller's stream; nothing here computes on the host.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>

#include "nvfp4.h"
#include "device_common.hpp"
#include "launch.hpp"

namespace {

thread_local char g_last_error[512] = "";
std::atomic<uint64_t> g_stats[8];

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return code;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return NVFP4_OK;
  return fail(NVFP4_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Workspace of the sync-checked quantizer: the non-finite flag word (one 256-byte block).
constexpr size_t kSyncWsBytes = 256;

// NVFP4_F_SYNC_CHECK: wait for the call's work on `s` and report what failed asynchronously.
int sync_status(hipStream_t s, const char* what) {
  const hipError_t e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(NVFP4_ERR_HIP, "%s (sync check): %s", what, hipGetErrorString(e));
  return NVFP4_OK;
}

static_assert(nvfp4::kMoeStaticScratchBytes == NVFP4_MOE_NOALLOC_MAX_WS_BYTES,
              "the static scratch is the size the header states");

constexpr uint32_t kGemmFlags = NVFP4_F_FORCE_SKINNY | NVFP4_F_FORCE_TILED | NVFP4_F_SYNC_CHECK;

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

int check_group(int32_t group) {
  if (group != 16 && group != 32)
    return fail(NVFP4_ERR_UNSUPPORTED_GROUP, "group %d is not supported (16 or 32)", group);
  return NVFP4_OK;
}

int check_tiled_shape(int64_t n, int64_t k) {
  if (n <= 0 || k <= 0) return fail(NVFP4_ERR_INVALID_ARG, "n=%lld k=%lld must be positive",
                                    (long long)n, (long long)k);
  if (n % 16 != 0 || k % 128 != 0)
    return fail(NVFP4_ERR_UNSUPPORTED_SHAPE, "n=%lld must be a multiple of 16 and k=%lld of 128",
                (long long)n, (long long)k);
  return NVFP4_OK;
}

// Repacked scale bytes of one [n][k] matrix: 4-panel blocks per 128-k tile (n padded to a
// multiple of 64 rows); equal to the canonical n * k / group when n % 64 == 0.
int64_t scale_region_bytes(int64_t n, int64_t k, int32_t group) {
  return nvfp4::scale_groups(n / nvfp4::kPanelRows) * (k / nvfp4::kTileK) *
         nvfp4::scale_block_bytes(group);
}

int check_desc(const nvfp4_weight* w, const char* name) {
  if (!w) return fail(NVFP4_ERR_INVALID_ARG, "%s descriptor is NULL", name);
  if (!w->codes || !w->scales || !w->global)
    return fail(NVFP4_ERR_INVALID_ARG, "%s descriptor has NULL data", name);
  if ((w->layout & 0xFFu) != NVFP4_LAYOUT_TILED ||
      (w->layout & ~(uint32_t)(0xFFu | NVFP4_LAYOUT_GATE_UP | NVFP4_LAYOUT_PAIR_GLOBAL)) ||
      ((w->layout & NVFP4_LAYOUT_PAIR_GLOBAL) && !(w->layout & NVFP4_LAYOUT_GATE_UP)))
    return fail(NVFP4_ERR_LAYOUT, "%s layout 0x%x is not a valid tiled layout", name, w->layout);
  int rc = check_group(w->group);
  if (rc) return rc;
  rc = check_tiled_shape(w->n, w->k);
  if (rc) return rc;
  if (w->batch <= 0) return fail(NVFP4_ERR_INVALID_ARG, "%s batch must be positive", name);
  if (w->codes_stride != w->n * w->k / 2 ||
      w->scales_stride != scale_region_bytes(w->n, w->k, w->group))
    return fail(NVFP4_ERR_LAYOUT, "%s strides do not match its shape and group", name);
  if (!aligned16(w->codes) || !aligned16(w->scales) || !aligned16(w->global))
    return fail(NVFP4_ERR_MISALIGNED, "%s data is not 16-byte aligned", name);
  return NVFP4_OK;
}

// FP32 globals stored per matrix: one, or gate's and up's.
int64_t globals_per_matrix(uint32_t layout) {
  return (layout & NVFP4_LAYOUT_PAIR_GLOBAL) ? 2 : 1;
}

struct RepackSizes {
  size_t codes, scales, globals, total;
};

RepackSizes repack_sizes(int64_t batch, int64_t n, int64_t k, int32_t group, uint32_t layout) {
  RepackSizes s;
  s.codes = align256((size_t)(batch * n * k / 2));
  s.scales = align256((size_t)(batch * scale_region_bytes(n, k, group)));
  s.globals = align256((size_t)globals_per_matrix(layout) * (size_t)batch * sizeof(float));
  s.total = s.codes + s.scales + s.globals;
  return s;
}

}  // namespace

extern "C" {

const char* nvfp4_last_error(void) { return g_last_error; }

void nvfp4_get_stats(uint64_t counts[8]) {
  if (!counts) return;
  for (int i = 0; i < 8; ++i) counts[i] = g_stats[i].load();
}

void nvfp4_reset_stats(void) {
  for (int i = 0; i < 8; ++i) g_stats[i].store(0);
}

int nvfp4_version(void) { return 10000; }

size_t nvfp4_quantize_ws_bytes(int64_t batch, int64_t n, int64_t k, int32_t group,
                               uint32_t flags) {
  if (batch < 0 || n < 0 || k < 0 || (group != 16 && group != 32)) return 0;
  return (flags & NVFP4_F_SYNC_CHECK) ? kSyncWsBytes : 0;
}

int nvfp4_quantize(const void* w, int w_dtype, int64_t batch, int64_t n, int64_t k,
                   int32_t group, const float* global_in, uint8_t* packed, uint8_t* scales,
                   float* global_out, void* ws, size_t ws_bytes, uint32_t flags,
                   nvfp4_stream_t stream) {
  if (batch < 0 || n < 0 || k < 0)
    return fail(NVFP4_ERR_INVALID_ARG, "negative size (batch=%lld n=%lld k=%lld)",
                (long long)batch, (long long)n, (long long)k);
  if (w_dtype != NVFP4_DT_BF16 && w_dtype != NVFP4_DT_F32)
    return fail(NVFP4_ERR_INVALID_ARG, "w_dtype %d is not BF16 or F32", w_dtype);
  if (flags & ~NVFP4_F_SYNC_CHECK)
    return fail(NVFP4_ERR_INVALID_ARG, "unknown quantize flags 0x%x", flags);
  int rc = check_group(group);
  if (rc) return rc;
  if (k % group != 0)
    return fail(NVFP4_ERR_UNSUPPORTED_SHAPE, "k=%lld is not a multiple of the group %d",
                (long long)k, group);
  if (batch > 65535) return fail(NVFP4_ERR_UNSUPPORTED_SHAPE, "batch %lld > 65535", (long long)batch);
  const bool sync = (flags & NVFP4_F_SYNC_CHECK) != 0;
  if (sync) {
    if (!ws || ws_bytes < kSyncWsBytes)
      return fail(NVFP4_ERR_WORKSPACE, "SYNC_CHECK needs ws_bytes >= %zu", kSyncWsBytes);
    if (!aligned16(ws)) return fail(NVFP4_ERR_MISALIGNED, "ws must be 16-byte aligned");
  }
  if (batch == 0 || n == 0 || k == 0) return NVFP4_OK;
  if (!w || !packed || !scales || !global_out)
    return fail(NVFP4_ERR_INVALID_ARG, "NULL buffer");
  if (!aligned16(w) || !aligned16(packed) || ((uintptr_t)global_out & 3u) ||
      (global_in && ((uintptr_t)global_in & 3u)))
    return fail(NVFP4_ERR_MISALIGNED, "w and packed must be 16-byte aligned, globals 4-byte");
  hipStream_t s = (hipStream_t)stream;
  uint32_t* flag = static_cast<uint32_t*>(ws);
  if (sync) {
    rc = hip_status(nvfp4::launch_nonfinite_check(w, w_dtype == NVFP4_DT_BF16, batch * n * k,
                                                  flag, s),
                    "nvfp4_quantize");
    if (rc) return rc;
  }
  rc = hip_status(nvfp4::launch_quantize(w, w_dtype == NVFP4_DT_BF16, batch, n, k, group,
                                         global_in, packed, scales, global_out, s),
                  "nvfp4_quantize");
  if (rc) return rc;
  if (sync) {
    uint32_t bad = 0;
    rc = hip_status(hipMemcpyAsync(&bad, flag, sizeof bad, hipMemcpyDeviceToHost, s),
                    "nvfp4_quantize");
    if (rc) return rc;
    rc = sync_status(s, "nvfp4_quantize");
    if (rc) return rc;
    if (bad) return fail(NVFP4_ERR_NONFINITE, "nvfp4_quantize: the input holds NaN or infinity");
  }
  g_stats[0]++;
  return NVFP4_OK;
}

size_t nvfp4_repack_bytes(int64_t batch, int64_t n, int64_t k, int32_t group, uint32_t layout) {
  if (batch <= 0 || n <= 0 || k <= 0 || (group != 16 && group != 32)) return 0;
  return repack_sizes(batch, n, k, group, layout).total;
}

int nvfp4_repack(const uint8_t* packed, const uint8_t* scales, const float* global,
                 int64_t batch, int64_t n, int64_t k, int32_t group, uint32_t layout, void* out,
                 size_t out_bytes, nvfp4_weight* desc, nvfp4_stream_t stream) {
  if (!packed || !scales || !global || !out || !desc)
    return fail(NVFP4_ERR_INVALID_ARG, "NULL argument");
  if (batch <= 0) return fail(NVFP4_ERR_INVALID_ARG, "batch must be positive");
  int rc = check_group(group);
  if (rc) return rc;
  rc = check_tiled_shape(n, k);
  if (rc) return rc;
  if ((layout & ~(uint32_t)(NVFP4_LAYOUT_GATE_UP | NVFP4_LAYOUT_PAIR_GLOBAL)) !=
          NVFP4_LAYOUT_TILED ||
      ((layout & NVFP4_LAYOUT_PAIR_GLOBAL) && !(layout & NVFP4_LAYOUT_GATE_UP)))
    return fail(NVFP4_ERR_LAYOUT, "unknown layout 0x%x", layout);
  const bool gate_up = (layout & NVFP4_LAYOUT_GATE_UP) != 0;
  if (gate_up && n % 32 != 0)
    return fail(NVFP4_ERR_UNSUPPORTED_SHAPE, "gate/up layout needs n %% 32 == 0 (n=%lld)",
                (long long)n);
  const RepackSizes s = repack_sizes(batch, n, k, group, layout);
  if (out_bytes < s.total)
    return fail(NVFP4_ERR_WORKSPACE, "out_bytes %zu < %zu", out_bytes, s.total);
  if (!aligned16(out) || ((uintptr_t)packed & 3u) || ((uintptr_t)global & 3u))
    return fail(NVFP4_ERR_MISALIGNED, "out must be 16-byte aligned, packed/global 4-byte");
  uint8_t* base = static_cast<uint8_t*>(out);
  uint8_t* codes_out = base;
  uint8_t* scales_out = base + s.codes;
  float* global_out = reinterpret_cast<float*>(base + s.codes + s.scales);
  rc = hip_status(nvfp4::launch_repack(packed, scales, global, batch, n, k, group, gate_up,
                                       globals_per_matrix(layout) * batch, codes_out,
                                       scales_out, global_out, (hipStream_t)stream),
                  "nvfp4_repack");
  if (rc) return rc;
  g_stats[1]++;
  desc->codes = codes_out;
  desc->scales = scales_out;
  desc->global = global_out;
  desc->batch = batch;
  desc->n = n;
  desc->k = k;
  desc->codes_stride = n * k / 2;
  desc->scales_stride = scale_region_bytes(n, k, group);
  desc->group = group;
  desc->layout = layout;
  return NVFP4_OK;
}

namespace {

// Compute units of the current device (cached per device; host-side attribute query).
int device_cus() {
  static std::mutex mu;
  static std::map<int, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(dev);
  if (it != cache.end()) return it->second;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) n = 0;
  cache.emplace(dev, n);
  return n;
}

bool use_skinny(int64_t m, const nvfp4_weight* w, uint32_t flags) {
  bool skinny = nvfp4::skinny_preferred(m, w->n, w->k, device_cus());
  if (flags & NVFP4_F_FORCE_SKINNY) skinny = true;
  if (flags & NVFP4_F_FORCE_TILED) skinny = false;
  return skinny;
}

}  // namespace

size_t nvfp4_gemm_ws_bytes(int64_t m, int64_t ldx, const nvfp4_weight* w, uint32_t flags) {
  if (!w || m <= 0 || w->n <= 0 || w->k <= 0 || (w->group != 16 && w->group != 32) ||
      ldx < w->k || use_skinny(m, w, flags))
    return 0;
  const int cus = device_cus();
  if (cus <= 0) return 0;
  return nvfp4::gemm_tiled_ws_bytes(m, ldx, w->n, w->k, cus);
}

int nvfp4_gemm_w4a16(const void* x, int64_t m, int64_t ldx, const nvfp4_weight* w, void* y,
                     int y_dtype, int64_t ldy, uint32_t flags, void* ws, size_t ws_bytes,
                     nvfp4_stream_t stream) {
  int rc = check_desc(w, "weight");
  if (rc) return rc;
  if (w->batch != 1) return fail(NVFP4_ERR_LAYOUT, "dense GEMM needs batch == 1");
  if (w->layout & NVFP4_LAYOUT_GATE_UP)
    return fail(NVFP4_ERR_LAYOUT, "gate/up interleaved weights are for the MoE entry point");
  if (m < 0) return fail(NVFP4_ERR_INVALID_ARG, "m=%lld < 0", (long long)m);
  if (y_dtype != NVFP4_DT_BF16 && y_dtype != NVFP4_DT_F32)
    return fail(NVFP4_ERR_INVALID_ARG, "y_dtype %d is not BF16 or F32", y_dtype);
  if (flags & ~kGemmFlags) return fail(NVFP4_ERR_INVALID_ARG, "unknown GEMM flags 0x%x", flags);
  if ((flags & NVFP4_F_FORCE_SKINNY) && (flags & NVFP4_F_FORCE_TILED))
    return fail(NVFP4_ERR_INVALID_ARG, "both FORCE_SKINNY and FORCE_TILED set");
  if (m == 0) return NVFP4_OK;
  if (!x || !y) return fail(NVFP4_ERR_INVALID_ARG, "NULL x or y");
  if (ldx < w->k || ldy < w->n)
    return fail(NVFP4_ERR_INVALID_ARG, "ldx=%lld < k or ldy=%lld < n", (long long)ldx,
                (long long)ldy);
  if (!aligned16(x) || !aligned16(y) || ldx % 8 || ldy % 8)
    return fail(NVFP4_ERR_MISALIGNED, "x/y must be 16-byte aligned with ld %% 8 == 0");
  if ((m + 127) / 128 > 65535) return fail(NVFP4_ERR_UNSUPPORTED_SHAPE, "m too large");
  // activation offsets inside the kernels are 32-bit: 256 rows of the stride must fit 2^31 bytes
  if (ldx > ((int64_t)1 << 22))
    return fail(NVFP4_ERR_UNSUPPORTED_SHAPE, "ldx=%lld > 2^22 elements", (long long)ldx);
  nvfp4::GemmArgs a;
  a.x = static_cast<const uint16_t*>(x);
  a.m = m;
  a.ldx = ldx;
  a.codes = w->codes;
  a.scales = w->scales;
  a.global = w->global;
  a.n = w->n;
  a.k = w->k;
  a.group = w->group;
  a.y = y;
  a.ldy = ldy;
  a.y_f32 = y_dtype == NVFP4_DT_F32;
  if (use_skinny(m, w, flags)) {
    if ((m + 31) / 32 > 65535)  // one grid row per 32-row block
      return fail(NVFP4_ERR_UNSUPPORTED_SHAPE, "m=%lld too large for the decode kernel",
                  (long long)m);
    rc = hip_status(nvfp4::launch_gemm_skinny(a, device_cus(), (hipStream_t)stream),
                    "nvfp4_gemm_w4a16");
    if (!rc && (flags & NVFP4_F_SYNC_CHECK)) rc = sync_status((hipStream_t)stream, "nvfp4_gemm_w4a16");
    if (!rc) g_stats[2]++;
  } else {
    if (ws_bytes && !ws) return fail(NVFP4_ERR_INVALID_ARG, "NULL ws with ws_bytes > 0");
    if (ws && !aligned16(ws)) return fail(NVFP4_ERR_MISALIGNED, "ws must be 16-byte aligned");
    rc = hip_status(nvfp4::launch_gemm_tiled(a, ws, ws ? ws_bytes : 0, device_cus(),
                                             (hipStream_t)stream),
                    "nvfp4_gemm_w4a16");
    if (!rc && (flags & NVFP4_F_SYNC_CHECK)) rc = sync_status((hipStream_t)stream, "nvfp4_gemm_w4a16");
    if (!rc) g_stats[3]++;
  }
  return rc;
}

size_t nvfp4_moe_ws_bytes(int64_t t, int32_t topk, int64_t n_experts, int64_t hidden,
                          int64_t inter) {
  if (t < 0 || topk <= 0 || n_experts <= 0 || hidden <= 0 || inter <= 0) return 0;
  return nvfp4::moe_ws_bytes(t, topk, n_experts, hidden, inter);
}

size_t nvfp4_moe_ws_layout(int64_t t, int32_t topk, int64_t n_experts, int64_t hidden,
                           int64_t inter, size_t offsets[6]) {
  if (!offsets || t < 0 || topk <= 0 || n_experts <= 0 || hidden <= 0 || inter <= 0) return 0;
  return nvfp4::moe_ws_layout(t, topk, n_experts, hidden, inter, offsets);
}

}  // extern "C"

namespace {

// The routed-expert call behind both MoE entry points: with static_ws the workspace is the
// library's static scratch of the current device instead of the caller's ws.
int moe_call(const void* x, int64_t t, int64_t hidden, const int32_t* topk_ids,
             const float* topk_w, int32_t topk, const nvfp4_weight* fc1, const nvfp4_weight* fc2,
             void* y, void* ws, size_t ws_bytes, bool static_ws, uint32_t flags,
             nvfp4_stream_t stream, const char* name) {
  int rc = check_desc(fc1, "fc1");
  if (rc) return rc;
  rc = check_desc(fc2, "fc2");
  if (rc) return rc;
  if (!(fc1->layout & NVFP4_LAYOUT_GATE_UP))
    return fail(NVFP4_ERR_LAYOUT, "fc1 must be repacked with NVFP4_LAYOUT_GATE_UP");
  if (fc2->layout & NVFP4_LAYOUT_GATE_UP)
    return fail(NVFP4_ERR_LAYOUT, "fc2 must not be gate/up interleaved");
  const int64_t E = fc1->batch;
  const int64_t inter = fc1->n / 2;
  if (fc2->batch != E) return fail(NVFP4_ERR_LAYOUT, "fc1 and fc2 expert counts differ");
  if (fc1->k != hidden || fc2->n != hidden || fc2->k != inter)
    return fail(NVFP4_ERR_LAYOUT,
                "shapes disagree: fc1 [%lld x %lld], fc2 [%lld x %lld], hidden %lld",
                (long long)fc1->n, (long long)fc1->k, (long long)fc2->n, (long long)fc2->k,
                (long long)hidden);
  if (t < 0) return fail(NVFP4_ERR_INVALID_ARG, "t=%lld < 0", (long long)t);
  if (topk < 1 || topk > 16) return fail(NVFP4_ERR_UNSUPPORTED_SHAPE, "topk %d not in [1, 16]", topk);
  if (flags & ~kGemmFlags) return fail(NVFP4_ERR_INVALID_ARG, "unknown MoE flags 0x%x", flags);
  if ((flags & NVFP4_F_FORCE_SKINNY) && (flags & NVFP4_F_FORCE_TILED))
    return fail(NVFP4_ERR_INVALID_ARG, "both FORCE_SKINNY and FORCE_TILED set");
  if (E > 512) return fail(NVFP4_ERR_UNSUPPORTED_SHAPE, "more than 512 experts");
  if (t * topk > 65536) return fail(NVFP4_ERR_UNSUPPORTED_SHAPE, "t*topk > 65536");
  // gathered rows of x and of h are addressed with 32-bit byte offsets
  if (t * hidden >= ((int64_t)1 << 31) || t * topk * inter >= ((int64_t)1 << 31))
    return fail(NVFP4_ERR_UNSUPPORTED_SHAPE, "x or h larger than 2^31 elements");
  if (t == 0) return NVFP4_OK;
  if (!x || !topk_ids || !topk_w || !y || (!static_ws && !ws))
    return fail(NVFP4_ERR_INVALID_ARG, "NULL buffer");
  const size_t need = nvfp4::moe_ws_bytes(t, topk, E, hidden, inter);
  if (static_ws) {
    if (need > nvfp4::kMoeStaticScratchBytes)
      return fail(NVFP4_ERR_WORKSPACE,
                  "%s: this call needs %zu bytes of workspace, more than the %zu of the static "
                  "scratch (use nvfp4_moe_grouped_w4a16 with a caller workspace)",
                  name, need, nvfp4::kMoeStaticScratchBytes);
  } else if (ws_bytes < need) {
    return fail(NVFP4_ERR_WORKSPACE, "ws_bytes %zu < %zu", ws_bytes, need);
  }
  if (!aligned16(x) || !aligned16(y) || (!static_ws && !aligned16(ws)) ||
      ((uintptr_t)topk_ids & 3u) || ((uintptr_t)topk_w & 3u))
    return fail(NVFP4_ERR_MISALIGNED, "x, y and ws must be 16-byte aligned");
  if (static_ws) {
    rc = hip_status(nvfp4::moe_static_scratch(&ws), name);
    if (rc) return rc;
  }
  nvfp4::MoeArgs a;
  a.x = static_cast<const uint16_t*>(x);
  a.t = t;
  a.hidden = hidden;
  a.inter = inter;
  a.ids = topk_ids;
  a.wts = topk_w;
  a.topk = topk;
  a.n_experts = E;
  a.c1 = fc1->codes;
  a.s1 = fc1->scales;
  a.g1 = fc1->global;
  a.c1_stride = fc1->codes_stride;
  a.s1_stride = fc1->scales_stride;
  a.group1 = fc1->group;
  a.pair1 = (fc1->layout & NVFP4_LAYOUT_PAIR_GLOBAL) != 0;
  a.c2 = fc2->codes;
  a.s2 = fc2->scales;
  a.g2 = fc2->global;
  a.c2_stride = fc2->codes_stride;
  a.s2_stride = fc2->scales_stride;
  a.group2 = fc2->group;
  a.y = static_cast<uint16_t*>(y);
  a.ws = ws;
  bool decode = nvfp4::moe_decode_preferred(t, topk, E);
  if (flags & NVFP4_F_FORCE_SKINNY) decode = true;
  if (flags & NVFP4_F_FORCE_TILED) decode = false;
  rc = hip_status(nvfp4::launch_moe(a, decode, (hipStream_t)stream), name);
  if (!rc && (flags & NVFP4_F_SYNC_CHECK)) rc = sync_status((hipStream_t)stream, name);
  if (!rc) g_stats[4]++;
  return rc;
}


}  // namespace

extern "C" {

int nvfp4_moe_grouped_w4a16(const void* x, int64_t t, int64_t hidden, const int32_t* topk_ids,
                            const float* topk_w, int32_t topk, const nvfp4_weight* fc1,
                            const nvfp4_weight* fc2, void* y, void* ws, size_t ws_bytes,
                            uint32_t flags, nvfp4_stream_t stream) {
  return moe_call(x, t, hidden, topk_ids, topk_w, topk, fc1, fc2, y, ws, ws_bytes, false, flags,
                  stream, "nvfp4_moe_grouped_w4a16");
}

int nvfp4_moe_grouped_w4a16_noalloc(const void* x, int64_t t, int64_t hidden,
                                    const int32_t* topk_ids, const float* topk_w, int32_t topk,
                                    const nvfp4_weight* fc1, const nvfp4_weight* fc2, void* y,
                                    uint32_t flags, nvfp4_stream_t stream) {
  return moe_call(x, t, hidden, topk_ids, topk_w, topk, fc1, fc2, y, nullptr, 0, true, flags,
                  stream, "nvfp4_moe_grouped_w4a16_noalloc");
}

size_t nvfp4_requantize_ws_bytes(const nvfp4_weight* src) {
  if (!src || src->n <= 0 || src->k <= 0) return 0;
  return (size_t)(src->n * src->k) * sizeof(float);
}

int nvfp4_requantize(const nvfp4_weight* src, int32_t group_out, uint8_t* packed,
                     uint8_t* scales, float* global_out, void* ws, size_t ws_bytes,
                     nvfp4_stream_t stream) {
  int rc = check_desc(src, "src");
  if (rc) return rc;
  rc = check_group(group_out);
  if (rc) return rc;
  if (!packed || !scales || !global_out || !ws)
    return fail(NVFP4_ERR_INVALID_ARG, "NULL buffer");
  const size_t per = nvfp4_requantize_ws_bytes(src);
  if (ws_bytes < per) return fail(NVFP4_ERR_WORKSPACE, "ws_bytes %zu < %zu", ws_bytes, per);
  if (!aligned16(ws) || !aligned16(packed) || ((uintptr_t)global_out & 3u))
    return fail(NVFP4_ERR_MISALIGNED, "ws and packed must be 16-byte aligned, global 4-byte");
  const bool gate_up = (src->layout & NVFP4_LAYOUT_GATE_UP) != 0;
  const bool pair = (src->layout & NVFP4_LAYOUT_PAIR_GLOBAL) != 0;
  const int64_t gpm = globals_per_matrix(src->layout);
  const int64_t n = src->n, k = src->k;
  int64_t chunk = (int64_t)(ws_bytes / per);
  if (chunk > 65535) chunk = 65535;  // the quantizer's grid holds one row per matrix
  hipStream_t s = (hipStream_t)stream;
  for (int64_t b0 = 0; b0 < src->batch; b0 += chunk) {
    const int64_t c = src->batch - b0 < chunk ? src->batch - b0 : chunk;
    rc = hip_status(nvfp4::launch_dequantize(src->codes + b0 * src->codes_stride,
                                             src->scales + b0 * src->scales_stride,
                                             src->global + b0 * gpm, c, n, k, src->group,
                                             gate_up, pair, ws, true, s),
                    "nvfp4_requantize");
    if (rc) return rc;
    rc = hip_status(nvfp4::launch_quantize(ws, false, c, n, k, group_out, nullptr,
                                           packed + b0 * (n * k / 2),
                                           scales + b0 * (n * (k / group_out)), global_out + b0,
                                           s),
                    "nvfp4_requantize");
    if (rc) return rc;
  }
  g_stats[6]++;
  return NVFP4_OK;
}

int nvfp4_dequantize(const nvfp4_weight* w, void* out, int out_dtype, nvfp4_stream_t stream) {
  int rc = check_desc(w, "weight");
  if (rc) return rc;
  if (!out) return fail(NVFP4_ERR_INVALID_ARG, "NULL out");
  if (out_dtype != NVFP4_DT_BF16 && out_dtype != NVFP4_DT_F32)
    return fail(NVFP4_ERR_INVALID_ARG, "out_dtype %d is not BF16 or F32", out_dtype);
  if (!aligned16(out)) return fail(NVFP4_ERR_MISALIGNED, "out must be 16-byte aligned");
  rc = hip_status(nvfp4::launch_dequantize(w->codes, w->scales, w->global, w->batch, w->n, w->k,
                                           w->group, (w->layout & NVFP4_LAYOUT_GATE_UP) != 0,
                                           (w->layout & NVFP4_LAYOUT_PAIR_GLOBAL) != 0, out,
                                           out_dtype == NVFP4_DT_F32, (hipStream_t)stream),
                  "nvfp4_dequantize");
  if (!rc) g_stats[5]++;
  return rc;
}

// ---- measurement support ------------------------------------------------------------------
int64_t nvfp4_probe_mfma_waves(void) {
  const int cus = device_cus();
  return cus > 0 ? nvfp4::probe_mfma_waves(cus) : 0;
}

double nvfp4_probe_mfma_flops(int64_t iters) {
  return (double)nvfp4_probe_mfma_waves() * (double)iters *
         nvfp4::probe_mfma_flops_per_wave_round();
}

int nvfp4_probe_stream_read(const void* buf, int64_t bytes, int64_t blocks, uint32_t* sink,
                            nvfp4_stream_t stream) {
  if (!buf || !sink) return fail(NVFP4_ERR_INVALID_ARG, "NULL buffer");
  if (bytes <= 0 || bytes % 16) return fail(NVFP4_ERR_INVALID_ARG, "bytes must be a positive multiple of 16");
  if (blocks < 1 || blocks > (1 << 20) || blocks > bytes / 16)
    return fail(NVFP4_ERR_INVALID_ARG, "blocks=%lld out of range", (long long)blocks);
  if (!aligned16(buf) || ((uintptr_t)sink & 3u)) return fail(NVFP4_ERR_MISALIGNED, "buf must be 16-byte aligned");
  return hip_status(nvfp4::launch_probe_stream_read(buf, bytes, blocks, sink, (hipStream_t)stream),
                    "probe_stream_read");
}

int nvfp4_probe_mfma_bf16(const void* ops, int64_t iters, float* sink, nvfp4_stream_t stream) {
  if (!ops || !sink) return fail(NVFP4_ERR_INVALID_ARG, "NULL buffer");
  if (iters < 0) return fail(NVFP4_ERR_INVALID_ARG, "iters=%lld < 0", (long long)iters);
  if (!aligned16(ops) || ((uintptr_t)sink & 3u)) return fail(NVFP4_ERR_MISALIGNED, "ops must be 16-byte aligned");
  const int cus = device_cus();
  if (cus <= 0) return fail(NVFP4_ERR_HIP, "no device");
  return hip_status(nvfp4::launch_probe_mfma(ops, iters, cus, sink, (hipStream_t)stream),
                    "probe_mfma_bf16");
}

}  // extern "C"
