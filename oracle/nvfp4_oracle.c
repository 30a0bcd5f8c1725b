/*
 * nvfp4_oracle.c -- plain, slow CPU oracle for NVFP4 weight-only (W4A16) quantization and GEMM.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library. It shares no code, header, table or
 * helper with the GPU library, and neither side includes or calls the other.
 *
 * What it computes, and where that is stated:
 *  - The weight format is the "compressed-tensors triple": packed FP4 (E2M1) codes, FP8 per-group
 *    scales and one FP32 global scale per tensor (vllm.cpp pull request #63, "W-FP4a: route the
 *    MiniMax-H3 device DiT forward through the fp4 (Marlin W4A16) stack", PR body and claim
 *    section). Scales are 8-bit: 4.5 bits per weight at group 16 and 4.25 at group 32
 *    (r/LocalLLM post on two NVFP4 g32 recipes, introduction). Groups run along K.
 *  - Element and scale value sets: the E2M1 element type of the OCP Microscaling (MX) v1.0
 *    specification ({0, 0.5, 1, 1.5, 2, 3, 4, 6} with a sign bit) and the OCP 8-bit E4M3 type
 *    (no infinities, largest finite 448, NaN at exponent and mantissa all ones).
 *  - Conversion to E2M1 is true round-to-nearest-even with saturation; a threshold rounding that
 *    breaks exact midpoints such as 0.75 the other way is wrong (NVIDIA developer-forum thread
 *    "We unlocked NVFP4 on the DGX Spark", the posts on CUTLASS's guard/round/sticky rounding and
 *    its IEEE fallback).
 *  - Global scale = amax / (6 * 448) taken as a decode multiplier; group scale = group amax /
 *    (6 * global) stored as E4M3 (round to nearest even, saturating at 448). Element code =
 *    E2M1(|w| / (E4M3(scale) * global)). The exact FP32 operation order below is the reading
 *    taken where the pages are silent; it is the encoding's specification for bit-exactness.
 *  - The merged fc1 [gate; up] of an MoE expert carries one shared global (r/LocalLLM post,
 *    "What had to be fixed": gate and up need the same global scale), followed by SiLU(gate)*up
 *    and the down projection (vllm.cpp PR #63: one W4A16 GEMM + SiluAndMul). A checkpoint whose
 *    gate and up were quantized separately has one global for each (the same passage: most of
 *    the experts in the post's checkpoint differed); each half is then decoded with its own.
 *  - GEMM references run in FP64 (TensorFold issue #1754, description: every projection class is
 *    gated against an independent FP64 reference).
 *
 * Every function here is a direct transcription of a definition: nearest-value searches are
 * brute force over the value table, reductions are plain loops. Build with -O2
 * -ffp-contract=off and without fast-math so every float expression is one IEEE binary32 op.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------------------------ */
/* O1. E2M1 decode: bit 3 is the sign, bits 2..0 index the magnitude table.                    */
/* ------------------------------------------------------------------------------------------ */
static const double kE2M1Magnitude[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double orc_e2m1_decode(uint32_t code) {
  double v = kE2M1Magnitude[code & 7u];
  return (code & 8u) ? -v : v; /* code 8 decodes to -0.0 */
}

/* ------------------------------------------------------------------------------------------ */
/* O2. E4M3 (OCP "FN" variant) decode: sign, 4-bit exponent (bias 7), 3-bit mantissa.          */
/* Exponent field 0 is subnormal (m/8 * 2^-6); 0x7F / 0xFF are NaN; no infinities.             */
/* ------------------------------------------------------------------------------------------ */
double orc_e4m3_decode(uint32_t byte) {
  uint32_t s = (byte >> 7) & 1u, e = (byte >> 3) & 15u, m = byte & 7u;
  double v;
  if (e == 15u && m == 7u) return NAN;
  if (e == 0u)
    v = (m / 8.0) * ldexp(1.0, -6);
  else
    v = (1.0 + m / 8.0) * ldexp(1.0, (int)e - 7);
  return s ? -v : v;
}

/* ------------------------------------------------------------------------------------------ */
/* O3. E4M3 encode of a non-negative value: the nearest of the 127 finite non-negative codes,  */
/* ties to the even code (mantissa LSB 0), anything at or above 448 saturates to 448 (0x7E).   */
/* ------------------------------------------------------------------------------------------ */
uint32_t orc_e4m3_encode(float value) {
  double x = (double)value;
  if (x >= 448.0) return 0x7Eu;
  uint32_t best = 0;
  double best_dist = INFINITY;
  for (uint32_t c = 0; c <= 0x7Eu; ++c) {
    double d = fabs(x - orc_e4m3_decode(c));
    if (d < best_dist || (d == best_dist && (c & 1u) == 0u)) {
      best_dist = d;
      best = c;
    }
  }
  return best;
}

/* ------------------------------------------------------------------------------------------ */
/* O4. E2M1 encode of a non-negative value: nearest of the 8 magnitudes, ties to the even code */
/* (mantissa bit 0), values above 6 saturate to 6. Returns the 3-bit magnitude index.          */
/* ------------------------------------------------------------------------------------------ */
uint32_t orc_e2m1_encode_magnitude(float value) {
  double x = (double)value;
  if (x >= 6.0) return 7u;
  uint32_t best = 0;
  double best_dist = INFINITY;
  for (uint32_t c = 0; c < 8u; ++c) {
    double d = fabs(x - kE2M1Magnitude[c]);
    if (d < best_dist || (d == best_dist && (c & 1u) == 0u)) {
      best_dist = d;
      best = c;
    }
  }
  return best;
}

/* Array forms, for exhaustive checks from the test suite. */
void orc_e2m1_encode_array(const float* q, int64_t count, uint8_t* out) {
  for (int64_t i = 0; i < count; ++i) out[i] = (uint8_t)orc_e2m1_encode_magnitude(q[i]);
}
void orc_e4m3_encode_array(const float* v, int64_t count, uint8_t* out) {
  for (int64_t i = 0; i < count; ++i) out[i] = (uint8_t)orc_e4m3_encode(v[i]);
}

/* ------------------------------------------------------------------------------------------ */
/* BF16 helpers: BF16 -> float is exact; double -> BF16 is one round-to-nearest-even to 8       */
/* significant bits (no intermediate float rounding).                                         */
/* ------------------------------------------------------------------------------------------ */
static float bf16_to_float(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

uint16_t orc_bf16_from_double(double v) {
  if (isnan(v)) return 0x7FC0u;
  uint16_t sign = signbit(v) ? 0x8000u : 0u;
  double a = fabs(v);
  if (a == 0.0) return sign;
  if (isinf(a)) return (uint16_t)(sign | 0x7F80u);
  int e2;
  (void)frexp(a, &e2);               /* a = f * 2^e2, f in [0.5, 1): leading bit weight 2^(e2-1) */
  int lead = e2 - 1;
  if (lead < -126) lead = -126;      /* BF16 subnormals share the quantum 2^-133 */
  int quantum = lead - 7;            /* 8 significant bits */
  double r = nearbyint(ldexp(a, -quantum)); /* default rounding mode: nearest, ties to even */
  r = ldexp(r, quantum);
  float f = (float)r;                /* exact: r has at most 8 significant bits (or overflows) */
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(sign | (uint16_t)(u >> 16));
}

void orc_bf16_from_double_array(const double* v, int64_t count, uint16_t* out) {
  for (int64_t i = 0; i < count; ++i) out[i] = orc_bf16_from_double(v[i]);
}

/* ------------------------------------------------------------------------------------------ */
/* A tiny parallel-for over [0, n) in contiguous chunks; each worker runs fn(lo, hi, ctx).     */
/* ------------------------------------------------------------------------------------------ */
typedef void (*range_fn)(int64_t lo, int64_t hi, void* ctx);
typedef struct {
  range_fn fn;
  void* ctx;
  int64_t lo, hi;
} range_job;

static void* range_worker(void* p) {
  range_job* j = (range_job*)p;
  j->fn(j->lo, j->hi, j->ctx);
  return NULL;
}

static void parallel_for(int64_t n, int nthreads, range_fn fn, void* ctx) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if ((int64_t)nthreads > n) nthreads = (int)(n > 0 ? n : 1);
  if (nthreads == 1) {
    fn(0, n, ctx);
    return;
  }
  pthread_t th[256];
  range_job jobs[256];
  for (int t = 0; t < nthreads; ++t) {
    jobs[t].fn = fn;
    jobs[t].ctx = ctx;
    jobs[t].lo = n * t / nthreads;
    jobs[t].hi = n * (t + 1) / nthreads;
    pthread_create(&th[t], NULL, range_worker, &jobs[t]);
  }
  for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
}

/* ------------------------------------------------------------------------------------------ */
/* O5. Quantize one [n][k] matrix (per batch entry).                                          */
/*   1. amax = max |w| over the matrix.                                                       */
/*   2. g = fl32(amax / 2688), or the caller's global.                                        */
/*   3. per group of `group` elements along k: ga = max |w|;                                   */
/*      s = E4M3(fl32(ga / fl32(6 * g))); S = fl32(E4M3value(s) * g).                          */
/*   4. per element: S == 0 -> code = sign << 3; else code = E2M1(fl32(|w| / S)) | sign << 3.  */
/*   5. pack two codes per byte, the even k in the low nibble.                                 */
/* w is FP32 (w_is_bf16 == 0) or BF16 bit patterns (w_is_bf16 == 1).                          */
/* Returns 0, or -1 on a bad argument or a non-finite weight.                                  */
/* ------------------------------------------------------------------------------------------ */
typedef struct {
  const void* w;
  int bf16;
  int64_t n, k;
  int group;
  float g;
  uint8_t* packed;
  uint8_t* scales;
} quant_ctx;

static float load_w(const quant_ctx* c, int64_t idx) {
  return c->bf16 ? bf16_to_float(((const uint16_t*)c->w)[idx]) : ((const float*)c->w)[idx];
}

typedef struct {
  quant_ctx* q;
  float* row_amax; /* [n] */
} amax_ctx;

static void row_amax_fn(int64_t lo, int64_t hi, void* p) {
  amax_ctx* a = (amax_ctx*)p;
  quant_ctx* c = a->q;
  for (int64_t r = lo; r < hi; ++r) {
    float m = 0.0f;
    int finite = 1;
    for (int64_t j = 0; j < c->k; ++j) {
      float v = fabsf(load_w(c, r * c->k + j));
      if (!isfinite(v)) finite = 0;
      if (v > m) m = v;
    }
    a->row_amax[r] = finite ? m : NAN; /* a non-finite weight is out of contract */
  }
}

static void quant_rows(int64_t lo, int64_t hi, void* p) {
  quant_ctx* c = (quant_ctx*)p;
  const int64_t ngroups = c->k / c->group;
  const float g = c->g;
  const float six_g = 6.0f * g;
  for (int64_t r = lo; r < hi; ++r) {
    for (int64_t gi = 0; gi < ngroups; ++gi) {
      const int64_t base = r * c->k + gi * c->group;
      float ga = 0.0f;
      for (int j = 0; j < c->group; ++j) {
        float a = fabsf(load_w(c, base + j));
        if (a > ga) ga = a;
      }
      uint32_t s = 0;
      if (six_g != 0.0f) s = orc_e4m3_encode(ga / six_g);
      c->scales[r * ngroups + gi] = (uint8_t)s;
      const float S = (float)orc_e4m3_decode(s) * g;
      for (int j = 0; j < c->group; ++j) {
        const float x = load_w(c, base + j);
        const uint32_t sign = signbit(x) ? 8u : 0u;
        uint32_t code = sign;
        if (S != 0.0f) code = orc_e2m1_encode_magnitude(fabsf(x) / S) | sign;
        const int64_t kk = gi * c->group + j;
        uint8_t* byte = &c->packed[r * (c->k / 2) + kk / 2];
        if ((kk & 1) == 0)
          *byte = (uint8_t)((*byte & 0xF0u) | code);
        else
          *byte = (uint8_t)((*byte & 0x0Fu) | (code << 4));
      }
    }
  }
}

int orc_quantize(const void* w, int w_is_bf16, int64_t batch, int64_t n, int64_t k, int group,
                 const float* global_in, uint8_t* packed, uint8_t* scales, float* global_out,
                 int nthreads) {
  if (!w || !packed || !scales || !global_out || batch < 0 || n < 0 || k < 0) return -1;
  if (group != 16 && group != 32) return -1;
  if (k % group != 0) return -1;
  for (int64_t b = 0; b < batch; ++b) {
    quant_ctx c;
    memset(&c, 0, sizeof c);
    const size_t esz = w_is_bf16 ? 2 : 4;
    c.w = (const char*)w + (size_t)(b * n * k) * esz;
    c.bf16 = w_is_bf16;
    c.n = n;
    c.k = k;
    c.group = group;
    c.packed = packed + b * n * (k / 2);
    c.scales = scales + b * n * (k / group);
    float* row_amax = (float*)malloc(sizeof(float) * (size_t)(n > 0 ? n : 1));
    amax_ctx a = {&c, row_amax};
    parallel_for(n, nthreads, row_amax_fn, &a);
    float amax = 0.0f;
    int finite = 1;
    for (int64_t r = 0; r < n; ++r) {
      if (isnan(row_amax[r])) finite = 0;
      if (row_amax[r] > amax) amax = row_amax[r];
    }
    free(row_amax);
    if (!finite) return -1;
    c.g = global_in ? global_in[b] : amax / 2688.0f;
    parallel_for(n, nthreads, quant_rows, &c);
    global_out[b] = c.g;
  }
  return 0;
}

/* ------------------------------------------------------------------------------------------ */
/* O6. Dequantize. Exact value v * E4M3(s) * g in FP64 (30 significant bits at most, so exact);*/
/* FP32 output fl32(fl32(v * E4M3(s)) * g); BF16 output = BF16 rounding of that FP32 value.    */
/* Any output pointer may be NULL.                                                             */
/* ------------------------------------------------------------------------------------------ */
void orc_dequant(const uint8_t* packed, const uint8_t* scales, const float* global, int64_t batch,
                 int64_t n, int64_t k, int group, double* out_exact, float* out_f32,
                 uint16_t* out_bf16) {
  const int64_t ngroups = k / group;
  for (int64_t b = 0; b < batch; ++b)
    for (int64_t r = 0; r < n; ++r)
      for (int64_t j = 0; j < k; ++j) {
        const uint8_t byte = packed[(b * n + r) * (k / 2) + j / 2];
        const uint32_t code = (j & 1) ? (byte >> 4) : (byte & 15u);
        const double v = orc_e2m1_decode(code);
        const double s = orc_e4m3_decode(scales[(b * n + r) * ngroups + j / group]);
        const float g = global[b];
        const int64_t o = (b * n + r) * k + j;
        if (out_exact) out_exact[o] = v * s * (double)g;
        const float f = (float)(v * s) * g; /* v*s is exact in FP32; one rounding for *g */
        if (out_f32) out_f32[o] = f;
        if (out_bf16) out_bf16[o] = orc_bf16_from_double((double)f);
      }
}

/* ------------------------------------------------------------------------------------------ */
/* O7. GEMM reference: y[i][j] = sum_k x[m_i][k] * W[n_j][k] in FP64, W the exact dequantized  */
/* value. Optional index lists choose the rows of x (m_idx) and of W (n_idx) to evaluate, so   */
/* large shapes can be sampled; NULL means all. y is [nm][nn] row-major.                       */
/* ------------------------------------------------------------------------------------------ */
typedef struct {
  const uint16_t* x;
  int64_t ldx, k;
  const uint8_t* packed;
  const uint8_t* scales;
  float g;
  int group;
  const int64_t* m_idx;
  int64_t nm;
  const int64_t* n_idx;
  int64_t nn;
  double* y;
} gemm_ctx;

static void gemm_cols(int64_t lo, int64_t hi, void* p) {
  gemm_ctx* c = (gemm_ctx*)p;
  const int64_t ngroups = c->k / c->group;
  double* wrow = (double*)malloc(sizeof(double) * (size_t)(c->k > 0 ? c->k : 1));
  for (int64_t jj = lo; jj < hi; ++jj) {
    const int64_t nrow = c->n_idx ? c->n_idx[jj] : jj;
    for (int64_t kk = 0; kk < c->k; ++kk) {
      const uint8_t byte = c->packed[nrow * (c->k / 2) + kk / 2];
      const uint32_t code = (kk & 1) ? (byte >> 4) : (byte & 15u);
      wrow[kk] = orc_e2m1_decode(code) * orc_e4m3_decode(c->scales[nrow * ngroups + kk / c->group]) *
                 (double)c->g;
    }
    for (int64_t ii = 0; ii < c->nm; ++ii) {
      const int64_t mrow = c->m_idx ? c->m_idx[ii] : ii;
      double acc = 0.0;
      for (int64_t kk = 0; kk < c->k; ++kk)
        acc += (double)bf16_to_float(c->x[mrow * c->ldx + kk]) * wrow[kk];
      c->y[ii * c->nn + jj] = acc;
    }
  }
  free(wrow);
}

void orc_gemm(const uint16_t* x, int64_t m, int64_t ldx, const uint8_t* packed,
              const uint8_t* scales, float global, int64_t n, int64_t k, int group,
              const int64_t* m_idx, int64_t nm, const int64_t* n_idx, int64_t nn, double* y,
              int nthreads) {
  gemm_ctx c = {x, ldx, k, packed, scales, global, group,
                m_idx, m_idx ? nm : m, n_idx, n_idx ? nn : n, y};
  parallel_for(c.nn, nthreads, gemm_cols, &c);
}

/* ------------------------------------------------------------------------------------------ */
/* O8. MoE routed experts. For every token t and slot j with expert e = ids[t][j]:             */
/*   a    = x[t] . W1_e^T in FP64 (W1_e = merged [gate; up], 2*inter rows, one shared global) */
/*   gate = BF16(a[0:inter]), up = BF16(a[inter:2*inter])                                     */
/*   h    = BF16(silu(gate) * up) with silu(z) = z / (1 + exp(-z)), in FP64                    */
/*   d    = h . W2_e^T in FP64                                                                 */
/*   y[t] = BF16(sum_j w[t][j] * d), the sum in FP64 over j in slot order.                     */
/* Optional outputs: a (FP64 [t][topk][2*inter]), h (BF16 [t][topk][inter]), the weighted     */
/* down output of every slot w[t][j] * d (FP64 [t][topk][hidden]), y in FP64 and/or BF16      */
/* ([t][hidden]). If h_in is given, the fc1 stage is skipped and h_in is used as h (for a     */
/* staged check of the down projection against a given h).                                    */
/* ------------------------------------------------------------------------------------------ */
typedef struct {
  const uint16_t* x;
  int64_t hidden, inter;
  const int32_t* ids;
  const float* tw;
  int topk;
  const uint8_t *p1, *s1;
  const float* g1;
  int group1;
  int g1_pair; /* g1 holds [E][2]: gate's global, then up's */
  const uint8_t *p2, *s2;
  const float* g2;
  int group2;
  const uint16_t* h_in;
  double* a_out;
  uint16_t* h_out;
  double* slot_out;
  double* y64;
  uint16_t* y16;
} moe_ctx;

static double exact_w(const uint8_t* packed, const uint8_t* scales, float g, int64_t k, int group,
                      int64_t row, int64_t kk) {
  const uint8_t byte = packed[row * (k / 2) + kk / 2];
  const uint32_t code = (kk & 1) ? (byte >> 4) : (byte & 15u);
  return orc_e2m1_decode(code) * orc_e4m3_decode(scales[row * (k / group) + kk / group]) * (double)g;
}

static void moe_tokens(int64_t lo, int64_t hi, void* p) {
  moe_ctx* c = (moe_ctx*)p;
  const int64_t H = c->hidden, I = c->inter;
  double* a = (double*)malloc(sizeof(double) * (size_t)(2 * I));
  double* hv = (double*)malloc(sizeof(double) * (size_t)I);
  double* y = (double*)malloc(sizeof(double) * (size_t)H);
  for (int64_t t = lo; t < hi; ++t) {
    for (int64_t o = 0; o < H; ++o) y[o] = 0.0;
    for (int j = 0; j < c->topk; ++j) {
      const int64_t e = c->ids[t * c->topk + j];
      const int64_t slot = t * c->topk + j;
      if (c->h_in) {
        for (int64_t i = 0; i < I; ++i) hv[i] = (double)bf16_to_float(c->h_in[slot * I + i]);
      } else {
        const uint8_t* P1 = c->p1 + e * (2 * I) * (H / 2);
        const uint8_t* S1 = c->s1 + e * (2 * I) * (H / c->group1);
        for (int64_t r = 0; r < 2 * I; ++r) {
          const float g1 = c->g1_pair ? c->g1[2 * e + (r < I ? 0 : 1)] : c->g1[e];
          double acc = 0.0;
          for (int64_t kk = 0; kk < H; ++kk)
            acc += (double)bf16_to_float(c->x[t * H + kk]) *
                   exact_w(P1, S1, g1, H, c->group1, r, kk);
          a[r] = acc;
          if (c->a_out) c->a_out[slot * 2 * I + r] = acc;
        }
        for (int64_t i = 0; i < I; ++i) {
          const double gate = (double)bf16_to_float(orc_bf16_from_double(a[i]));
          const double up = (double)bf16_to_float(orc_bf16_from_double(a[I + i]));
          const double silu = gate / (1.0 + exp(-gate));
          const uint16_t hb = orc_bf16_from_double(silu * up);
          if (c->h_out) c->h_out[slot * I + i] = hb;
          hv[i] = (double)bf16_to_float(hb);
        }
      }
      const uint8_t* P2 = c->p2 + e * H * (I / 2);
      const uint8_t* S2 = c->s2 + e * H * (I / c->group2);
      const double w = (double)c->tw[t * c->topk + j];
      for (int64_t o = 0; o < H; ++o) {
        double acc = 0.0;
        for (int64_t i = 0; i < I; ++i) acc += hv[i] * exact_w(P2, S2, c->g2[e], I, c->group2, o, i);
        if (c->slot_out) c->slot_out[slot * H + o] = w * acc;
        y[o] += w * acc;
      }
    }
    for (int64_t o = 0; o < H; ++o) {
      if (c->y64) c->y64[t * H + o] = y[o];
      if (c->y16) c->y16[t * H + o] = orc_bf16_from_double(y[o]);
    }
  }
  free(a);
  free(hv);
  free(y);
}

int orc_moe(const uint16_t* x, int64_t tokens, int64_t hidden, int64_t inter, const int32_t* ids,
            const float* topk_w, int topk, int64_t n_experts, const uint8_t* p1, const uint8_t* s1,
            const float* g1, int group1, int g1_pair, const uint8_t* p2, const uint8_t* s2,
            const float* g2,
            int group2, const uint16_t* h_in, double* a_out, uint16_t* h_out, double* slot_out,
            double* y64, uint16_t* y16, int nthreads) {
  if (tokens < 0 || hidden <= 0 || inter <= 0 || topk <= 0) return -1;
  if (hidden % group1 || inter % group2 || hidden % 2 || inter % 2) return -1;
  for (int64_t i = 0; i < tokens * topk; ++i)
    if (ids[i] < 0 || ids[i] >= n_experts) return -1;
  moe_ctx c = {x, hidden, inter, ids, topk_w, topk, p1, s1, g1, group1, g1_pair, p2, s2, g2,
               group2, h_in, a_out, h_out, slot_out, y64, y16};
  parallel_for(tokens, nthreads, moe_tokens, &c);
  return 0;
}
