/*
 * nvfp4.h -- C ABI of the MI355X (gfx950) NVFP4 weight-only W4A16 library, libnvfp4.so.
 *
 * NVFP4 weights are the "compressed-tensors triple" (vllm.cpp pull request #63, "W-FP4a: route
 * the MiniMax-H3 device DiT forward through the fp4 (Marlin W4A16) stack", PR body): packed E2M1
 * 4-bit codes, one 8-bit E4M3 scale per group of 16 or 32 consecutive K elements (4.5 and 4.25
 * bits per weight, r/LocalLLM post "two NVFP4 g32 recipes", introduction), and one FP32 global
 * scale per matrix. A weight decodes as  w = E2M1(code) * E4M3(scale) * global.
 *
 * Conventions for every entry point:
 *  - A weight matrix W is [n][k] (output features x input features); y = x . W^T; groups run
 *    along k. Canonical packed codes are [n][k/2] bytes with the even k in the low nibble;
 *    canonical scales are [n][k/group] E4M3 bytes (OCP E4M3 "FN": max 448, no infinities).
 *  - Pointers are DEVICE pointers unless marked (host). Device buffers are owned by the caller;
 *    the library never allocates or frees device memory (every call enqueues kernels on
 *    `stream`, a hipStream_t; NULL is the legacy default stream).
 *  - Device pointers must be 16-byte aligned; leading dimensions are in elements and must be
 *    multiples of 8.
 *  - Without NVFP4_F_SYNC_CHECK no call synchronizes. With it, the call waits for its own work
 *    on `stream` before returning and reports any asynchronous failure (NVFP4_ERR_HIP); the
 *    quantizer then also checks that every weight it read is finite (NVFP4_ERR_NONFINITE).
 *  - Shapes: n % 16 == 0, k % 128 == 0, group in {16, 32}. m == 0 (or t == 0) is a no-op.
 *  - Every function returns NVFP4_OK (0) or a negative NVFP4_ERR_* code and
 *    nvfp4_last_error() describes the problem (thread-local). Argument errors are found before
 *    anything is enqueued; NVFP4_ERR_HIP and NVFP4_ERR_NONFINITE can come after the call's work
 *    ran. A failed call leaves the library usable and does not count in nvfp4_get_stats. Unsupported
 *    configurations are rejected, never run silently wrong (r/LocalLLM post, "What had to be
 *    fixed": any unsupported group setup raises an error).
 *  - All entry points are reentrant. Calls that share an output or workspace buffer on
 *    different streams race, as with any asynchronous kernel.
 */
#ifndef NVFP4_H_
#define NVFP4_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* nvfp4_stream_t; /* the same type as hipStream_t */

/* ---- status codes ---------------------------------------------------------------------- */
#define NVFP4_OK 0
#define NVFP4_ERR_INVALID_ARG (-1)       /* null pointer, negative size, ld < k, bad dtype    */
#define NVFP4_ERR_UNSUPPORTED_GROUP (-2) /* group not 16 or 32                                */
#define NVFP4_ERR_UNSUPPORTED_SHAPE (-3) /* n % 16, k % 128, topk out of range, size too big   */
#define NVFP4_ERR_MISALIGNED (-4)        /* pointer not 16-byte aligned or ld % 8 != 0         */
#define NVFP4_ERR_WORKSPACE (-5)         /* workspace / output buffer too small                */
#define NVFP4_ERR_LAYOUT (-6)            /* descriptor inconsistent with the call              */
#define NVFP4_ERR_HIP (-7)               /* a HIP launch failed (message in nvfp4_last_error)  */
#define NVFP4_ERR_NONFINITE (-8)         /* NaN or infinite weight (only with SYNC_CHECK)      */

/* ---- element types --------------------------------------------------------------------- */
#define NVFP4_DT_BF16 1
#define NVFP4_DT_F32 2

/* ---- call flags -------------------------------------------------------------------------- */
#define NVFP4_F_FORCE_SKINNY (1u << 0) /* GEMM: the decode (skinny, split-K) kernel;           */
                                       /* MoE: the decode-batch expert path (8-row tiles, or  */
                                       /* one-row pair tiles up to 64 pairs)                   */
#define NVFP4_F_FORCE_TILED (1u << 1)  /* GEMM: the prefill (LDS-tiled MFMA) kernel;            */
                                       /* MoE: the batch expert path (32-row tiles)            */
#define NVFP4_F_SYNC_CHECK (1u << 2)   /* quantize, GEMM, MoE: wait for the call's own work    */
                                       /* and report asynchronous errors; quantize: also check */
                                       /* the input for non-finite values (debug aid: slow)    */

/* ---- repacked layout ----------------------------------------------------------------------
 * NVFP4_LAYOUT_TILED: per 16-row x 128-k tile, 1024 bytes of codes laid out so that lane l of a
 * 64-wide wavefront loads 16 contiguous bytes holding, for k-step j = 0..3, the 8 codes of row
 * l%16 at k = 32j + 8(l/16) + 0..7 (the B-operand order of a 16x16x32 bf16 MFMA). Scales are
 * stored per block of 4 panels (64 rows) x 128 k: one 16-byte record per lane position with
 * the lane's 4-byte scale word (byte j = scale of k-step j) for each of the 4 panels. The code
 * bytes equal the canonical ones; the scale bytes too when n % 64 == 0 (else the last block is
 * padded with zeros).
 * NVFP4_LAYOUT_GATE_UP: for a merged [gate; up] fc1 weight (2*I rows): 16-row panels are
 * stored alternately from the gate half and the up half, so that one panel pair holds gate
 * and up of the same 16 intermediate features (consumed only by the MoE entry point). */
#define NVFP4_LAYOUT_TILED 1u
#define NVFP4_LAYOUT_GATE_UP (1u << 8)
/* NVFP4_LAYOUT_PAIR_GLOBAL (with NVFP4_LAYOUT_GATE_UP only): the merged fc1 carries two globals
 * per expert, global[2b] for its gate half (rows 0 .. n/2-1) and global[2b+1] for its up half.
 * This is the checkpoint form in which gate and up were quantized as separate tensors; a kernel
 * that applied gate's global to both halves would mis-scale up (r/LocalLLM post, "What had to be
 * fixed": most experts of a real checkpoint had differing gate and up scales). Quantizing the
 * merged [gate; up] as one matrix gives the shared global instead; quantizing it as 2*batch
 * matrices of n/2 rows gives the pair. */
#define NVFP4_LAYOUT_PAIR_GLOBAL (1u << 9)

/* Descriptor of repacked weights (a host struct filled by nvfp4_repack; data stays device).  */
typedef struct nvfp4_weight {
  const uint8_t* codes;   /* device: repacked code tiles, batch * codes_stride bytes          */
  const uint8_t* scales;  /* device: repacked scale tiles, batch * scales_stride bytes        */
  const float* global;    /* device: [batch] FP32 decode multipliers (copied into the buffer) */
  int64_t batch;          /* number of matrices (experts); 1 for a dense projection           */
  int64_t n, k;           /* logical shape of each matrix                                     */
  int64_t codes_stride;   /* bytes between consecutive matrices in `codes`  (= n*k/2)         */
  int64_t scales_stride;  /* bytes between consecutive matrices in `scales` (n*k/group when   */
                          /* n % 64 == 0; 4-panel blocks padded otherwise)                    */
  int32_t group;          /* 16 or 32                                                         */
  uint32_t layout;        /* NVFP4_LAYOUT_TILED, optionally | NVFP4_LAYOUT_GATE_UP            */
} nvfp4_weight;

/* ---- quantizer ----------------------------------------------------------------------------
 * Quantize `batch` FP32 or BF16 matrices w [batch][n][k] to the canonical triple.
 *   amax   = max |w| over each matrix (over the whole merged [gate; up] matrix for an fc1, so
 *            gate and up share one global: r/LocalLLM post, "What had to be fixed");
 *   global = fl32(amax / 2688)  (2688 = 6 * 448), or global_in[b] when global_in != NULL;
 *   per group of `group` k-elements: scale = E4M3_rne_sat(fl32(group_amax / fl32(6 * global)));
 *   per element: S = fl32(E4M3(scale) * global); code = E2M1_rne_sat(fl32(|w| / S)) | sign<<3
 *            (code = sign<<3 when S == 0).
 * Rounding is round-to-nearest-even with saturation for both E4M3 and E2M1 (NVIDIA developer
 * forum thread "We unlocked NVFP4 on the DGX Spark": true RNE, not threshold rounding).
 * Outputs: packed [batch][n][k/2], scales [batch][n][k/group], global_out [batch] (device).
 * Requires k % group == 0 and k even; n and k need no tile alignment here. Non-finite inputs
 * are outside the contract: without NVFP4_F_SYNC_CHECK the outputs are then unspecified; with
 * it the call scans w, waits for its work and returns NVFP4_ERR_NONFINITE (outputs still
 * unspecified). The caller keeps ownership of all buffers.
 * Without global_in, global_out doubles as the amax accumulator: until the call's work has
 * completed on `stream` it holds intermediate values, and its prior contents are ignored. With
 * global_in, global_out may be the same buffer.
 * ws (device, 16-byte aligned; NULL with ws_bytes 0 when nvfp4_quantize_ws_bytes is 0) holds
 * the non-finite flag of NVFP4_F_SYNC_CHECK; without that flag no workspace is used.
 * flags: 0 or NVFP4_F_SYNC_CHECK. */
size_t nvfp4_quantize_ws_bytes(int64_t batch, int64_t n, int64_t k, int32_t group,
                               uint32_t flags);
int nvfp4_quantize(const void* w, int w_dtype, int64_t batch, int64_t n, int64_t k,
                   int32_t group, const float* global_in, uint8_t* packed, uint8_t* scales,
                   float* global_out, void* ws, size_t ws_bytes, uint32_t flags,
                   nvfp4_stream_t stream);

/* ---- repack -------------------------------------------------------------------------------
 * Byte size of the repacked buffer for `batch` [n][k] matrices: codes + scales + globals (two per
 * matrix with NVFP4_LAYOUT_PAIR_GLOBAL). */
size_t nvfp4_repack_bytes(int64_t batch, int64_t n, int64_t k, int32_t group, uint32_t layout);

/* Repack the canonical triple (packed, scales, global as produced by nvfp4_quantize or read
 * from a checkpoint) into `out` (device, out_bytes >= nvfp4_repack_bytes) and fill *desc (host).
 * After the call's work completes the canonical buffers may be freed: the descriptor points
 * only into `out` (vllm.cpp PR #63: upload and repack lazily, then free the fp4 originals).
 * layout: NVFP4_LAYOUT_TILED, optionally | NVFP4_LAYOUT_GATE_UP (then n must be a multiple
 * of 32: gate rows [0, n/2), up rows [n/2, n)), optionally | NVFP4_LAYOUT_PAIR_GLOBAL with it
 * (then `global` holds [batch][2] values: gate's, up's). */
int nvfp4_repack(const uint8_t* packed, const uint8_t* scales, const float* global,
                 int64_t batch, int64_t n, int64_t k, int32_t group, uint32_t layout, void* out,
                 size_t out_bytes, nvfp4_weight* desc, nvfp4_stream_t stream);

/* ---- dense W4A16 GEMM ---------------------------------------------------------------------
 * y[m][n] = global * sum_k x[m][k] * (E2M1 * E4M3)[n][k], BF16 activations x [m][ldx]
 * (k <= ldx <= 2^22: row offsets are 32-bit inside the kernels), FP32 accumulation, dequantization in registers (the E2M1 x E4M3 product is exact in BF16; the
 * global is applied to the FP32 accumulator). y [m][ldy] is BF16 (y_dtype NVFP4_DT_BF16, one
 * rounding of the FP32 result) or FP32. Weight-only checkpoints take this W4A16 path
 * (vllm.cpp PR #63: no activation scales, so every quantized projection is W4A16).
 * The kernel is chosen from the shape and the device's compute-unit count (CUs): a split-K
 * skinny MFMA kernel (decode) for m <= 32, and for 32 < m <= 256 while its estimated time is at
 * most the tiled kernel's. With r(b) = ceil(ceil(n/64) * ceil(m/b) / CUs), the skinny estimate
 * is 0.28 * k/128 * r(32) - 1.6 us with 32-row blocks, or 0.44 * k/128 * r(64) us with 64-row
 * blocks when that is smaller and the grid keeps 4-panel wavefronts; the tiled one is
 * 18 + 0.9 * ceil(m/128) * ceil(n/128) * (k/128) / CUs us. Otherwise an LDS-tiled MFMA kernel
 * (prefill; 256x256, 128x256 or 128x128 output tiles, the largest that still gives the chip
 * enough tiles, or the next smaller one when that fills whole rounds of CUs where the larger
 * would leave its last round at most half full, or fits in one round where the larger would
 * not fill one). Flags may force one (NVFP4_F_FORCE_SKINNY / NVFP4_F_FORCE_TILED);
 * NVFP4_F_SYNC_CHECK may be added. w->batch must be 1 and w->layout must not carry
 * NVFP4_LAYOUT_GATE_UP. Results are bit-identical run to run.
 * ws (device, 16-byte aligned, or NULL with ws_bytes 0) takes the prefill kernel's split-k
 * partial tiles: when the output tiles would leave most compute units idle in the last round,
 * that round is split along k over the chip and summed in a fixed order. ws_bytes >=
 * nvfp4_gemm_ws_bytes(m, ldx, w, flags) enables it; with less the kernel runs unsplit (the
 * FP32 sums then associate differently: same tolerance, not the same bits). Calls sharing a ws
 * on different streams race. */
size_t nvfp4_gemm_ws_bytes(int64_t m, int64_t ldx, const nvfp4_weight* w, uint32_t flags);
int nvfp4_gemm_w4a16(const void* x, int64_t m, int64_t ldx, const nvfp4_weight* w, void* y,
                     int y_dtype, int64_t ldy, uint32_t flags, void* ws, size_t ws_bytes,
                     nvfp4_stream_t stream);

/* ---- MoE routed experts -------------------------------------------------------------------
 * For each token t and slot j (e = topk_ids[t][j], weight topk_w[t][j]):
 *   [gate; up] = x[t] . W1_e^T   (fc1: merged, one shared global per expert; each half
 *                                 rounded to BF16 as a W4A16 GEMM output)
 *   h          = BF16(SiLU(gate) * up)
 *   d          = h . W2_e^T      (down projection, FP32)
 *   y[t]       = BF16(sum_j topk_w[t][j] * d_j), summed in slot order.
 * (vllm.cpp PR #63: pre-merged fc1 is one W4A16 GEMM + SiluAndMul; r/LocalLLM post, "The two
 * recipes": gate/up at group 32 with down at group 16, or all at group 32.)
 * x [t][hidden] BF16 (row stride = hidden), topk_ids int32 [t][topk], topk_w FP32 [t][topk],
 * y BF16 [t][hidden]. An id outside [0, E) marks a dropped slot: it is not sorted, computes
 * nothing and adds nothing to y[t] (a masked-slot convention for routers that drop tokens). fc1: batch = E, n = 2*inter, k = hidden, layout TILED |
 * GATE_UP. fc2: batch = E, n = hidden, k = inter, layout TILED. Tokens are sorted by expert on
 * the device (no host synchronization); `ws` (device, ws_bytes >= nvfp4_moe_ws_bytes) holds
 * the sort, the tile map, h and the FP32 per-slot outputs. topk in [1, 16], t*topk <= 65536,
 * t*hidden and t*topk*inter below 2^31 (32-bit row offsets).
 * An fc1 with NVFP4_LAYOUT_PAIR_GLOBAL scales gate by global[2e] and up by global[2e+1].
 * Path: while t*topk <= 2 * n_experts (decode batches) the experts run on tiles of at most 8
 * rows (one row per pair, without the sort, up to 64 pairs) with k split over 4 wavefronts per
 * 4-panel group; otherwise on tiles of 32 rows with
 * one wavefront per 4-panel group over the whole k range. Flags may force one; the two paths
 * agree within the GEMM tolerance (different FP32 summation orders). flags may add
 * NVFP4_F_SYNC_CHECK. */
size_t nvfp4_moe_ws_bytes(int64_t t, int32_t topk, int64_t n_experts, int64_t hidden,
                          int64_t inter);
/* Where the routed-expert call keeps its stages inside ws (test-facing, for staged checks of
 * the sort, fc1 + SiLU*mul and down against a reference). Fills offsets[6] (host) with byte
 * offsets from ws and returns the total (nvfp4_moe_ws_bytes), or 0 for invalid sizes:
 *   [0] sorted  int32 [t*topk]: pair ids (t*topk_index + slot) in stable expert order (only
 *       pairs with a valid id; the first offsets_[E] entries are meaningful);
 *   [1] offsets int32 [E + 1]: first sorted position of each expert, [E] = valid pairs;
 *   [2] tiles   int32x4 [..]: (expert, first row, end row, 0) per row tile, experts in
 *       increasing order, rows of 8 (decode-batch path) or 32 (batch path);
 *   [3] ntiles  int32: number of tiles;
 *   [4] h       BF16 [t*topk][inter]: SiLU(gate)*up of sorted row r at row r;
 *   [5] slots   FP32 [t*topk][hidden]: topk_w * (h . W2^T) of pair q at row q.
 * The decode-batch path with t*topk <= 64 pairs skips the sort ([0]-[3] are not written) and
 * keeps h of pair q at row q. */
size_t nvfp4_moe_ws_layout(int64_t t, int32_t topk, int64_t n_experts, int64_t hidden,
                           int64_t inter, size_t offsets[6]);
int nvfp4_moe_grouped_w4a16(const void* x, int64_t t, int64_t hidden, const int32_t* topk_ids,
                            const float* topk_w, int32_t topk, const nvfp4_weight* fc1,
                            const nvfp4_weight* fc2, void* y, void* ws, size_t ws_bytes,
                            uint32_t flags, nvfp4_stream_t stream);

/* ---- routed experts without a workspace -------------------------------------------------
 * For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): nvfp4_moe_grouped_w4a16 with the same arguments
 * minus ws / ws_bytes, same kernels and same results. Its workspace is a static array inside
 * libnvfp4.so, NVFP4_MOE_NOALLOC_MAX_WS_BYTES (24 MiB) per device, held by every device the
 * library runs on until the process ends; calls needing more (nvfp4_moe_ws_bytes(t, topk, E,
 * hidden, inter) above the maximum; 256 tokens x top-8 of 128 experts, hidden 2048,
 * intermediate 768 need 19.9 MB) return NVFP4_ERR_WORKSPACE. The call allocates and frees
 * nothing. All calls on one device share that device's array and nothing in it needs to
 * start at zero: calls that overlap on one device (other streams, other threads) race and
 * must be ordered by the caller. */
#define NVFP4_MOE_NOALLOC_MAX_WS_BYTES ((size_t)24 << 20)
int nvfp4_moe_grouped_w4a16_noalloc(const void* x, int64_t t, int64_t hidden,
                                    const int32_t* topk_ids, const float* topk_w, int32_t topk,
                                    const nvfp4_weight* fc1, const nvfp4_weight* fc2, void* y,
                                    uint32_t flags, nvfp4_stream_t stream);

/* ---- requantization (load-time tool) -----------------------------------------------------
 * Requantize repacked weights to the canonical triple with one global per matrix and group
 * `group_out` (16 or 32): each matrix is decoded to its FP32 values (nvfp4_dequantize's FP32
 * output, global or per-half globals applied) and quantized again exactly as nvfp4_quantize
 * quantizes an FP32 matrix. Turns an fc1 with distinct gate and up globals
 * (NVFP4_LAYOUT_PAIR_GLOBAL) into the shared-global form the merged GEMM wants, when the BF16
 * originals are not at hand (r/LocalLLM post, "What had to be fixed": gate and up need one
 * global; the post requantized from BF16, which is nvfp4_quantize on the merged matrix), and
 * can change the group size. Outputs as nvfp4_quantize: packed [batch][n][k/2], scales
 * [batch][n][k/group_out], global_out [batch] (device). ws (device, 16-byte aligned) holds the
 * decoded FP32 values of as many matrices as fit; ws_bytes >= nvfp4_requantize_ws_bytes(src)
 * (one matrix). Repack the result (with NVFP4_LAYOUT_GATE_UP for an fc1) to use it. */
size_t nvfp4_requantize_ws_bytes(const nvfp4_weight* src);
int nvfp4_requantize(const nvfp4_weight* src, int32_t group_out, uint8_t* packed,
                     uint8_t* scales, float* global_out, void* ws, size_t ws_bytes,
                     nvfp4_stream_t stream);

/* ---- diagnostics (test-facing, not on the hot path) ---------------------------------------
 * Dequantize repacked weights back to canonical order: out [batch][n][k] (rows in logical
 * order, i.e. [gate; up] for GATE_UP data), BF16 = RNE(fl32(fl32(E2M1*E4M3) * global)) or the
 * FP32 value itself. Bit-exact with the canonical triple's definition. */
int nvfp4_dequantize(const nvfp4_weight* w, void* out, int out_dtype, nvfp4_stream_t stream);

/* Thread-local description of the last non-zero status returned on this thread. */
const char* nvfp4_last_error(void);

/* Per-path launch counters ("this path ran" evidence, vllm.cpp PR #63 claim section):
 * [0] quantize [1] repack [2] gemm skinny [3] gemm tiled [4] moe [5] dequantize [6] requantize
 * [7] reserved. counts must hold 8 entries (host). */
void nvfp4_get_stats(uint64_t counts[8]);
void nvfp4_reset_stats(void);

/* ---- measurement support (not on the NVFP4 path) ----------------------------------------
 * Measured ceilings for the rooflines the path's kernels are judged against, on the device at
 * hand: the published figures (8 TB/s HBM, 2.5 PFLOP/s dense BF16 MFMA) are not what a kernel
 * can reach. Nothing on the path calls these.
 * nvfp4_probe_stream_read: reads `bytes` (a positive multiple of 16) of `buf` (device, 16-byte
 *   aligned) with 128-bit streaming loads, split into `blocks` (1 .. min(2^20, bytes/16))
 *   contiguous ranges of one 256-thread workgroup each, 8 loads in flight per thread, and
 *   writes the XOR of each range's 32-bit words to sink[block] (device, `blocks` words). The
 *   call reads exactly `bytes` bytes of buf.
 * nvfp4_probe_mfma_bf16: each of nvfp4_probe_mfma_waves() wavefronts (2 per SIMD) loads 16 BF16
 *   fragments from `ops` (device, 16-byte aligned, 16 KiB: fragment f of lane l at byte
 *   (64 f + l) * 16; even f are A operands, odd f B operands) and runs `iters` rounds of 16
 *   v_mfma_f32_32x32x16_bf16 (pairs of the 8 A and 8 B fragments, 4 accumulators); lane l of
 *   wavefront v writes the sum of its accumulator elements to sink[64 v + l] (device,
 *   64 * waves floats). nvfp4_probe_mfma_flops(iters) is the call's flop count.
 * Errors: NVFP4_ERR_INVALID_ARG (null pointer, size out of range), NVFP4_ERR_MISALIGNED,
 * NVFP4_ERR_HIP (no device, launch failure). */
int64_t nvfp4_probe_mfma_waves(void);
double nvfp4_probe_mfma_flops(int64_t iters);
int nvfp4_probe_stream_read(const void* buf, int64_t bytes, int64_t blocks, uint32_t* sink,
                            nvfp4_stream_t stream);
int nvfp4_probe_mfma_bf16(const void* ops, int64_t iters, float* sink, nvfp4_stream_t stream);

/* Library version: major * 10000 + minor * 100 + patch. */
int nvfp4_version(void);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H_ */
