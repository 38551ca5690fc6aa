/* nvfp4.h — C ABI of the NVFP4 block-scaled linear library for AMD MI355X (gfx950).
 *
 * The operation. An NVFP4 weight is an [N][K] matrix stored as it ships in ModelOpt /
 * FP4-Local checkpoints (bloomery issue #565, "NVIDIA FP4-Local checkpoints on DGX
 * Spark (TP=1, TP=2): format, model and speed plan in rounds", section 4 "Round 1",
 * PRs #489 and #490): U8 bytes holding two 4-bit E2M1 codes, one F8_E4M3 scale per
 * 16 consecutive elements along K ("group-16"; Rocket engineering log, entry
 * "Rank-local E256 MoE misses the Qwen K1 and K4 step budgets", setup table), and
 * one fp32 tensor scale for the whole matrix. Element (n, k) has the value
 *     e2m1(code[n][k]) * e4m3(scale[n][k/16]) * ts.
 * The linear layer computes y[m][n] = sum_k x[m][k] * w(n, k) in fp32.
 *
 * Layouts (all row-major, all buffers caller-owned device memory):
 *   codes   [N][K/2]  uint8, byte j of a row holds k = 2j in its low nibble and
 *                      k = 2j+1 in its high nibble;
 *   scales  [N][K/16] uint8, OCP E4M3FN bytes (bias 7, max 448, 0x7F/0xFF = NaN);
 *   ts      [1]       fp32 (a device pointer, so a caller can keep it resident);
 *   BF16 activations  uint16 bit patterns [M][ldx];
 *   NVFP4 activations codes [M][K/2] + scales [M][K/16] + one fp32 ts per row [M].
 * E2M1 codes: bit 3 = sign, bits 0..2 index {0, 0.5, 1, 1.5, 2, 3, 4, 6}.
 *
 * Conventions shared by every entry point:
 *   - Ownership: the library never allocates, frees or synchronizes. All pointers are
 *     device memory owned by the caller, except `workspace_bytes` (host).
 *   - Streams: all work is enqueued on `stream` (a hipStream_t; NULL = the default
 *     stream). Calls return as soon as the work is enqueued.
 *   - Argument errors are detected on the host before anything is enqueued; the call
 *     then returns a non-zero status and enqueues nothing (misaligned or too-large
 *     inputs are refused by name, as the pages' engine refuses misaligned vector views
 *     and unchecked integer conversions: issue #565 section 10, PRs #520 and #984).
 *   - Data faults are reported asynchronously: when `faults` is non-NULL the kernels
 *     OR bits of NVFP4_FAULT_* into that device word. Outputs are undefined when a
 *     call returns a non-OK status or sets a fault bit.
 *   - Check mode (flags & NVFP4_F_CHECK, nvfp4_linear and nvfp4_grouped_linear): before
 *     the product, the call scans its operands' data and ORs into *faults
 *       NVFP4_FAULT_NAN_SCALE  for an E4M3 scale byte that is NaN (0x7F or 0xFF) or a
 *                              tensor scale that is NaN or infinite (weight or NVFP4
 *                              activation operand; every expert of a grouped call);
 *       NVFP4_FAULT_NONFINITE  for a NaN or infinite BF16 activation value;
 *     (the pages' engine refuses NaN scale bytes and rows whose scaled values overflow,
 *     issue #565 section 10, PRs #597 and #710). The scan is separate launches on the
 *     same stream; without the flag nothing is scanned and the product kernels are the
 *     same as with it. Check mode needs a non-NULL `faults` (NVFP4_ERR_NULL otherwise).
 *     The product still runs: a NaN scale gives NaN in the outputs it touches.
 *   - The tensor scale is applied once, to the fp32 accumulator (the store scales by
 *     it, as the pages' prompt GEMM scales each slot by its expert's tensor scale:
 *     issue #565 section 4, PR #545).
 *   - Kernels keep no state between calls; results are deterministic (fixed
 *     reduction order, no floating-point atomics).
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum nvfp4_status {
  NVFP4_OK = 0,
  NVFP4_ERR_NULL = 1,      /* a required pointer is NULL */
  NVFP4_ERR_SHAPE = 2,     /* a size is <= 0, K % 32 != 0, a leading dimension is too
                              small, or a size does not fit the kernels' indices */
  NVFP4_ERR_ALIGN = 3,     /* a base pointer or leading dimension breaks the 16-byte
                              alignment a row needs (scales: 2 bytes) */
  NVFP4_ERR_ARG = 4,       /* an unknown enum value, or top_k / num_experts out of range */
  NVFP4_ERR_WORKSPACE = 5, /* workspace smaller than the size the call needs */
  NVFP4_ERR_LAUNCH = 6     /* the HIP runtime refused a kernel launch */
} nvfp4_status;

/* activation kinds */
enum { NVFP4_ACT_BF16 = 0, NVFP4_ACT_NVFP4 = 1, NVFP4_ACT_BF16_QUANTIZE = 2 };
/* quantizer input types and tensor-scale modes */
enum { NVFP4_IN_BF16 = 0, NVFP4_IN_F32 = 1 };
enum { NVFP4_TS_PER_ROW = 0, NVFP4_TS_PER_TENSOR = 1 };
/* grouped call: which x row a route reads, and what is written */
enum { NVFP4_ROWS_PER_TOKEN = 0, NVFP4_ROWS_PER_ROUTE = 1 };
enum { NVFP4_OUT_ROUTES = 0, NVFP4_OUT_SWIGLU_BF16 = 1, NVFP4_OUT_COMBINE = 2 };
/* OR'ed into out_mode of a grouped call: reuse the route grouping already in the workspace */
enum { NVFP4_OUT_REUSE_GROUPING = 0x100 };
/* fault bits */
enum { NVFP4_FAULT_NONFINITE = 1u, NVFP4_FAULT_BAD_ROUTE = 2u, NVFP4_FAULT_NAN_SCALE = 4u };
/* call flags (nvfp4_linear, nvfp4_grouped_linear) */
enum { NVFP4_F_CHECK = 1u };

/* Human-readable name of a status code (static storage). */
const char* nvfp4_status_string(int32_t status);

/* nvfp4_linear — y[m][n] = sum_k x[m][k] * w(n, k), fp32 accumulation, fp32 output.
 *
 * W4A16 (act_kind = NVFP4_ACT_BF16): x is BF16 bits [M][ldx] (ldx >= K, ldx % 8 == 0,
 *   x 16-byte aligned); x_scales and x_ts must be NULL. The activations BF16 times the
 *   exactly decoded weight e2m1*e4m3 (exact in BF16) accumulate in fp32; y = acc * ts.
 * W4A4 (act_kind = NVFP4_ACT_NVFP4): x is NVFP4 codes [M][K/2] (16-byte aligned),
 *   x_scales [M][K/16], x_ts [M] per-row tensor scales (as nvfp4_quantize_act writes
 *   them with NVFP4_TS_PER_ROW); ldx is ignored. Both operands are decoded exactly;
 *   y[m][n] = acc * (x_ts[m] * ts). (W4A16 and W4A4 variants: issue #565 section 4,
 *   PRs #682 and #687.)
 * W4A4 with in-call quantization (act_kind = NVFP4_ACT_BF16_QUANTIZE), for one row, M = 1
 *   and K <= 8192: x is BF16 as for W4A16; the row is quantized inside the call by the
 *   per-row rule of nvfp4_quantize_act (NVFP4_TS_PER_ROW) and multiplied as W4A4, bit for
 *   bit the result of nvfp4_quantize_act followed by the NVFP4_ACT_NVFP4 call, in one
 *   launch and with no stored codes (the activation quantization folded into the kernel
 *   that uses it, as the pages plan for their prompt kernels: issue #565 section 4,
 *   "Remaining Round 1 items"). Every workgroup quantizes the whole row, so for more rows
 *   the two calls are faster; they are refused here. x_scales and x_ts must be NULL. A row
 *   holding a NaN or Inf gives NaN outputs.
 * Weight: w_codes [N][K/2] (16-byte aligned), w_scales [N][K/16] (2-byte aligned),
 *   w_ts [1]. y [M][ldy] fp32, ldy >= N. K % 32 == 0.
 * M <= 16 streams the weight once for all rows (each weight byte is read once for all
 *   M rows, as the pages' multi-row MTP verify does: issue #565 section 4, PRs #808
 *   and #707); larger M runs the tiled matrix-core GEMM.
 * flags: 0 or NVFP4_F_CHECK (see "Check mode" above); faults: a device word or NULL
 *   (NULL only without NVFP4_F_CHECK); with NVFP4_ACT_BF16_QUANTIZE a non-finite row
 *   value is reported as NVFP4_FAULT_NONFINITE in check mode.
 * Errors: NVFP4_ERR_NULL, _SHAPE (also M != 1 or K > 8192 with NVFP4_ACT_BF16_QUANTIZE),
 *   _ALIGN, _ARG (unknown act_kind or flag bit), _LAUNCH. */
nvfp4_status nvfp4_linear(int32_t act_kind, const void* x, const uint8_t* x_scales,
                          const float* x_ts, int64_t ldx, int64_t M, int64_t N, int64_t K,
                          const uint8_t* w_codes, const uint8_t* w_scales, const float* w_ts,
                          float* y, int64_t ldy, uint32_t flags, uint32_t* faults,
                          void* stream);

/* nvfp4_quantize_act — quantize rows to NVFP4 on the device, bit-exactly by the rule
 *     ts      = amax / 2688            (2688 = 6 * 448; amax over the row or the tensor)
 *     ratio_b = (amax_b / 6) / ts      (0 when ts == 0; amax_b over the 16-block b)
 *     s_b     = E4M3_RNE(ratio_b)      (nearest, ties to even, saturating at 448)
 *     q_k     = x_k / (e4m3(s_b) * ts) (+-0 when that denominator is 0)
 *     code_k  = E2M1_RNE(q_k)          (nearest, ties to even, saturating at 6;
 *                                       the sign is the sign bit of q, so -0 -> 0x8)
 * each step one correctly rounded fp32 operation, left to right.
 * in_type NVFP4_IN_BF16: x is BF16 bits [M][ldx]; NVFP4_IN_F32: x is fp32 [M][ldx];
 *   ldx >= K, x rows 16-byte aligned.
 * ts_mode NVFP4_TS_PER_ROW: ts is [M] (one per row; the W4A4 activation form);
 *   NVFP4_TS_PER_TENSOR: ts is [1] (the weight form; ts[0] is also used as scratch
 *   while the call runs).
 * codes [M][K/2] (16-byte aligned), scales [M][K/16]. K % 32 == 0.
 * A NaN or Inf input sets NVFP4_FAULT_NONFINITE in *faults (when non-NULL); the pages'
 * quantizers refuse non-finite values (issue #565 section 10, PR #597).
 * Errors: NVFP4_ERR_NULL, _SHAPE, _ALIGN, _ARG, _LAUNCH. */
nvfp4_status nvfp4_quantize_act(int32_t in_type, const void* x, int64_t ldx, int64_t M,
                                int64_t K, int32_t ts_mode, uint8_t* codes, uint8_t* scales,
                                float* ts, uint32_t* faults, void* stream);

/* nvfp4_grouped_linear — the expert-grouped form for a routed MoE layer.
 *
 * E experts share one shape: w_codes [E][N][K/2], w_scales [E][N][K/16], w_ts [E].
 * T tokens each pick top_k distinct experts: topk_ids [T][top_k] int32 in [0, E).
 * Route r = t * top_k + j (token t, its j-th pick). Routes are grouped by expert
 * (a stable counting sort, expert-ascending), and each active expert's weight is
 * streamed once for all of its routes (issue #565 section 4, PR #808 and PR #740;
 * expert-first offsets as in the Rocket log entry "Rank-local E256 MoE ...").
 *
 * rows_mode NVFP4_ROWS_PER_TOKEN: x has T rows and route r reads row t;
 *           NVFP4_ROWS_PER_ROUTE: x has T*top_k rows and route r reads row r.
 * x: act_kind/x/x_scales/x_ts/ldx as in nvfp4_linear (NVFP4 rows hold one ts per x
 *    row), with act_kind NVFP4_ACT_BF16 or NVFP4_ACT_NVFP4 only: the in-call
 *    quantization NVFP4_ACT_BF16_QUANTIZE is refused here (NVFP4_ERR_ARG).
 * out_mode NVFP4_OUT_ROUTES: y is fp32 [T*top_k][N], row r = x_row(r) w_e^T * ts_e.
 *          NVFP4_OUT_SWIGLU_BF16: N even; y is BF16 bits [T*top_k][N/2], row r =
 *            bf16_rne(silu(g) * u) with g = h[0:N/2], u = h[N/2:N] of the route's fp32
 *            row h (SwiGLU rounded once to BF16, as the pages keep the down input in
 *            BF16 rounded to nearest even: issue #565 section 4, PR #914); h
 *            bit-equals the NVFP4_OUT_ROUTES row of the same call shape. silu(g) =
 *            g / (1 + e^-g) is evaluated with the hardware's exp2 and reciprocal (a few
 *            fp32 ulp), so a result is within one BF16 ulp of the correctly rounded one
 *            and equal to it almost everywhere.
 *          NVFP4_OUT_COMBINE: needs topk_w [T][top_k] fp32; y is fp32 [T][N],
 *            y[t] = sum over t's routes in ascending expert id of
 *            (topk_w[t][j] * ts_e) * (x_row(r) w_e^T), accumulated in fp32 in that order
 *            (the ordered combine with the tensor scale folded into the router weight:
 *            Rocket log entry "The expert split decodes the same tokens; ...", section
 *            "Why rows and not partial sums").
 * topk_w is ignored unless out_mode is NVFP4_OUT_COMBINE.
 * NVFP4_OUT_REUSE_GROUPING (OR'ed into NVFP4_OUT_COMBINE only): the workspace already
 *   holds the route grouping of these topk_ids, left there by an earlier grouped call
 *   on the same stream with the same topk_ids, T, top_k and num_experts (the gate_up
 *   call of the same layer); the grouping is not recomputed. The grouping occupies the
 *   same leading bytes of the workspace in every output form, so one workspace sized
 *   for the combine serves both calls. Bad routes were reported by the earlier call.
 *   Passing stale topk_ids or a different workspace gives unspecified (but in-bounds)
 *   results. Any other out_mode with this bit is NVFP4_ERR_ARG.
 * Decode-sized batches stream each active expert's weight once for all its routes;
 *   prompt-sized ones (routes averaging >= 32 per active expert) run MFMA tiles of one
 *   expert's routes (the pages' expert-grouped prompt GEMM, each expert read once per
 *   batch: issue #565 section 4, PR #740).
 * workspace: device scratch (the route grouping, and the fp32 per-route rows for
 *   NVFP4_OUT_COMBINE); pass workspace = NULL to receive the needed size in
 *   *workspace_bytes (nothing is enqueued); otherwise *workspace_bytes is its size.
 *   Its contents need no initialisation: every byte the call reads it writes first.
 * flags: 0 or NVFP4_F_CHECK (see "Check mode" above; scans every expert's scales).
 * Sizes: one expert's codes (N * K/2 bytes) must fit 32-bit offsets.
 * Expert ids out of range or repeated within a token set NVFP4_FAULT_BAD_ROUTE; such
 *   routes are dropped (their rows are zero; they add nothing to a combine).
 * Errors: NVFP4_ERR_NULL, _SHAPE, _ALIGN, _ARG, _WORKSPACE, _LAUNCH. */
nvfp4_status nvfp4_grouped_linear(int32_t act_kind, const void* x, const uint8_t* x_scales,
                                  const float* x_ts, int64_t ldx, int32_t rows_mode,
                                  int64_t T, int32_t top_k, int64_t N, int64_t K,
                                  int32_t num_experts, const uint8_t* w_codes,
                                  const uint8_t* w_scales, const float* w_ts,
                                  const int32_t* topk_ids, const float* topk_w,
                                  int32_t out_mode, void* y, void* workspace,
                                  size_t* workspace_bytes, uint32_t flags, uint32_t* faults,
                                  void* stream);

/* nvfp4_grouped_linear_noalloc — nvfp4_grouped_linear for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, and harnesses that
 * forbid allocation. Same arguments and results as nvfp4_grouped_linear without
 * `workspace` / `workspace_bytes`: the call uses the library's fixed scratch array of
 * NVFP4_NOALLOC_SCRATCH_BYTES on the current device (hipGetDevice, which must be the device
 * `stream` runs on), and calls no allocating routine. Each GPU holds its array from its
 * first such call until the process ends.
 * Limit: a call whose workspace would exceed NVFP4_NOALLOC_SCRATCH_BYTES (see
 *   nvfp4_grouped_linear's workspace query) returns NVFP4_ERR_WORKSPACE, enqueuing nothing.
 *   16 MiB covers the route grouping of up to ~10^6 routes and the fp32 per-route rows of
 *   a decode-sized NVFP4_OUT_COMBINE (e.g. 128 routes x 2048 columns = 1 MiB).
 * Sharing: every call on one GPU uses the same array and leaves its contents there (the
 *   route grouping first, so NVFP4_OUT_REUSE_GROUPING works between two of these calls
 *   on one stream, the later reusing the earlier's grouping). Calls that can overlap on
 *   one GPU (two streams, two threads) race on the array and give undefined results:
 *   order them on one stream. The kernels write every scratch byte they read, so no
 *   clearing is needed between calls.
 * Errors: as nvfp4_grouped_linear; _LAUNCH also when the device's scratch address cannot
 *   be obtained. */
#define NVFP4_NOALLOC_SCRATCH_BYTES (16u << 20)
nvfp4_status nvfp4_grouped_linear_noalloc(int32_t act_kind, const void* x,
                                          const uint8_t* x_scales, const float* x_ts,
                                          int64_t ldx, int32_t rows_mode, int64_t T,
                                          int32_t top_k, int64_t N, int64_t K,
                                          int32_t num_experts, const uint8_t* w_codes,
                                          const uint8_t* w_scales, const float* w_ts,
                                          const int32_t* topk_ids, const float* topk_w,
                                          int32_t out_mode, void* y, uint32_t flags,
                                          uint32_t* faults, void* stream);

/* nvfp4_prefetch — next-weight prefetch: reads [buf, buf + bytes) on `stream` and discards
 * the values, so that the bytes are in the caches (L2 and the 256 MB Infinity Cache) when a
 * later call reads them. For a sequence of layers, issue it for layer i + 1's weight codes
 * and scales on a second stream (of the same priority) while layer i runs, and have layer
 * i + 1 wait for it: each weight byte then leaves HBM once, ahead of the call that needs
 * it, so that call does not wait for the ramp and tail of its own HBM stream (the pages
 * prefetch weight rows into L2 ahead of the gemv calls that read them: issue #565
 * section 4, "Remaining Round 1 items"). Nothing is written; results of other calls do
 * not change.
 * Measured on MI355X for the 28 MB decode weights: it does not pay while the previous
 * layer runs, since the HBM read of the next weight and the running call share the L2 and
 * the fabric (a chain of graph-replayed decode launches takes 18.4 us per layer with it
 * against 9.8 us without). Its use is a weight read while the GPU is otherwise idle, for
 * instance the first layer's during host-side work between decode steps.
 * buf: device memory, 16-byte aligned; bytes: 16 .. 2^31 - 16, a multiple of 16.
 * workgroups: the most workgroups the read may use (1 .. 8192; 0: 512), which bounds its
 *   share of the chip while it overlaps another call.
 * Errors: NVFP4_ERR_NULL, _SHAPE, _ALIGN, _ARG, _LAUNCH. */
nvfp4_status nvfp4_prefetch(const void* buf, int64_t bytes, int32_t workgroups, void* stream);

/* nvfp4_read_probe — measurement support, not part of the layer: one plain streaming read
 * of `bytes` bytes at `buf` in one launch, the measured single-launch read roof that the
 * weight-streaming calls are compared against (the pages set their decode paths beside a
 * measured local roof as well as the nominal one: Rocket engineering log, entry on the
 * GDN decode path on GB10, roofline table).
 * buf: device memory, 16-byte aligned; bytes: 16 .. 2^31 - 16, a multiple of 16.
 * loads_per_thread: 1, 2, 4, 8 or 16 sixteen-byte loads per thread (the launch shape;
 *   each workgroup reads loads_per_thread * 4 KiB).
 * sink: a device word the kernel may overwrite (it keeps the loads live; its value is
 *   meaningless).
 * Errors: NVFP4_ERR_NULL, _SHAPE, _ALIGN, _ARG, _LAUNCH. */
nvfp4_status nvfp4_read_probe(const void* buf, int64_t bytes, int32_t loads_per_thread,
                              uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H */
