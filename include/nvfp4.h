/*
 * nvfp4.h -- C ABI of the NVFP4 W4A4 block-scaled quantization and GEMV/GEMM
 * library for AMD Instinct MI355X (gfx950).
 *
 * What is computed.  The page "TensorRT Edge-LLM Completes the MLPerf Edge
 * Agentic Benchmark 6.4x Faster on Jetson AGX Thor", section "Using NVFP4
 * quantization to accelerate Qwen3.6-27B inference", runs every linear layer
 * of the model (language-model head included) with both weights and
 * activations in NVFP4, the weights quantized once after training, because
 * low-batch decoding is limited by DRAM bandwidth.  The section "Using
 * tree-based multi-token prediction to accelerate LLM inference" verifies a
 * 16-node candidate tree in one forward pass (M = 16 rows), and "Reusing KV
 * cache across agent turns" prefills only a new suffix (M of a few hundred).
 * The pages do not spell out NVFP4's bits; this library follows the public
 * definition:
 *   - element: E2M1, 4 bits (sign, 2 exponent bits with bias 1, 1 mantissa
 *     bit); magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6};
 *   - block scale: one FP8 E4M3FN byte per 16 contiguous K-elements
 *     (bias 7, subnormals, largest finite 448, 0x7F/0xFF are NaN);
 *   - tensor scale: one fp32 decode scale g per tensor.
 *   A quantized value decodes as  x = e2m1(code) * e4m3(scale) * g.
 *
 * Quantization of a 16-block x[0..15] (all steps correctly rounded fp32, no
 * fused multiply-add):
 *   amax = max|x_i|;   s = (g == 0) ? 0 : (amax / 6) / g
 *   sb = E4M3(s) rounded to nearest even, saturating at 448;   sv = e4m3(sb)
 *   d = sv * g;   inv = (d == 0) ? 0 : 1 / d
 *   code_i = E2M1(x_i * inv) rounded to nearest even, saturating at 6; the
 *            code's sign bit is the sign bit of x_i * inv (so -0 -> 0x8).
 * Weights use g_w = amax|W| / 2688 (2688 = 6 * 448), computed on the device.
 * Activations take a static, calibrated g_a supplied by the caller.
 *
 * Layout (row-major, K is the contraction dimension and is contiguous):
 *   codes  uint8 [rows][K/2]  byte j holds element 2j in its low nibble and
 *                             element 2j+1 in its high nibble;
 *   scales uint8 [rows][K/16] one E4M3 byte per block;
 *   W is [N][K] (one row per output feature), A is [M][K], C is [M][N]:
 *     C[m][n] = sum_k a_hat[m][k] * w_hat[n][k]
 *
 * Conventions for every entry point:
 *   - All data pointers are device pointers, allocated and owned by the
 *     caller; the library allocates nothing and keeps no state between calls.
 *   - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL means
 *     the default stream) and is stream-ordered; no call synchronizes.
 *   - Arguments are validated on the host before anything is enqueued.  A
 *     rejected call enqueues nothing and returns its status; no call aborts.
 *     A failed kernel launch returns NVFP4_ERR_HIP; faults during execution
 *     surface at the caller's next synchronization of the stream.
 *   - Sizes: rows (M, N) >= 0 (0 is a valid empty call); K >= 16 and
 *     K % 16 == 0; every dimension product must stay below 2^31 elements.
 *   - Array pointers must be 16-byte aligned; the fp32 tensor-scale pointers
 *     (a_global, w_global) must be 4-byte aligned.
 *   - Validation order: dtype/path, shapes, then (for a non-empty call)
 *     NULL pointers, then alignment.
 *   - Results are bit-identical from run to run (fixed reduction orders, no
 *     floating-point atomics on results).
 *   - Non-finite inputs are outside the contract.
 *   - Calls are re-entrant; calls on different streams may run concurrently
 *     as long as they do not write the same buffers.
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NVFP4_OK = 0,
  NVFP4_ERR_NULL = 1,   /* a required pointer is NULL                          */
  NVFP4_ERR_SHAPE = 2,  /* negative size, K < 16, K % 16 != 0, or too large      */
  NVFP4_ERR_ALIGN = 3,  /* a pointer is not 16-byte aligned                      */
  NVFP4_ERR_DTYPE = 4,  /* unsupported dtype or path selector                    */
  NVFP4_ERR_HIP = 5,    /* the HIP runtime rejected a launch                     */
  NVFP4_ERR_SCRATCH = 6 /* nvfp4_gemm_scratch: the product needs more workspace
                           than the fixed scratch holds                        */
} nvfp4_status;

typedef enum {
  NVFP4_F32 = 0,   /* IEEE binary32                                   */
  NVFP4_BF16 = 1   /* bfloat16, rounded to nearest even when written  */
} nvfp4_dtype;

/* Path selector for nvfp4_gemm_ex.  The first three are the library's
 * automatic choices; the kernel selectors run one named kernel and return
 * NVFP4_ERR_SHAPE when that kernel does not take the product.  They exist so
 * that every kernel can be checked against the others and against a
 * reference; the result contract is the same for all of them. */
typedef enum {
  NVFP4_PATH_AUTO = 0,    /* M <= 16: skinny path; otherwise the tiled path       */
  NVFP4_PATH_SKINNY = 1,  /* weight-streaming path, any M (tiles M by 16)         */
  NVFP4_PATH_TILED = 2,   /* LDS-tiled MFMA path, any M                           */
  NVFP4_KERNEL_GEMV_FP4 = 3,          /* FP4 matrix-core GEMV: M <= 2, K % 1024 == 0,
                                         1024 <= K <= 8192                        */
  NVFP4_KERNEL_GEMV_FLAT = 4,         /* memory-order GEMV: M <= 2, K % 256 == 0,
                                         K >= 2048 (within its LDS budget)        */
  NVFP4_KERNEL_M16 = 5,               /* M-tile weight stream on f16 matrix cores:
                                         M <= 16, K % 128 == 0 (never split here) */
  NVFP4_KERNEL_SKINNY256 = 6,         /* skinny kernel, K % 256 == 0, any M       */
  NVFP4_KERNEL_SKINNY16 = 7,          /* skinny kernel, any K, any M              */
  NVFP4_KERNEL_TILED_PERSISTENT = 8,  /* persistent 64x160-tile MFMA kernel,
                                         K % 1024 == 0                            */
  NVFP4_KERNEL_TILED = 9,             /* 128x128-tile MFMA kernel, any shape      */
  NVFP4_KERNEL_M16_STREAM = 10        /* persistent weight stream on f16 matrix
                                         cores: M <= 16, K % 1024 == 0 (or a
                                         multiple of 1536, 2048 or 2560)          */
} nvfp4_path;

/* Offline weight quantization (post-training, done once).
 *   w         [N][K] in w_dt (NVFP4_F32 or NVFP4_BF16), device.
 *   w_codes   out: [N][K/2] packed E2M1 codes.
 *   w_scales  out: [N][K/16] E4M3 block scales.
 *   w_global  out: one float, g_w = fl32(amax|W| / 2688) (0 for an all-zero W).
 *             Also used as the accumulator of the amax pass, so it must not
 *             alias any other argument.
 * Cites: the page section "Using NVFP4 quantization to accelerate Qwen3.6-27B
 * inference" (weights quantized once, after training). */
nvfp4_status nvfp4_quantize_weights(const void* w, nvfp4_dtype w_dt, int64_t N, int64_t K,
                                    uint8_t* w_codes, uint8_t* w_scales, float* w_global,
                                    void* stream);

/* On-the-fly activation quantization.
 *   a         [M][K] in a_dt (NVFP4_F32 or NVFP4_BF16), device.
 *   a_global  in: one float on the device, the static calibrated decode scale g_a.
 *   a_codes   out: [M][K/2];  a_scales out: [M][K/16].
 * Cites: the same section (activations are NVFP4 as well as weights). */
nvfp4_status nvfp4_quantize_act(const void* a, nvfp4_dtype a_dt, int64_t M, int64_t K,
                                const float* a_global, uint8_t* a_codes, uint8_t* a_scales,
                                void* stream);

/* Dynamic activation tensor scale, computed on the device from the
 * activations themselves instead of a static calibrated value.
 *   a         [M][K] in a_dt (NVFP4_F32 or NVFP4_BF16), device.
 *   a_global  out: one float, g_a = fl32(amax|A| / 2688) (0 for an all-zero
 *             A): the weights' formula.  Also the amax accumulator for large
 *             tensors, so it must not alias any other argument.
 * Stream-ordered before nvfp4_quantize_act / nvfp4_quantize_gemm, which read
 * it from the device.  One kernel up to 2^20 elements (a decode row), three
 * beyond.
 * Cites: the page section "Using NVFP4 quantization to accelerate Qwen3.6-27B
 * inference" (activations are NVFP4; the pages stress a calibrated checkpoint,
 * of which this is the dynamic alternative). */
nvfp4_status nvfp4_act_global_scale(const void* a, nvfp4_dtype a_dt, int64_t M, int64_t K, float* a_global,
                                    void* stream);

/* NVFP4 W4A4 GEMM:  out[m][n] = g_a * g_w * sum_k e2m1(qa)*sa * e2m1(qw)*sw.
 *   a_codes [M][K/2], a_scales [M][K/16], a_global (device float): activations.
 *   w_codes [N][K/2], w_scales [N][K/16], w_global (device float): weights.
 *   out     [M][N] in out_dt (NVFP4_F32 or NVFP4_BF16).
 * Accumulation is in fp32; the result is within 1e-3 * sum_k |a_hat*w_hat| of
 * the exact product.  M <= 16 (single-stream decode, 16-node tree
 * verification) runs the weight-streaming skinny path; larger M (suffix
 * prefill) runs the LDS-tiled MFMA path.
 * Cites: the sections on NVFP4 quantization, tree-based multi-token
 * prediction (one pass over 16 candidates) and KV-cache reuse (suffix prefill). */
nvfp4_status nvfp4_gemm(int64_t M, int64_t K, int64_t N,
                        const uint8_t* a_codes, const uint8_t* a_scales, const float* a_global,
                        const uint8_t* w_codes, const uint8_t* w_scales, const float* w_global,
                        void* out, nvfp4_dtype out_dt, void* stream);

/* nvfp4_gemm with an explicit path or kernel (nvfp4_path); same arguments
 * and result contract.  An unknown selector -> NVFP4_ERR_DTYPE; a kernel
 * selector whose kernel does not take (M, K, N) -> NVFP4_ERR_SHAPE. */
nvfp4_status nvfp4_gemm_ex(int64_t M, int64_t K, int64_t N,
                           const uint8_t* a_codes, const uint8_t* a_scales, const float* a_global,
                           const uint8_t* w_codes, const uint8_t* w_scales, const float* w_global,
                           void* out, nvfp4_dtype out_dt, int path, void* stream);

/* The kernel (an NVFP4_KERNEL_* value of nvfp4_path) that nvfp4_gemm_ws runs
 * for an (M, K, N) product with a workspace of workspace_bytes bytes (0:
 * nvfp4_gemm), or 0 for an empty or invalid product.  A pure function of its
 * arguments and the device's compute-unit count; enqueues nothing.
 * Cites: the page sections on NVFP4 quantization (M = 1 decode), tree-based
 * multi-token prediction (M = 16) and KV-cache reuse (suffix prefill). */
int nvfp4_gemm_dispatch(int64_t M, int64_t K, int64_t N, int64_t workspace_bytes);

/* Size in bytes of the workspace with which nvfp4_gemm_ws splits the
 * contraction of an (M, K, N) product over several workgroups; 0 when it
 * would not (M outside 3..16, K not a multiple of 128, a short K (a multiple
 * of 256 up to 8192) with N <= 16384, which a kernel without a split serves
 * faster, or enough rows to fill the GPU without a split).  Depends only on
 * (M, K, N) and the current device's compute-unit count (one HIP attribute
 * query; nothing is enqueued).  At the tree-verification pass of a down-projection
 * (M = 16, K = 25600, N = 5120) it is a few MiB.
 * Cites: the section on tree-based multi-token prediction (one pass over the
 * 16 candidates: few output rows, a long contraction). */
int64_t nvfp4_gemm_workspace_bytes(int64_t M, int64_t K, int64_t N);

/* nvfp4_gemm with a caller-owned workspace; same arguments and result
 * contract as nvfp4_gemm.
 *   workspace        device memory, 16-byte aligned, or NULL with
 *                    workspace_bytes == 0 (then exactly nvfp4_gemm).
 *   workspace_bytes  its size.  With at least nvfp4_gemm_workspace_bytes(M,
 *                    K, N) bytes the product splits K over workgroups, each
 *                    writing fp32 partial sums there; the last workgroup of
 *                    a row block to finish adds them in a fixed order, so the
 *                    result is still bit-identical from run to run.  A
 *                    smaller workspace runs the unsplit kernels.
 * The workspace must be all zero before its first use (its leading counters
 * must read zero on entry); every call leaves them zero again, so it is
 * cleared once, not per call.  Calls sharing a workspace must be ordered on
 * one stream.  Errors: workspace_bytes < 0 -> NVFP4_ERR_SHAPE; NULL with
 * workspace_bytes > 0 -> NVFP4_ERR_NULL; misaligned -> NVFP4_ERR_ALIGN.
 * Cites: the sections on NVFP4 quantization and tree-based multi-token
 * prediction. */
nvfp4_status nvfp4_gemm_ws(int64_t M, int64_t K, int64_t N,
                           const uint8_t* a_codes, const uint8_t* a_scales, const float* a_global,
                           const uint8_t* w_codes, const uint8_t* w_scales, const float* w_global,
                           void* out, nvfp4_dtype out_dt, void* workspace, int64_t workspace_bytes,
                           void* stream);

/* Size in bytes of the fixed per-device scratch array of nvfp4_gemm_scratch. */
#define NVFP4_SCRATCH_BYTES 4194304

/* nvfp4_gemm_ws for callers that cannot allocate or pass a workspace: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The split-K workspace is a fixed device array inside the
 * library, NVFP4_SCRATCH_BYTES (4 MiB) per device, held until the process
 * ends; the call allocates nothing.  Same arguments and result contract as
 * nvfp4_gemm, and bit-identical to nvfp4_gemm_ws with a large enough
 * workspace (the same kernels and split plan).
 *   - A product whose nvfp4_gemm_workspace_bytes exceeds NVFP4_SCRATCH_BYTES
 *     is rejected with NVFP4_ERR_SCRATCH, enqueuing nothing (on a 256-CU
 *     MI355X no split plan needs more than about 2 MiB).
 *   - Every call on a device shares that device's array and leaves its
 *     counters zero for the next: calls that overlap on one GPU (on different
 *     streams, or graph replays running concurrently) race and may produce
 *     wrong results.  Keep them ordered on one stream.
 *   - The first call on a device takes the array's device address and
 *     enqueues, on `stream`, a small kernel that clears its counter area
 *     (also when that call is being captured into a graph).
 * Validation as nvfp4_gemm; NVFP4_ERR_HIP if the array's address cannot be
 * taken. */
nvfp4_status nvfp4_gemm_scratch(int64_t M, int64_t K, int64_t N,
                                const uint8_t* a_codes, const uint8_t* a_scales, const float* a_global,
                                const uint8_t* w_codes, const uint8_t* w_scales, const float* w_global,
                                void* out, nvfp4_dtype out_dt, void* stream);

/* NVFP4 W4A4 GEMM whose output is also emitted in NVFP4: the product of one
 * layer of a prefill becomes the quantized activations of the next.
 *   a_*, w_*, out, out_dt: as nvfp4_gemm (out is required).
 *   y_global  in: device float, the static calibrated decode scale of the output.
 *   y_codes   out: [M][N/2];  y_scales out: [M][N/16]: bit-identical to
 *             nvfp4_quantize_act(out, out_dt, M, N, y_global, ...) applied to
 *             the stored out (so bf16 outputs are quantized after rounding).
 * N % 16 == 0 (the output's blocks run along N), else NVFP4_ERR_SHAPE.  For
 * M > 16 with K a multiple of 1024 this is one kernel: the epilogue of the
 * tiled GEMM quantizes each 16-column block of its tile while writing it, so
 * the output is not read back; other shapes run the GEMM, then the
 * quantization (two launches, same results).
 * Cites: the page sections "Using NVFP4 quantization to accelerate
 * Qwen3.6-27B inference" (weights and activations NVFP4) and "Reusing KV
 * cache across agent turns" (a suffix prefill passes through every layer). */
nvfp4_status nvfp4_gemm_quantize_output(int64_t M, int64_t K, int64_t N,
                                        const uint8_t* a_codes, const uint8_t* a_scales, const float* a_global,
                                        const uint8_t* w_codes, const uint8_t* w_scales, const float* w_global,
                                        void* out, nvfp4_dtype out_dt, const float* y_global, uint8_t* y_codes,
                                        uint8_t* y_scales, void* stream);

/* Activation quantization and GEMM in one call: the decode step's
 * nvfp4_quantize_act + nvfp4_gemm.
 *   a         [M][K] raw activations in a_dt (NVFP4_F32 or NVFP4_BF16), device.
 *   a_global  in: device float, the static calibrated decode scale g_a.
 *   w_codes, w_scales, w_global, out, out_dt: as nvfp4_gemm.
 *   a_codes   out: [M][K/2];  a_scales out: [M][K/16]: the activations' NVFP4
 *             form, bit-identical to nvfp4_quantize_act; required (they are
 *             also the intermediate when the call runs as two launches).
 * out is bit-identical to nvfp4_quantize_act followed by nvfp4_gemm.  For
 * M <= 2 with K a multiple of 1024 in [1024, 8192] this is one kernel: each
 * workgroup quantizes the activation rows into its LDS while its first
 * weight loads are in flight (the standalone quantization launch and its
 * round trip through memory disappear from the decode step); other shapes run
 * the two launches.  N == 0 only quantizes.  Validation as nvfp4_gemm, with
 * a_dt checked with out_dt and a, a_global, a_codes, a_scales always required
 * for M > 0.
 * Cites: the page section "Using NVFP4 quantization to accelerate Qwen3.6-27B
 * inference" (NVFP4 activations shrink the memory traffic of low-batch
 * decode, which is bandwidth bound). */
nvfp4_status nvfp4_quantize_gemm(int64_t M, int64_t K, int64_t N,
                                 const void* a, nvfp4_dtype a_dt, const float* a_global,
                                 const uint8_t* w_codes, const uint8_t* w_scales, const float* w_global,
                                 void* out, nvfp4_dtype out_dt, uint8_t* a_codes, uint8_t* a_scales,
                                 void* stream);

/* nvfp4_quantize_gemm with the activations' tensor scale computed on the
 * device: the decode step's nvfp4_act_global_scale + nvfp4_quantize_act +
 * nvfp4_gemm.
 *   a_global  out: device float, g_a = fl32(amax|A| / 2688) (0 for an all-zero
 *             or empty A), bit-identical to nvfp4_act_global_scale; it must
 *             not alias any other argument.
 *   other arguments as nvfp4_quantize_gemm; a_codes / a_scales are quantized
 *             with that g_a and out is bit-identical to the three calls.
 * For M <= 2 with K a multiple of 1024 in [1024, 8192] this is one kernel:
 * every workgroup reduces the largest magnitude of the rows it already loads
 * for quantization, so neither the scale launch nor its round trip through
 * memory remains; workgroup 0 stores g_a.  Other shapes run the scale kernel,
 * then nvfp4_quantize_gemm's launches.  M == 0 only sets g_a = 0.
 * Errors as nvfp4_quantize_gemm, a_global always required.
 * Cites: the page section "Using NVFP4 quantization to accelerate Qwen3.6-27B
 * inference" (NVFP4 activations; a dynamic per-tensor scale is the alternative
 * to the calibrated one). */
nvfp4_status nvfp4_quantize_gemm_dynamic(int64_t M, int64_t K, int64_t N,
                                         const void* a, nvfp4_dtype a_dt, float* a_global,
                                         const uint8_t* w_codes, const uint8_t* w_scales, const float* w_global,
                                         void* out, nvfp4_dtype out_dt, uint8_t* a_codes, uint8_t* a_scales,
                                         void* stream);

/* FP8 E4M3 KV-cache codec: encode.
 *   x      [n] KV values in x_dt (NVFP4_F32 or NVFP4_BF16), device, any layout
 *          (the codec is elementwise).
 *   scale  in: device float, the tensor's static decode scale s (a
 *          calibration sets s = amax / 448).
 *   q      out: [n] E4M3FN bytes.
 * Per element, in correctly rounded fp32: inv = (s == 0) ? 0 : 1 / s,
 * y = x * inv, q = E4M3(y) rounded to nearest even, saturating at +-448, with
 * the sign bit of y.  n < 2^40; x and q 16-byte aligned.
 * Cites: the page section "Using NVFP4 quantization to accelerate
 * Qwen3.6-27B inference" (the KV cache is FP8). */
nvfp4_status nvfp4_kv_fp8_encode(const void* x, nvfp4_dtype x_dt, int64_t n, const float* scale, uint8_t* q,
                                 void* stream);

/* FP8 E4M3 KV-cache codec: decode.  x[i] = fl32(e4m3(q[i]) * s), written as
 * fp32 or rounded to nearest even bf16 (x_dt).  Arguments as the encoder's. */
nvfp4_status nvfp4_kv_fp8_decode(const uint8_t* q, int64_t n, const float* scale, void* x, nvfp4_dtype x_dt,
                                 void* stream);

/* Greedy (temperature-0) acceptance of a verified candidate tree.
 *   n_nodes  1..64 tree nodes in topological order; node 0 is the root.
 *   parent   [n_nodes] int32, device: parent[0] = -1, 0 <= parent[v] < v
 *            (an index outside [0, v) rejects node v).
 *   draft    [n_nodes] int32, device: node v's drafted token (entry 0 unused).
 *   greedy   [n_nodes] int32, device: the target's argmax token after node v.
 *   result   out [3 + n_nodes] int32, device: end node, accepted draft count L,
 *            bonus token, then the L accepted nodes root-child first, then -1.
 * Node v is accepted when its parent is and draft[v] == greedy[parent[v]];
 * the path ends at the deepest accepted node (lowest index on ties) and the
 * bonus token is greedy[end]: one verification advances L + 1 tokens.
 * Cites: the page section "Using tree-based multi-token prediction to
 * accelerate LLM inference" (one forward pass verifies the tree; the
 * matching path is accepted) and the benchmark's temperature 0. */
nvfp4_status nvfp4_tree_accept(int64_t n_nodes, const int32_t* parent, const int32_t* draft, const int32_t* greedy,
                               int32_t* result, void* stream);

/* LM head over a candidate tree plus greedy acceptance, in one call.
 *   M        1..16 tree nodes (rows); K, N (vocabulary): as nvfp4_gemm, with the
 *            nodes' NVFP4 activations a_* and the LM-head weights w_*.
 *   parent, draft: as nvfp4_tree_accept.
 *   logits   optional out [M][N] fp32 (may be NULL when K % 128 == 0: the
 *            argmax is then fused into the GEMM and the logits are not
 *            written; other K need it).
 *   greedy   out [M] int32: each row's argmax (lowest column on ties; -0.0
 *            orders just below +0.0).
 *   result   out [3 + M] int32: as nvfp4_tree_accept.
 *   keys     workspace of 1024 64-bit words (8 KiB), device, 8-byte aligned,
 *            caller-owned: must be all zero on entry and is all zero again on
 *            return (clear it once before first use; calls sharing it must be
 *            stream-ordered).
 * Deterministic: the argmax merges per-workgroup maxima with atomic maxima
 * (64 slots per row), whose result does not depend on their order.  The
 * slots are folded after the product: by a small acceptance kernel, or, on
 * the persistent weight-stream kernel, by that kernel's last workgroup to
 * finish (found by an arrival counter kept in the last slot of the same
 * workspace), which also runs the acceptance: one launch per call.
 * Cites: the sections on tree-based multi-token prediction (16-node tree
 * verified in one pass) and NVFP4 quantization (the LM head is NVFP4). */
nvfp4_status nvfp4_tree_verify(int64_t M, int64_t K, int64_t N,
                               const uint8_t* a_codes, const uint8_t* a_scales, const float* a_global,
                               const uint8_t* w_codes, const uint8_t* w_scales, const float* w_global,
                               const int32_t* parent, const int32_t* draft, float* logits, int32_t* greedy,
                               int32_t* result, uint64_t* keys, void* stream);

/* Read-only streaming ceiling: reads the a_bytes bytes at a and the b_bytes
 * bytes at b once (16-byte loads, each wave a contiguous span, the loads
 * marked non-temporal); every lane folds the four words of each of its loads
 * by XOR and writes sink[0] = its fold only if that equals magic.  Run over the codes and scales of a weight matrix it
 * measures how fast plain HIP code reads exactly the bytes a GEMV or M = 16
 * GEMM of that matrix must read: the ceiling those products are reported
 * against, beside the 8 TB/s of the HBM specification.
 *   a, b     device arrays, 16-byte aligned (either may be NULL when its size
 *            is 0); a_bytes, b_bytes multiples of 16 below 2^31.
 *   sink     device uint32, 4-byte aligned (not written in practice).
 * Errors: a size out of range -> NVFP4_ERR_SHAPE; a NULL array with a size or
 * a NULL sink -> NVFP4_ERR_NULL; misaligned -> NVFP4_ERR_ALIGN.
 * Cites: the page section "Using NVFP4 quantization to accelerate Qwen3.6-27B
 * inference" (low-batch decoding is bound by DRAM bandwidth). */
nvfp4_status nvfp4_stream_read(const void* a, int64_t a_bytes, const void* b, int64_t b_bytes, uint32_t* sink,
                               uint32_t magic, void* stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* nvfp4_status_string(nvfp4_status s);

/* ABI version of this header (bumped on any signature change). */
int nvfp4_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H */
