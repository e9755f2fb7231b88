// Host-side launchers of the NVFP4 kernels (internal to the library; the
// public C ABI is include/nvfp4.h).  Arguments are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

// Per-16-block quantization of a [rows][K] tensor (fp32, or bf16 when `bf16`)
// with the decode scale read from device memory at `g`.
hipError_t launch_quantize(const void* x, bool bf16, int64_t rows, int64_t K, const float* g,
                           uint8_t* codes, uint8_t* scales, hipStream_t stream);

// g = amax|w| / 2688 over `elems` elements, written to the device float `g`.
hipError_t launch_weight_global(const void* w, bool bf16, int64_t elems, float* g,
                                hipStream_t stream);
// The same for activations; one workgroup and one launch up to 2^20 elements.
hipError_t launch_act_global(const void* a, bool bf16, int64_t elems, float* g, hipStream_t stream);

struct GemmArgs {
  int M, K, N;
  const uint8_t* ac;  // activation codes [M][K/2]
  const uint8_t* as;  // activation scales [M][K/16]
  const float* ga;    // activation decode scale (device)
  const uint8_t* wc;  // weight codes [N][K/2]
  const uint8_t* ws;  // weight scales [N][K/16]
  const float* gw;    // weight decode scale (device)
  void* out;          // [M][N]
  bool out_bf16;
  // Fused activation quantization (FP4 GEMV only): when a_raw is set, the
  // kernel quantizes the [M][K] activation rows itself with *ga and writes
  // their codes and scales to ac_out / as_out; ac and as are then unused.
  const void* a_raw = nullptr;
  bool a_raw_bf16 = false;
  uint8_t* ac_out = nullptr;
  uint8_t* as_out = nullptr;
  // Fused row argmax (gemm_m16 only): when set, each activation row's largest
  // output (lowest column on ties) is merged by an atomic maximum of
  // argmax_key() into argmax_keys[slot][m], slot = workgroup % kKeySlots
  // ([kKeySlots][16] words, zero on entry); out may then be NULL.
  uint64_t* argmax_keys = nullptr;
  // Caller-owned device workspace (gemm_m16 only): when at least
  // gemm_m16_workspace_bytes() large, long K is split over workgroups.  Its
  // first bytes are arrival counters that must be zero on entry and are zero
  // again when the kernel ends.
  void* workspace = nullptr;
  int64_t workspace_bytes = 0;
  // Output quantization (persistent tiled kernel only, N % 16 == 0): when
  // y_codes is set, every 16-column block of each output row, rounded to the
  // output dtype as stored, is also quantized with the decode scale *y_global
  // exactly as quant_blocks_kernel would quantize the stored output, into
  // y_codes [M][N/2] and y_scales [M][N/16].
  const float* y_global = nullptr;
  uint8_t* y_codes = nullptr;
  uint8_t* y_scales = nullptr;
  // Fused GEMV only (a_raw set): when ga_dynamic is set the tensor scale is not read from ga:
  // every workgroup computes g_a = fl32(amax|A| / 2688) from the raw rows it
  // holds, uses it, and workgroup 0 stores it to *ga_dynamic.
  float* ga_dynamic = nullptr;
  // Fused tree acceptance (persistent M = 16 stream only, with argmax_keys):
  // when tree_result is set, the last workgroup to finish folds the keys,
  // resets them to zero and runs the greedy acceptance of the M-node tree
  // tree_parent / tree_draft, writing tree_greedy [M] and tree_result [3 + M]
  // (the layout of tree_accept_kernel).  Word 0 of key slot kKeySlots - 1 is
  // then its arrival counter (the kernel merges no key into that slot).
  const int32_t* tree_parent = nullptr;
  const int32_t* tree_draft = nullptr;
  int32_t* tree_greedy = nullptr;
  int32_t* tree_result = nullptr;
};

constexpr int kKeySlots = 64;  // argmax key slots per row (zero between calls)

// FP8 E4M3 KV-cache codec (kv_fp8.hip).
hipError_t launch_kv_fp8_encode(const void* x, bool bf16, int64_t n, const float* scale, uint8_t* q,
                                hipStream_t stream);
hipError_t launch_kv_fp8_decode(const uint8_t* q, int64_t n, const float* scale, void* x, bool bf16,
                                hipStream_t stream);

// Greedy tree verification over the LM head (tree.hip).  The argmax keys
// ([kKeySlots][16]) are reduced, and reset to zero, by the acceptance kernel.
hipError_t launch_argmax_rows(const float* logits, int M, int N, uint64_t* keys, hipStream_t stream);
hipError_t launch_tree_accept(int n, const int32_t* parent, const int32_t* draft, const int32_t* greedy_in,
                              uint64_t* keys, int32_t* greedy_out, int32_t* result, hipStream_t stream);

// Kernels of the product, numbered as the kernel selectors of nvfp4_path in
// include/nvfp4.h.
enum KernelId : int {
  kKernelGemvFp4 = 3,          // gemv_fp4_kernel: FP4 matrix-core GEMV, M <= 2
  kKernelGemvFlat = 4,         // gemv_flat_kernel: memory-order GEMV, M <= 2
  kKernelM16 = 5,              // gemm_m16_kernel: weight streaming on f16 matrix cores, M <= 16
  kKernelSkinny256 = 6,        // gemm_skinny256_kernel: K % 256 == 0, any M
  kKernelSkinny16 = 7,         // gemm_skinny_kernel: any K, any M
  kKernelTiledPersistent = 8,  // gemm_wg_tiled_kernel: K % 1024 == 0
  kKernelTiled = 9,            // gemm_tiled_kernel: any shape
  kKernelM16Stream = 10,       // gemm_m16_stream_kernel: persistent weight stream, M <= 16, tall N
};

// Weight-streaming path (built for M <= 16; the skinny kernels tile larger M
// by 16 rows): skinny_kernel_choice() names the kernel launch_gemm_skinny()
// runs.
int skinny_kernel_choice(const GemmArgs& a);
hipError_t launch_gemm_skinny(const GemmArgs& a, hipStream_t stream);

// FP4 matrix-core GEMV for M <= 2 (K % 1024 == 0, 1024 <= K <= 8192 within
// its LDS budget); launch only where gemv_fp4_supported() holds.
bool gemv_fp4_supported(const GemmArgs& a);
hipError_t launch_gemv_fp4(const GemmArgs& a, hipStream_t stream);

// Memory-order GEMV for M <= 2 (K % 256 == 0, K >= 2048, within its limits).
bool gemv_flat_supported(const GemmArgs& a);
hipError_t launch_gemv_flat(const GemmArgs& a, hipStream_t stream);

// Skinny kernels: K % 256 == 0, and any K (a multiple of 16); any M.
hipError_t launch_gemm_skinny256(const GemmArgs& a, hipStream_t stream);
hipError_t launch_gemm_skinny16(const GemmArgs& a, hipStream_t stream);

// Weight-streaming GEMM for 1 <= M <= 16 on f16 matrix cores (K % 128 == 0;
// any K in one pass).  gemm_m16_workspace_bytes() is the workspace that lets
// it split K over workgroups (0 when it would not).
bool gemm_m16_supported(const GemmArgs& a);
bool gemm_m16_small_prefers_skinny(const GemmArgs& a);  // the skinny kernel serves this product instead
bool gemm_m16_preferred(const GemmArgs& a);  // 3 <= M <= 16, supported, and faster than the alternatives
int64_t gemm_m16_workspace_bytes(const GemmArgs& a);
hipError_t launch_gemm_m16(const GemmArgs& a, hipStream_t stream);

// Persistent weight stream for 1 <= M <= 16 over a tall matrix (one
// workgroup per CU, K walked in chunks of 8-20 lines: K a multiple of 1024,
// 1536, 2048 or 2560; N * K / 2 < 2^31).  Preferred (M >= 3) from 10 groups
// of 16 rows per CU on; never splits K.  Takes argmax_keys like the M-tile
// kernel.
bool gemm_m16_stream_supported(const GemmArgs& a);
bool gemm_m16_stream_preferred(const GemmArgs& a);
hipError_t launch_gemm_m16_stream(const GemmArgs& a, hipStream_t stream);

// LDS-tiled MFMA path for large M: the persistent kernel where
// gemm_tiled_persistent_supported() holds (K % 1024 == 0), else the simple
// tiled kernel.  gemm_tiled_quant_out_supported() tells whether
// launch_gemm_tiled() honours y_codes (the persistent kernel with N % 16 ==
// 0); launch_gemm_tiled() ignores y_codes otherwise.
bool gemm_tiled_persistent_supported(const GemmArgs& a);
hipError_t launch_gemm_tiled_persistent(const GemmArgs& a, hipStream_t stream);
hipError_t launch_gemm_tiled_simple(const GemmArgs& a, hipStream_t stream);
hipError_t launch_gemm_tiled(const GemmArgs& a, hipStream_t stream);
bool gemm_tiled_quant_out_supported(const GemmArgs& a);

// Fixed device scratch (scratch.hip) for callers that cannot allocate: the
// size of the per-device array (NVFP4_SCRATCH_BYTES in include/nvfp4.h), and
// the current device's address of it (taken once per device, when its counter
// area is also cleared by a kernel on `stream`).
constexpr int64_t kScratchBytes = (int64_t)4 << 20;
hipError_t scratch_workspace(void** out, hipStream_t stream);

// Read-only stream over two arrays (stream.hip): the measured read ceiling
// of a weight matrix's codes and scales.  sink[0] is written only if the XOR
// of everything read equals `magic`.
hipError_t launch_read_stream(const uint8_t* a, int64_t a_bytes, const uint8_t* b, int64_t b_bytes, uint32_t* sink,
                              uint32_t magic, hipStream_t stream);

}  // namespace nvfp4
