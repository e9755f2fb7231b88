// C ABI of the NVFP4 library (declared in include/nvfp4.h): argument
// validation on the host, then dispatch to the HIP kernels.  Validation makes
// no HIP call, so a rejected call enqueues nothing and is safe without a GPU.
#include "nvfp4.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace {

constexpr int64_t kMaxElems = (int64_t)1 << 31;  // exclusive bound on any dimension product
constexpr int64_t kMaxGridY = 65535;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }
bool dtype_ok(int dt) { return dt == NVFP4_F32 || dt == NVFP4_BF16; }

// Checks rows >= 0, K >= 16, K % 16 == 0 and rows * K < 2^31.
bool shape_ok(int64_t rows, int64_t K) {
  if (rows < 0 || K < 16 || (K % 16) != 0 || K >= kMaxElems) return false;
  return rows == 0 || rows < kMaxElems / K;
}

nvfp4_status from_hip(hipError_t e) { return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP; }

}  // namespace

extern "C" {

const char* nvfp4_status_string(nvfp4_status s) {
  switch (s) {
    case NVFP4_OK: return "ok";
    case NVFP4_ERR_NULL: return "a required pointer is NULL";
    case NVFP4_ERR_SHAPE: return "invalid shape (sizes must be >= 0, K >= 16, K % 16 == 0, products < 2^31)";
    case NVFP4_ERR_ALIGN: return "pointer not aligned (arrays: 16 bytes, scalars: 4 bytes)";
    case NVFP4_ERR_DTYPE: return "unsupported dtype or path";
    case NVFP4_ERR_HIP: return "HIP runtime error while launching";
    case NVFP4_ERR_SCRATCH: return "the product needs more split-K workspace than the fixed scratch holds";
  }
  return "unknown status";
}

int nvfp4_abi_version(void) { return 11; }

nvfp4_status nvfp4_quantize_weights(const void* w, nvfp4_dtype w_dt, int64_t N, int64_t K,
                                    uint8_t* w_codes, uint8_t* w_scales, float* w_global,
                                    void* stream) {
  if (!dtype_ok(w_dt)) return NVFP4_ERR_DTYPE;
  if (!shape_ok(N, K)) return NVFP4_ERR_SHAPE;
  if (!w_global) return NVFP4_ERR_NULL;
  if (!aligned4(w_global)) return NVFP4_ERR_ALIGN;
  if (N > 0) {
    if (!w || !w_codes || !w_scales) return NVFP4_ERR_NULL;
    if (!aligned16(w) || !aligned16(w_codes) || !aligned16(w_scales)) return NVFP4_ERR_ALIGN;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf16 = w_dt == NVFP4_BF16;
  hipError_t e = nvfp4::launch_weight_global(w, bf16, N * K, w_global, s);
  if (e != hipSuccess || N == 0) return from_hip(e);
  return from_hip(nvfp4::launch_quantize(w, bf16, N, K, w_global, w_codes, w_scales, s));
}

nvfp4_status nvfp4_act_global_scale(const void* a, nvfp4_dtype a_dt, int64_t M, int64_t K, float* a_global,
                                    void* stream) {
  if (!dtype_ok(a_dt)) return NVFP4_ERR_DTYPE;
  if (!shape_ok(M, K)) return NVFP4_ERR_SHAPE;
  if (!a_global) return NVFP4_ERR_NULL;
  if (!aligned4(a_global)) return NVFP4_ERR_ALIGN;
  if (M > 0) {
    if (!a) return NVFP4_ERR_NULL;
    if (!aligned16(a)) return NVFP4_ERR_ALIGN;
  }
  return from_hip(nvfp4::launch_act_global(a, a_dt == NVFP4_BF16, M * K, a_global, static_cast<hipStream_t>(stream)));
}

nvfp4_status nvfp4_quantize_act(const void* a, nvfp4_dtype a_dt, int64_t M, int64_t K,
                                const float* a_global, uint8_t* a_codes, uint8_t* a_scales,
                                void* stream) {
  if (!dtype_ok(a_dt)) return NVFP4_ERR_DTYPE;
  if (!shape_ok(M, K)) return NVFP4_ERR_SHAPE;
  if (M == 0) return NVFP4_OK;
  if (!a || !a_global || !a_codes || !a_scales) return NVFP4_ERR_NULL;
  if (!aligned16(a) || !aligned4(a_global) || !aligned16(a_codes) || !aligned16(a_scales))
    return NVFP4_ERR_ALIGN;
  return from_hip(nvfp4::launch_quantize(a, a_dt == NVFP4_BF16, M, K, a_global, a_codes, a_scales,
                                         static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

bool path_ok(int path) { return path >= NVFP4_PATH_AUTO && path <= NVFP4_KERNEL_M16_STREAM; }

// Grid rows a path launches for M activation rows (grid.y is at most 65535).
int64_t grid_rows(int path, int64_t M) {
  const bool tiled = path == NVFP4_PATH_TILED || path == NVFP4_KERNEL_TILED_PERSISTENT || path == NVFP4_KERNEL_TILED;
  return tiled ? (M + 127) / 128 : (M + 15) / 16;
}

// Whether an explicitly selected kernel takes the product.
bool kernel_takes(int k, const nvfp4::GemmArgs& g) {
  switch (k) {
    case NVFP4_KERNEL_GEMV_FP4: return nvfp4::gemv_fp4_supported(g);
    case NVFP4_KERNEL_GEMV_FLAT: return nvfp4::gemv_flat_supported(g);
    case NVFP4_KERNEL_M16: return nvfp4::gemm_m16_supported(g);
    case NVFP4_KERNEL_M16_STREAM: return nvfp4::gemm_m16_stream_supported(g);
    case NVFP4_KERNEL_SKINNY256: return g.K % 256 == 0;
    case NVFP4_KERNEL_TILED_PERSISTENT: return nvfp4::gemm_tiled_persistent_supported(g);
    default: return true;  // the skinny16 and simple tiled kernels take any shape
  }
}

hipError_t launch_path(int path, const nvfp4::GemmArgs& g, hipStream_t s) {
  switch (path) {
    case NVFP4_PATH_SKINNY: return nvfp4::launch_gemm_skinny(g, s);
    case NVFP4_PATH_TILED: return nvfp4::launch_gemm_tiled(g, s);
    case NVFP4_KERNEL_GEMV_FP4: return nvfp4::launch_gemv_fp4(g, s);
    case NVFP4_KERNEL_GEMV_FLAT: return nvfp4::launch_gemv_flat(g, s);
    case NVFP4_KERNEL_M16: return nvfp4::launch_gemm_m16(g, s);
    case NVFP4_KERNEL_M16_STREAM: return nvfp4::launch_gemm_m16_stream(g, s);
    case NVFP4_KERNEL_SKINNY256: return nvfp4::launch_gemm_skinny256(g, s);
    case NVFP4_KERNEL_SKINNY16: return nvfp4::launch_gemm_skinny16(g, s);
    case NVFP4_KERNEL_TILED_PERSISTENT: return nvfp4::launch_gemm_tiled_persistent(g, s);
    default: return nvfp4::launch_gemm_tiled_simple(g, s);
  }
}

// Validation of nvfp4_gemm_ex / nvfp4_gemm_ws / nvfp4_gemm_scratch; on success
// *path is the resolved path or kernel and *g the arguments (g->M == 0 or
// g->N == 0: nothing to run).
nvfp4_status gemm_validate(int64_t M, int64_t K, int64_t N,
                           const uint8_t* a_codes, const uint8_t* a_scales, const float* a_global,
                           const uint8_t* w_codes, const uint8_t* w_scales, const float* w_global,
                           void* out, nvfp4_dtype out_dt, int* path, void* workspace, int64_t workspace_bytes,
                           nvfp4::GemmArgs* g) {
  if (!dtype_ok(out_dt)) return NVFP4_ERR_DTYPE;
  if (!path_ok(*path)) return NVFP4_ERR_DTYPE;
  if (!shape_ok(M, K) || !shape_ok(N, K)) return NVFP4_ERR_SHAPE;
  if (M > 0 && N >= kMaxElems / M) return NVFP4_ERR_SHAPE;
  if (workspace_bytes < 0) return NVFP4_ERR_SHAPE;
  if (*path == NVFP4_PATH_AUTO) *path = M <= 16 ? NVFP4_PATH_SKINNY : NVFP4_PATH_TILED;
  if (grid_rows(*path, M) > kMaxGridY) return NVFP4_ERR_SHAPE;
  g->M = (int)M;
  g->K = (int)K;
  g->N = (int)N;
  if (M == 0 || N == 0) return NVFP4_OK;
  if (!a_codes || !a_scales || !a_global || !w_codes || !w_scales || !w_global || !out)
    return NVFP4_ERR_NULL;
  if (workspace_bytes > 0 && !workspace) return NVFP4_ERR_NULL;
  if (!aligned16(a_codes) || !aligned16(a_scales) || !aligned16(w_codes) ||
      !aligned16(w_scales) || !aligned16(out) || !aligned4(a_global) || !aligned4(w_global) ||
      (workspace && !aligned16(workspace)))
    return NVFP4_ERR_ALIGN;
  g->ac = a_codes;
  g->as = a_scales;
  g->ga = a_global;
  g->wc = w_codes;
  g->ws = w_scales;
  g->gw = w_global;
  g->out = out;
  g->out_bf16 = out_dt == NVFP4_BF16;
  g->workspace = workspace_bytes > 0 ? workspace : nullptr;
  g->workspace_bytes = workspace_bytes;
  if (*path >= NVFP4_KERNEL_GEMV_FP4 && !kernel_takes(*path, *g)) return NVFP4_ERR_SHAPE;
  return NVFP4_OK;
}

// nvfp4_gemm_ex / nvfp4_gemm_ws: validation, then the chosen path or kernel.
nvfp4_status gemm_impl(int64_t M, int64_t K, int64_t N,
                       const uint8_t* a_codes, const uint8_t* a_scales, const float* a_global,
                       const uint8_t* w_codes, const uint8_t* w_scales, const float* w_global,
                       void* out, nvfp4_dtype out_dt, int path, void* workspace, int64_t workspace_bytes,
                       void* stream) {
  nvfp4::GemmArgs g;
  const nvfp4_status st = gemm_validate(M, K, N, a_codes, a_scales, a_global, w_codes, w_scales, w_global, out,
                                        out_dt, &path, workspace, workspace_bytes, &g);
  if (st != NVFP4_OK || g.M == 0 || g.N == 0) return st;
  return from_hip(launch_path(path, g, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

nvfp4_status nvfp4_gemm_ex(int64_t M, int64_t K, int64_t N,
                           const uint8_t* a_codes, const uint8_t* a_scales, const float* a_global,
                           const uint8_t* w_codes, const uint8_t* w_scales, const float* w_global,
                           void* out, nvfp4_dtype out_dt, int path, void* stream) {
  return gemm_impl(M, K, N, a_codes, a_scales, a_global, w_codes, w_scales, w_global, out, out_dt, path,
                   nullptr, 0, stream);
}

int64_t nvfp4_gemm_workspace_bytes(int64_t M, int64_t K, int64_t N) {
  if (M < 3 || M > 16 || !shape_ok(M, K) || !shape_ok(N, K) || N < 1 || N >= kMaxElems / M) return 0;
  nvfp4::GemmArgs g;
  g.M = (int)M;
  g.K = (int)K;
  g.N = (int)N;
  if (nvfp4::gemm_m16_small_prefers_skinny(g)) return 0;  // runs the skinny kernel, unsplit
  return nvfp4::gemm_m16_workspace_bytes(g);
}

int nvfp4_gemm_dispatch(int64_t M, int64_t K, int64_t N, int64_t workspace_bytes) {
  if (M < 1 || N < 1 || !shape_ok(M, K) || !shape_ok(N, K) || N >= kMaxElems / M || workspace_bytes < 0) return 0;
  nvfp4::GemmArgs g;
  g.M = (int)M;
  g.K = (int)K;
  g.N = (int)N;
  g.workspace = workspace_bytes > 0 ? &g : nullptr;  // only its presence and size matter here
  g.workspace_bytes = workspace_bytes;
  if (M > 16) return nvfp4::gemm_tiled_persistent_supported(g) ? NVFP4_KERNEL_TILED_PERSISTENT : NVFP4_KERNEL_TILED;
  return nvfp4::skinny_kernel_choice(g);
}

nvfp4_status nvfp4_gemm_ws(int64_t M, int64_t K, int64_t N,
                           const uint8_t* a_codes, const uint8_t* a_scales, const float* a_global,
                           const uint8_t* w_codes, const uint8_t* w_scales, const float* w_global,
                           void* out, nvfp4_dtype out_dt, void* workspace, int64_t workspace_bytes,
                           void* stream) {
  return gemm_impl(M, K, N, a_codes, a_scales, a_global, w_codes, w_scales, w_global, out, out_dt,
                   NVFP4_PATH_AUTO, workspace, workspace_bytes, stream);
}

nvfp4_status nvfp4_gemm_scratch(int64_t M, int64_t K, int64_t N,
                                const uint8_t* a_codes, const uint8_t* a_scales, const float* a_global,
                                const uint8_t* w_codes, const uint8_t* w_scales, const float* w_global,
                                void* out, nvfp4_dtype out_dt, void* stream) {
  int path = NVFP4_PATH_AUTO;
  nvfp4::GemmArgs g;
  nvfp4_status st = gemm_validate(M, K, N, a_codes, a_scales, a_global, w_codes, w_scales, w_global, out, out_dt,
                                  &path, nullptr, 0, &g);
  if (st != NVFP4_OK || g.M == 0 || g.N == 0) return st;
  const int64_t need = nvfp4_gemm_workspace_bytes(M, K, N);
  if (need > nvfp4::kScratchBytes) return NVFP4_ERR_SCRATCH;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (need > 0) {
    void* ws = nullptr;
    const hipError_t e = nvfp4::scratch_workspace(&ws, s);
    if (e != hipSuccess) return NVFP4_ERR_HIP;
    g.workspace = ws;
    g.workspace_bytes = nvfp4::kScratchBytes;
  }
  return from_hip(launch_path(path, g, s));
}

nvfp4_status nvfp4_gemm_quantize_output(int64_t M, int64_t K, int64_t N,
                                        const uint8_t* a_codes, const uint8_t* a_scales, const float* a_global,
                                        const uint8_t* w_codes, const uint8_t* w_scales, const float* w_global,
                                        void* out, nvfp4_dtype out_dt, const float* y_global, uint8_t* y_codes,
                                        uint8_t* y_scales, void* stream) {
  if (!dtype_ok(out_dt)) return NVFP4_ERR_DTYPE;
  if (!shape_ok(M, K) || !shape_ok(N, K) || !shape_ok(M, N > 0 ? N : 16) || N % 16 != 0) return NVFP4_ERR_SHAPE;
  if (M > 0 && N >= kMaxElems / M) return NVFP4_ERR_SHAPE;
  if ((M <= 16 ? (M + 15) / 16 : (M + 127) / 128) > kMaxGridY) return NVFP4_ERR_SHAPE;
  if (M == 0 || N == 0) return NVFP4_OK;
  if (!a_codes || !a_scales || !a_global || !w_codes || !w_scales || !w_global || !out || !y_global || !y_codes ||
      !y_scales)
    return NVFP4_ERR_NULL;
  if (!aligned16(a_codes) || !aligned16(a_scales) || !aligned16(w_codes) || !aligned16(w_scales) ||
      !aligned16(out) || !aligned4(a_global) || !aligned4(w_global) || !aligned4(y_global) || !aligned16(y_codes) ||
      !aligned16(y_scales))
    return NVFP4_ERR_ALIGN;
  nvfp4::GemmArgs g;
  g.M = (int)M;
  g.K = (int)K;
  g.N = (int)N;
  g.ac = a_codes;
  g.as = a_scales;
  g.ga = a_global;
  g.wc = w_codes;
  g.ws = w_scales;
  g.gw = w_global;
  g.out = out;
  g.out_bf16 = out_dt == NVFP4_BF16;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (M > 16 && nvfp4::gemm_tiled_quant_out_supported(g)) {  // one kernel: quantized in the epilogue
    g.y_global = y_global;
    g.y_codes = y_codes;
    g.y_scales = y_scales;
    return from_hip(nvfp4::launch_gemm_tiled(g, s));
  }
  hipError_t e = M <= 16 ? nvfp4::launch_gemm_skinny(g, s) : nvfp4::launch_gemm_tiled(g, s);
  if (e != hipSuccess) return from_hip(e);
  return from_hip(nvfp4::launch_quantize(out, g.out_bf16, M, N, y_global, y_codes, y_scales, s));
}

nvfp4_status nvfp4_quantize_gemm(int64_t M, int64_t K, int64_t N,
                                 const void* a, nvfp4_dtype a_dt, const float* a_global,
                                 const uint8_t* w_codes, const uint8_t* w_scales, const float* w_global,
                                 void* out, nvfp4_dtype out_dt, uint8_t* a_codes, uint8_t* a_scales,
                                 void* stream) {
  if (!dtype_ok(a_dt) || !dtype_ok(out_dt)) return NVFP4_ERR_DTYPE;
  if (!shape_ok(M, K) || !shape_ok(N, K)) return NVFP4_ERR_SHAPE;
  if (M > 0 && N >= kMaxElems / M) return NVFP4_ERR_SHAPE;
  if ((M <= 16 ? (M + 15) / 16 : (M + 127) / 128) > kMaxGridY) return NVFP4_ERR_SHAPE;
  if (M == 0) return NVFP4_OK;
  if (!a || !a_global || !a_codes || !a_scales) return NVFP4_ERR_NULL;
  if (N > 0 && (!w_codes || !w_scales || !w_global || !out)) return NVFP4_ERR_NULL;
  if (!aligned16(a) || !aligned4(a_global) || !aligned16(a_codes) || !aligned16(a_scales))
    return NVFP4_ERR_ALIGN;
  if (N > 0 && (!aligned16(w_codes) || !aligned16(w_scales) || !aligned16(out) || !aligned4(w_global)))
    return NVFP4_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  nvfp4::GemmArgs g;
  g.M = (int)M;
  g.K = (int)K;
  g.N = (int)N;
  g.ac = a_codes;
  g.as = a_scales;
  g.ga = a_global;
  g.wc = w_codes;
  g.ws = w_scales;
  g.gw = w_global;
  g.out = out;
  g.out_bf16 = out_dt == NVFP4_BF16;
  if (N > 0 && nvfp4::gemv_fp4_supported(g)) {  // one kernel: quantize in its set-up
    g.a_raw = a;
    g.a_raw_bf16 = a_dt == NVFP4_BF16;
    g.ac_out = a_codes;
    g.as_out = a_scales;
    return from_hip(nvfp4::launch_gemv_fp4(g, s));
  }
  hipError_t e = nvfp4::launch_quantize(a, a_dt == NVFP4_BF16, M, K, a_global, a_codes, a_scales, s);
  if (e != hipSuccess || N == 0) return from_hip(e);
  return from_hip(M <= 16 ? nvfp4::launch_gemm_skinny(g, s) : nvfp4::launch_gemm_tiled(g, s));
}

nvfp4_status nvfp4_quantize_gemm_dynamic(int64_t M, int64_t K, int64_t N,
                                         const void* a, nvfp4_dtype a_dt, float* a_global,
                                         const uint8_t* w_codes, const uint8_t* w_scales, const float* w_global,
                                         void* out, nvfp4_dtype out_dt, uint8_t* a_codes, uint8_t* a_scales,
                                         void* stream) {
  if (!dtype_ok(a_dt) || !dtype_ok(out_dt)) return NVFP4_ERR_DTYPE;
  if (!shape_ok(M, K) || !shape_ok(N, K)) return NVFP4_ERR_SHAPE;
  if (M > 0 && N >= kMaxElems / M) return NVFP4_ERR_SHAPE;
  if ((M <= 16 ? (M + 15) / 16 : (M + 127) / 128) > kMaxGridY) return NVFP4_ERR_SHAPE;
  if (!a_global) return NVFP4_ERR_NULL;
  if (!aligned4(a_global)) return NVFP4_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (M == 0) return from_hip(nvfp4::launch_act_global(a, a_dt == NVFP4_BF16, 0, a_global, s));  // g_a = 0
  if (!a || !a_codes || !a_scales) return NVFP4_ERR_NULL;
  if (N > 0 && (!w_codes || !w_scales || !w_global || !out)) return NVFP4_ERR_NULL;
  if (!aligned16(a) || !aligned16(a_codes) || !aligned16(a_scales)) return NVFP4_ERR_ALIGN;
  if (N > 0 && (!aligned16(w_codes) || !aligned16(w_scales) || !aligned16(out) || !aligned4(w_global)))
    return NVFP4_ERR_ALIGN;
  nvfp4::GemmArgs g;
  g.M = (int)M;
  g.K = (int)K;
  g.N = (int)N;
  g.ac = a_codes;
  g.as = a_scales;
  g.ga = a_global;
  g.wc = w_codes;
  g.ws = w_scales;
  g.gw = w_global;
  g.out = out;
  g.out_bf16 = out_dt == NVFP4_BF16;
  if (N > 0 && nvfp4::gemv_fp4_supported(g)) {  // one kernel: scale and quantization in its set-up
    g.a_raw = a;
    g.a_raw_bf16 = a_dt == NVFP4_BF16;
    g.ac_out = a_codes;
    g.as_out = a_scales;
    g.ga_dynamic = a_global;
    return from_hip(nvfp4::launch_gemv_fp4(g, s));
  }
  hipError_t e = nvfp4::launch_act_global(a, a_dt == NVFP4_BF16, M * K, a_global, s);
  if (e == hipSuccess) e = nvfp4::launch_quantize(a, a_dt == NVFP4_BF16, M, K, a_global, a_codes, a_scales, s);
  if (e != hipSuccess || N == 0) return from_hip(e);
  return from_hip(M <= 16 ? nvfp4::launch_gemm_skinny(g, s) : nvfp4::launch_gemm_tiled(g, s));
}

nvfp4_status nvfp4_kv_fp8_encode(const void* x, nvfp4_dtype x_dt, int64_t n, const float* scale, uint8_t* q,
                                 void* stream) {
  if (!dtype_ok(x_dt)) return NVFP4_ERR_DTYPE;
  if (n < 0 || n >= ((int64_t)1 << 40)) return NVFP4_ERR_SHAPE;
  if (n == 0) return NVFP4_OK;
  if (!x || !scale || !q) return NVFP4_ERR_NULL;
  if (!aligned16(x) || !aligned16(q) || !aligned4(scale)) return NVFP4_ERR_ALIGN;
  return from_hip(nvfp4::launch_kv_fp8_encode(x, x_dt == NVFP4_BF16, n, scale, q, static_cast<hipStream_t>(stream)));
}

nvfp4_status nvfp4_kv_fp8_decode(const uint8_t* q, int64_t n, const float* scale, void* x, nvfp4_dtype x_dt,
                                 void* stream) {
  if (!dtype_ok(x_dt)) return NVFP4_ERR_DTYPE;
  if (n < 0 || n >= ((int64_t)1 << 40)) return NVFP4_ERR_SHAPE;
  if (n == 0) return NVFP4_OK;
  if (!x || !scale || !q) return NVFP4_ERR_NULL;
  if (!aligned16(x) || !aligned16(q) || !aligned4(scale)) return NVFP4_ERR_ALIGN;
  return from_hip(nvfp4::launch_kv_fp8_decode(q, n, scale, x, x_dt == NVFP4_BF16, static_cast<hipStream_t>(stream)));
}

nvfp4_status nvfp4_tree_accept(int64_t n_nodes, const int32_t* parent, const int32_t* draft, const int32_t* greedy,
                               int32_t* result, void* stream) {
  if (n_nodes < 1 || n_nodes > 64) return NVFP4_ERR_SHAPE;
  if (!parent || !draft || !greedy || !result) return NVFP4_ERR_NULL;
  if (!aligned4(parent) || !aligned4(draft) || !aligned4(greedy) || !aligned4(result)) return NVFP4_ERR_ALIGN;
  return from_hip(nvfp4::launch_tree_accept((int)n_nodes, parent, draft, greedy, nullptr, nullptr, result,
                                            static_cast<hipStream_t>(stream)));
}

nvfp4_status nvfp4_tree_verify(int64_t M, int64_t K, int64_t N,
                               const uint8_t* a_codes, const uint8_t* a_scales, const float* a_global,
                               const uint8_t* w_codes, const uint8_t* w_scales, const float* w_global,
                               const int32_t* parent, const int32_t* draft, float* logits, int32_t* greedy,
                               int32_t* result, uint64_t* keys, void* stream) {
  if (M < 1 || M > 16 || N < 1 || !shape_ok(M, K) || !shape_ok(N, K) || N >= kMaxElems / M) return NVFP4_ERR_SHAPE;
  if (!a_codes || !a_scales || !a_global || !w_codes || !w_scales || !w_global || !parent || !draft || !greedy ||
      !result || !keys)
    return NVFP4_ERR_NULL;
  if (!aligned16(a_codes) || !aligned16(a_scales) || !aligned16(w_codes) || !aligned16(w_scales) ||
      !aligned4(a_global) || !aligned4(w_global) || !aligned4(parent) || !aligned4(draft) || !aligned4(greedy) ||
      !aligned4(result) || ((uintptr_t)keys & 7u) != 0 || (logits && !aligned16(logits)))
    return NVFP4_ERR_ALIGN;
  nvfp4::GemmArgs g;
  g.M = (int)M;
  g.K = (int)K;
  g.N = (int)N;
  g.ac = a_codes;
  g.as = a_scales;
  g.ga = a_global;
  g.wc = w_codes;
  g.ws = w_scales;
  g.gw = w_global;
  g.out = logits;
  g.out_bf16 = false;
  const bool fused = nvfp4::gemm_m16_supported(g);
  if (!fused && !logits) return NVFP4_ERR_NULL;  // the unfused form needs the logits
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (fused) {
    g.argmax_keys = keys;
    if (nvfp4::gemm_m16_stream_preferred(g)) {  // acceptance fused into the product's last workgroup
      g.tree_parent = parent;
      g.tree_draft = draft;
      g.tree_greedy = greedy;
      g.tree_result = result;
      return from_hip(nvfp4::launch_gemm_m16_stream(g, s));
    }
    e = nvfp4::launch_gemm_m16(g, s);
  } else {
    e = nvfp4::launch_gemm_skinny(g, s);
    if (e == hipSuccess) e = nvfp4::launch_argmax_rows(logits, (int)M, (int)N, keys, s);
  }
  if (e != hipSuccess) return from_hip(e);
  return from_hip(nvfp4::launch_tree_accept((int)M, parent, draft, nullptr, keys, greedy, result, s));
}

nvfp4_status nvfp4_stream_read(const void* a, int64_t a_bytes, const void* b, int64_t b_bytes, uint32_t* sink,
                               uint32_t magic, void* stream) {
  if (a_bytes < 0 || b_bytes < 0 || a_bytes >= kMaxElems || b_bytes >= kMaxElems || a_bytes % 16 || b_bytes % 16)
    return NVFP4_ERR_SHAPE;
  if (!sink || (a_bytes > 0 && !a) || (b_bytes > 0 && !b)) return NVFP4_ERR_NULL;
  if (!aligned4(sink) || (a_bytes > 0 && !aligned16(a)) || (b_bytes > 0 && !aligned16(b))) return NVFP4_ERR_ALIGN;
  return from_hip(nvfp4::launch_read_stream(static_cast<const uint8_t*>(a), a_bytes, static_cast<const uint8_t*>(b),
                                            b_bytes, sink, magic, static_cast<hipStream_t>(stream)));
}

nvfp4_status nvfp4_gemm(int64_t M, int64_t K, int64_t N,
                        const uint8_t* a_codes, const uint8_t* a_scales, const float* a_global,
                        const uint8_t* w_codes, const uint8_t* w_scales, const float* w_global,
                        void* out, nvfp4_dtype out_dt, void* stream) {
  return nvfp4_gemm_ex(M, K, N, a_codes, a_scales, a_global, w_codes, w_scales, w_global, out,
                       out_dt, NVFP4_PATH_AUTO, stream);
}

}  // extern "C"
