// NVFP4 quantization kernels for gfx950: weight tensor-scale reduction and
// the per-16-block quantizer shared by weights and activations.
//
// Follows the NVFP4 quantization of weights (once, after training) and of
// activations on the page "TensorRT Edge-LLM Completes the MLPerf Edge Agentic
// Benchmark 6.4x Faster on Jetson AGX Thor", section "Using NVFP4 quantization
// to accelerate Qwen3.6-27B inference".  Every float step is a correctly
// rounded fp32 operation with no contraction into fused multiply-adds (this
// file is built with -ffp-contract=off and correctly rounded division), so
// the codes and scales are reproducible bit for bit.
#include "device_common.h"
#include "launch.h"

#pragma clang fp contract(off)

namespace nvfp4 {
namespace {

constexpr int kQuantThreads = 256;

// Eight consecutive inputs as fp32 (bf16 widens exactly).
__device__ __forceinline__ void load8(const float* p, float v[8]) {
  const f4_t a = *reinterpret_cast<const f4_t*>(p);
  const f4_t b = *reinterpret_cast<const f4_t*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void load8(const uint16_t* p, float v[8]) {
  const u4_t w = *reinterpret_cast<const u4_t*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

// One lane quantizes 8 elements; the lane pair (2j, 2j+1) holds 16-block j of
// the flattened [rows][K] tensor (K % 16 == 0, so blocks never straddle rows).
// The pair exchanges its partial amax, both lanes derive the same scale, each
// stores its 4 bytes of packed codes and the even lane stores the scale byte.
template <typename In>
__global__ __launch_bounds__(kQuantThreads) void quant_blocks_kernel(
    const In* __restrict__ x, int64_t n8, const float* __restrict__ g_ptr,
    uint32_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int64_t t = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x;
  const bool valid = t < n8;
  // Lanes past the end read the first run (n8 > 0) and use zeros; without a
  // branch around the load, and with the tensor scale fetched by a vector load
  // issued right behind it, the two memory round trips overlap (a scalar load
  // of the scale was waited for before the data load could start).
  float v[8];
  load8(x + (valid ? t : 0) * 8, v);
  const __amdgpu_buffer_rsrc_t gr =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(g_ptr), (short)0, 4, 0x00020000);
  const float g = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(gr, 0, 0, 0));
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = valid ? v[i] : 0.0f;
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[i]));
  // n8 is even and waves hold an even number of lanes, so both lanes of a
  // pair are valid or both are not; every lane takes part in the exchange.
  amax = __builtin_fmaxf(amax, __shfl_xor(amax, 1));

  const float s = (g == 0.0f) ? 0.0f : (amax / 6.0f) / g;
  const uint32_t sb = e4m3_from_nonneg(s);
  const float d = e4m3_to_f32(sb) * g;
  const float inv = (d == 0.0f) ? 0.0f : 1.0f / d;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] *= inv;
  const uint32_t word = e2m1x8_from_f32(v);
  if (valid) {
    codes[t] = word;
    if ((t & 1) == 0) scales[t >> 1] = (uint8_t)sb;
  }
}

__global__ void zero_word_kernel(uint32_t* p) { *p = 0u; }

// Largest |x| over the tensor, accumulated into *acc as fp32 bits with an
// unsigned atomic max (non-negative floats order like their bit patterns, so
// the result does not depend on the order of the updates).
template <typename In>
__global__ __launch_bounds__(kQuantThreads) void amax_kernel(const In* __restrict__ x, int64_t n8,
                                                             uint32_t* __restrict__ acc) {
  float m = 0.0f;
  for (int64_t t = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x; t < n8;
       t += (int64_t)gridDim.x * kQuantThreads) {
    float v[8];
    load8(x + t * 8, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) m = __builtin_fmaxf(m, __builtin_fabsf(v[i]));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = __builtin_fmaxf(m, __shfl_xor(m, off));
  __shared__ float wave_max[kQuantThreads / 64];
  if ((threadIdx.x & 63) == 0) wave_max[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float b = wave_max[0];
#pragma unroll
    for (int i = 1; i < kQuantThreads / 64; ++i) b = __builtin_fmaxf(b, wave_max[i]);
    atomicMax(acc, __float_as_uint(b));
  }
}

// g_w = fl32(amax / 2688), 2688 = 6 * 448, written over the amax bits.
__global__ void finalize_global_kernel(uint32_t* p) {
  const float amax = __uint_as_float(*p);
  *reinterpret_cast<float*>(p) = amax / 2688.0f;
}

// One workgroup computes g = fl32(amax / 2688) of a small tensor directly (no
// atomics, no clearing launch): the decode step's single activation row.
constexpr int kSmallAmaxThreads = 1024;
constexpr int64_t kSmallAmaxMax = (int64_t)1 << 20;  // elements served by one workgroup

template <typename In>
__global__ __launch_bounds__(kSmallAmaxThreads) void amax_small_kernel(const In* __restrict__ x, int64_t n8,
                                                                       float* __restrict__ g) {
  float m = 0.0f;
  for (int64_t t = threadIdx.x; t < n8; t += kSmallAmaxThreads) {
    float v[8];
    load8(x + t * 8, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) m = __builtin_fmaxf(m, __builtin_fabsf(v[i]));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = __builtin_fmaxf(m, __shfl_xor(m, off));
  __shared__ float wave_max[kSmallAmaxThreads / 64];
  if ((threadIdx.x & 63) == 0) wave_max[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float b = wave_max[0];
#pragma unroll
    for (int i = 1; i < kSmallAmaxThreads / 64; ++i) b = __builtin_fmaxf(b, wave_max[i]);
    *g = b / 2688.0f;
  }
}

template <typename In>
hipError_t launch_quant_blocks(const void* x, int64_t elems, const float* g, uint8_t* codes,
                               uint8_t* scales, hipStream_t stream) {
  const int64_t n8 = elems / 8;
  if (n8 == 0) return hipSuccess;
  const int64_t grid = (n8 + kQuantThreads - 1) / kQuantThreads;
  quant_blocks_kernel<In><<<dim3((unsigned)grid), dim3(kQuantThreads), 0, stream>>>(
      static_cast<const In*>(x), n8, g, reinterpret_cast<uint32_t*>(codes), scales);
  return hipGetLastError();
}

template <typename In>
hipError_t launch_amax(const void* x, int64_t elems, uint32_t* acc, hipStream_t stream) {
  const int64_t n8 = elems / 8;
  zero_word_kernel<<<1, 1, 0, stream>>>(acc);
  if (n8 > 0) {
    int64_t grid = (n8 + kQuantThreads - 1) / kQuantThreads;
    if (grid > 4096) grid = 4096;  // grid-stride: 16 workgroups per CU is plenty
    amax_kernel<In><<<dim3((unsigned)grid), dim3(kQuantThreads), 0, stream>>>(
        static_cast<const In*>(x), n8, acc);
  }
  finalize_global_kernel<<<1, 1, 0, stream>>>(acc);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize(const void* x, bool bf16, int64_t rows, int64_t K, const float* g,
                           uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  const int64_t elems = rows * K;
  return bf16 ? launch_quant_blocks<uint16_t>(x, elems, g, codes, scales, stream)
              : launch_quant_blocks<float>(x, elems, g, codes, scales, stream);
}

hipError_t launch_act_global(const void* a, bool bf16, int64_t elems, float* g, hipStream_t stream) {
  if (elems > kSmallAmaxMax) return launch_weight_global(a, bf16, elems, g, stream);
  if (bf16) amax_small_kernel<uint16_t><<<1, kSmallAmaxThreads, 0, stream>>>(static_cast<const uint16_t*>(a), elems / 8, g);
  else amax_small_kernel<float><<<1, kSmallAmaxThreads, 0, stream>>>(static_cast<const float*>(a), elems / 8, g);
  return hipGetLastError();
}

hipError_t launch_weight_global(const void* w, bool bf16, int64_t elems, float* g,
                                hipStream_t stream) {
  uint32_t* acc = reinterpret_cast<uint32_t*>(g);
  return bf16 ? launch_amax<uint16_t>(w, elems, acc, stream)
              : launch_amax<float>(w, elems, acc, stream);
}

}  // namespace nvfp4
