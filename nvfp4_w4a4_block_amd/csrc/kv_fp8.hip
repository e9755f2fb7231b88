// FP8 E4M3 KV-cache codec.
//
// The page "TensorRT Edge-LLM Completes the MLPerf Edge Agentic Benchmark
// 6.4x Faster on Jetson AGX Thor" (section "Using NVFP4 quantization to
// accelerate Qwen3.6-27B inference") keeps the KV cache in FP8 beside the
// NVFP4 weights and activations.  Here: E4M3FN with one static fp32 decode
// scale s per tensor.  Encode: inv = fl32(1/s) (0 when s == 0), y =
// fl32(x * inv), code = E4M3 of y rounded to nearest even, saturating at 448,
// sign bit of y.  Decode: fl32(e4m3(code) * s), as fp32 or rounded to bf16.
// Both kernels stream: 16 elements per thread per chunk, a few chunks' loads
// in flight per thread, a guarded tail for n % 16.  The streams are read once:
// their loads carry the non-temporal hint (measured 7% faster encode, 12%
// faster decode; the same hint on the stores made the decode slower).
#pragma clang fp contract(off)
#include "device_common.h"
#include "launch.h"

namespace nvfp4 {
namespace {


__device__ __forceinline__ uint32_t encode_e4m3_signed(float y) {
  return e4m3_from_nonneg(__builtin_fabsf(y)) | ((__float_as_uint(y) >> 24) & 0x80u);
}

// Four values -> four E4M3 bytes (value i in byte i) with the hardware
// conversion after clamping to +-448.  On gfx950 this equals
// encode_e4m3_signed for every finite input (checked on 50M inputs: every
// E4M3 midpoint and its float32 neighbours, subnormals, signed zeros and
// saturating values): round to nearest even, and the clamp supplies the
// saturation that the conversion alone would turn into NaN.
__device__ __forceinline__ uint32_t encode4_e4m3(float a, float b, float c, float d) {
  const float lo = -448.0f, hi = 448.0f;
  a = __builtin_fminf(__builtin_fmaxf(a, lo), hi);
  b = __builtin_fminf(__builtin_fmaxf(b, lo), hi);
  c = __builtin_fminf(__builtin_fmaxf(c, lo), hi);
  d = __builtin_fminf(__builtin_fmaxf(d, lo), hi);
  const int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

template <bool BF16>
__device__ __forceinline__ void load16(const void* x, int64_t c, float* v) {
  if constexpr (BF16) {
    const u4_t* p = reinterpret_cast<const u4_t*>(x) + 2 * c;
    const u4_t a = __builtin_nontemporal_load(p), b = __builtin_nontemporal_load(p + 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(a[i] << 16);
      v[2 * i + 1] = __uint_as_float(a[i] & 0xFFFF0000u);
      v[8 + 2 * i] = __uint_as_float(b[i] << 16);
      v[8 + 2 * i + 1] = __uint_as_float(b[i] & 0xFFFF0000u);
    }
  } else {
    const u4_t* p = reinterpret_cast<const u4_t*>(x) + 4 * c;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u4_t a = __builtin_nontemporal_load(p + j);
#pragma unroll
      for (int i = 0; i < 4; ++i) v[4 * j + i] = __uint_as_float(a[i]);
    }
  }
}

template <bool BF16>
__device__ __forceinline__ float load1(const void* x, int64_t i) {
  if constexpr (BF16) return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(x)[i] << 16);
  else return reinterpret_cast<const float*>(x)[i];
}

template <bool BF16, int kChunksPerThread>
__global__ __launch_bounds__(256) void kv_encode_kernel(const void* x, int64_t n, const float* s_ptr, uint8_t* q) {
  const float s = *s_ptr;
  const float inv = s == 0.0f ? 0.0f : 1.0f / s;
  const int64_t chunks = n / 16;
  const int64_t T = (int64_t)gridDim.x * blockDim.x;
  for (int64_t c0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c0 < chunks; c0 += T * kChunksPerThread) {
    float v[kChunksPerThread][16];
#pragma unroll
    for (int u = 0; u < kChunksPerThread; ++u)
      if (c0 + u * T < chunks) load16<BF16>(x, c0 + u * T, v[u]);
#pragma unroll
    for (int u = 0; u < kChunksPerThread; ++u) {
      if (c0 + u * T < chunks) {
        u4_t w;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          w[j] = encode4_e4m3(v[u][4 * j] * inv, v[u][4 * j + 1] * inv, v[u][4 * j + 2] * inv, v[u][4 * j + 3] * inv);
        reinterpret_cast<u4_t*>(q)[c0 + u * T] = w;
      }
    }
  }
  const int64_t i = 16 * chunks + (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // tail (< 16 elements)
  if (blockIdx.x == 0 && i < n) q[i] = (uint8_t)encode_e4m3_signed(load1<BF16>(x, i) * inv);
}

template <bool BF16>
__device__ __forceinline__ void store16(void* x, int64_t c, const float* v) {
  if constexpr (BF16) {
    u4_t a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = (uint32_t)f32_to_bf16_rne(v[2 * i]) | ((uint32_t)f32_to_bf16_rne(v[2 * i + 1]) << 16);
      b[i] = (uint32_t)f32_to_bf16_rne(v[8 + 2 * i]) | ((uint32_t)f32_to_bf16_rne(v[8 + 2 * i + 1]) << 16);
    }
    u4_t* p = reinterpret_cast<u4_t*>(x) + 2 * c;
    p[0] = a;
    p[1] = b;
  } else {
    u4_t* p = reinterpret_cast<u4_t*>(x) + 4 * c;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      p[j] = u4_t{__float_as_uint(v[4 * j]), __float_as_uint(v[4 * j + 1]), __float_as_uint(v[4 * j + 2]),
                  __float_as_uint(v[4 * j + 3])};
  }
}

template <bool BF16, int kChunksPerThread>
__global__ __launch_bounds__(256) void kv_decode_kernel(const uint8_t* q, int64_t n, const float* s_ptr, void* x) {
  const float s = *s_ptr;
  const int64_t chunks = n / 16;
  const int64_t T = (int64_t)gridDim.x * blockDim.x;
  for (int64_t c0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c0 < chunks; c0 += T * kChunksPerThread) {
    u4_t w[kChunksPerThread];
#pragma unroll
    for (int u = 0; u < kChunksPerThread; ++u)
      if (c0 + u * T < chunks) w[u] = __builtin_nontemporal_load(reinterpret_cast<const u4_t*>(q) + c0 + u * T);
#pragma unroll
    for (int u = 0; u < kChunksPerThread; ++u) {
      if (c0 + u * T < chunks) {
        float v[16];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8(w[u][j], false);
          const f2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8(w[u][j], true);
          v[4 * j] = lo.x * s;
          v[4 * j + 1] = lo.y * s;
          v[4 * j + 2] = hi.x * s;
          v[4 * j + 3] = hi.y * s;
        }
        store16<BF16>(x, c0 + u * T, v);
      }
    }
  }
  const int64_t i = 16 * chunks + (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (blockIdx.x == 0 && i < n) {
    const float v = e4m3_to_f32(q[i]) * s;
    if constexpr (BF16) reinterpret_cast<uint16_t*>(x)[i] = f32_to_bf16_rne(v);
    else reinterpret_cast<float*>(x)[i] = v;
  }
}

// Grid-stride launch: at most 16384 workgroups, two 16-element chunks per
// thread and pass with all their loads in flight.  A sweep on MI355X over one
// layer's K and V (48.2M elements) found 2 chunks x 16384 workgroups about 5%
// faster than 4 x 4096 and the other points within noise.
constexpr int kKvChunks = 2;
constexpr int64_t kKvMaxGrid = 16384;

unsigned grid_for(int64_t n) {
  const int64_t chunks = n / 16;
  int64_t g = (chunks + 255) / 256;
  if (g > kKvMaxGrid) g = kKvMaxGrid;
  return (unsigned)(g < 1 ? 1 : g);
}

}  // namespace

hipError_t launch_kv_fp8_encode(const void* x, bool bf16, int64_t n, const float* scale, uint8_t* q,
                                hipStream_t stream) {
  if (bf16) kv_encode_kernel<true, kKvChunks><<<grid_for(n), 256, 0, stream>>>(x, n, scale, q);
  else kv_encode_kernel<false, kKvChunks><<<grid_for(n), 256, 0, stream>>>(x, n, scale, q);
  return hipGetLastError();
}

hipError_t launch_kv_fp8_decode(const uint8_t* q, int64_t n, const float* scale, void* x, bool bf16,
                                hipStream_t stream) {
  if (bf16) kv_decode_kernel<true, kKvChunks><<<grid_for(n), 256, 0, stream>>>(q, n, scale, x);
  else kv_decode_kernel<false, kKvChunks><<<grid_for(n), 256, 0, stream>>>(q, n, scale, x);
  return hipGetLastError();
}

}  // namespace nvfp4
