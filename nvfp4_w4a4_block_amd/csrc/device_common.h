// Device-side helpers shared by the NVFP4 kernels (gfx950 / CDNA4).
//
// NVFP4 as used for weights and activations on the page "TensorRT Edge-LLM
// Completes the MLPerf Edge Agentic Benchmark 6.4x Faster on Jetson AGX Thor"
// (section "Using NVFP4 quantization to accelerate Qwen3.6-27B inference"),
// with the public bit definition: E2M1 elements, one E4M3 scale per 16
// contiguous K-elements, one fp32 tensor scale.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef float f2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u2_t __attribute__((ext_vector_type(2)));

constexpr int kBlock = 16;          // K-elements per E4M3 scale
constexpr float kE4M3Max = 448.0f;  // largest finite E4M3FN magnitude

// ---------------------------------------------------------------------------
// Encoders (used by the quantization kernels; every step is exact or
// correctly rounded fp32, so the bytes are reproducible on any IEEE machine).
// ---------------------------------------------------------------------------

// Non-negative fp32 -> E4M3FN byte, round to nearest even, saturating at 448.
// Values below 2^-6 land on the subnormal grid m * 2^-9 (m = 0..8; m = 8 is
// the smallest normal, whose byte is also 8).  Larger values keep 3 of fp32's
// 23 mantissa bits with a round-half-even carry into the exponent.
__device__ __forceinline__ uint32_t e4m3_from_nonneg(float s) {
  if (!(s < kE4M3Max)) return 0x7Eu;
  if (s < 0.015625f) return (uint32_t)__builtin_rintf(s * 512.0f);
  const uint32_t b = __float_as_uint(s);
  const uint32_t r = b + 0x7FFFFu + ((b >> 20) & 1u);
  return ((((r >> 23) - 120u) << 3) | ((r >> 20) & 7u));
}

// E4M3FN byte (finite) -> fp32, exact (hardware OCP fp8 conversion).
__device__ __forceinline__ float e4m3_to_f32(uint32_t byte) {
  return __builtin_amdgcn_cvt_f32_fp8(byte, 0);
}

// fp32 -> E2M1 code, round to nearest even, saturating at 6; sign bit taken
// from the input's sign bit.  Decision points are the midpoints between the
// magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}; a midpoint goes to the even code.
// gfx950's v_cvt_scalef32_pk_fp4_f32 with a unit scale is this function: it
// was checked equal to the compare ladder
//   c = (a > .25) + (a >= .75) + (a > 1.25) + (a >= 1.75) + (a > 2.5) + (a >= 3.5) + (a > 5),
//   a = |y|, code = c | sign bit << 3
// on every finite fp32 value (4,278,190,080 of them).  One instruction
// converts two values into one byte of a word; the other bytes are kept.
__device__ __forceinline__ uint32_t e2m1_from_f32(float y) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, y, 0.0f, 1.0f, 0) & 0xFu;
}

// Eight values -> their E2M1 codes, element j in nibble j of the word.
__device__ __forceinline__ uint32_t e2m1x8_from_f32(const float (&y)[8]) {
  uint32_t w = 0u;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[0], y[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[2], y[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[4], y[5], 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[6], y[7], 1.0f, 3);
  return w;
}

// ---------------------------------------------------------------------------
// Dequantization to MFMA operands.
// One 16-block x[0..15] with decode scale g -> its E4M3 scale byte (returned)
// and 16 E2M1 codes in two words (element 2j in the low nibble of byte j).
// The same fp32 sequence as every quantizer in this library: amax, s =
// (amax / 6) / g, scale byte, d = sv * g, inv = 1 / d, codes of x_i * inv.
// Each step is one correctly rounded operation (the library is built with
// correctly rounded division); there is no sum, so nothing can be contracted
// into a fused multiply-add.
__device__ __forceinline__ uint32_t quantize_block16(const float* x, float g, uint32_t& w0, uint32_t& w1) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(x[i]));
  const float s = (g == 0.0f) ? 0.0f : (amax / 6.0f) / g;
  const uint32_t sb = e4m3_from_nonneg(s);
  const float d = e4m3_to_f32(sb) * g;
  const float inv = (d == 0.0f) ? 0.0f : 1.0f / d;
  float y0[8], y1[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    y0[i] = x[i] * inv;
    y1[i] = x[8 + i] * inv;
  }
  w0 = e2m1x8_from_f32(y0);
  w1 = e2m1x8_from_f32(y1);
  return sb;
}

// ---------------------------------------------------------------------------

// Two E4M3 scale bytes (low two bytes of `w`) -> f16 pair, exact: every E4M3
// value (2^-9 .. 448) is a normal f16.
__device__ __forceinline__ h2_t e4m3x2_to_h2(uint32_t w) {
  const f2_t f = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
  return h2_t{(_Float16)f.x, (_Float16)f.y};
}

// Eight packed E2M1 codes (a 32-bit word, element 2j in the low nibble of
// byte j) times one block scale `s` -> eight f16 values in k order.
// The gfx950 conversion is exact for a unit scale (it only honours the
// exponent of its scale operand), so the E4M3 scale is applied with a packed
// f16 multiply; the product e2m1 * e4m3 has at most 6 significant bits and
// lies in [2^-10, 2688], so it is exact in f16.
__device__ __forceinline__ h8_t dequant8(uint32_t w, _Float16 s) {
  const h2_t s2 = {s, s};
  const h2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2;
  const h2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2;
  const h2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2;
  const h2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2;
  return h8_t{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t b = __float_as_uint(f);
  return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

// Argmax key of logit v at column n: the float's bits mapped to an unsigned
// order (negative values below positive ones, -0 just below +0) in the high
// word and the complement of n in the low word, so that the maximum key is the
// largest value at its lowest column.  Keys of finite values are never 0.
__device__ __forceinline__ uint64_t argmax_key(float v, uint32_t n) {
  const uint32_t b = __float_as_uint(v);
  const uint32_t ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((uint64_t)ord << 32) | (uint64_t)(0xFFFFFFFFu - n);
}

__device__ __forceinline__ f4_t mfma16x16x32(h8_t a, h8_t b, f4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Greedy acceptance of a candidate tree (page "TensorRT Edge-LLM Completes
// the MLPerf Edge Agentic Benchmark 6.4x Faster on Jetson AGX Thor", section
// "Using tree-based multi-token prediction to accelerate LLM inference"),
// run by one whole wave: lane v < n holds node v's parent index, draft token
// and greedy token (n <= 64, nodes in topological order, node 0 the root).
// Node u is accepted when its parent is and its draft equals the parent's
// greedy token; a parent outside [0, u) rejects it.  result = [end, L,
// bonus, path[0 .. L-1], -1 ...] (3 + n entries): the deepest accepted node
// (lowest index on ties), its depth, its greedy token, and the nodes at depths
// 1 .. L on the way to it.  The walk runs in node order in scalar registers,
// reading the parent's acceptance bit, depth and greedy token across lanes.
__device__ __forceinline__ void tree_walk_wave(int n, int32_t par, int32_t dr, int32_t gv, int32_t* result) {
  const int t = (int)(threadIdx.x & 63);
  uint64_t okm = 1;     // bit v: node v accepted (the root is)
  int32_t depth_v = 0;  // lane v: depth of node v
  int end = 0, dend = 0;
  for (int u = 1; u < n; ++u) {
    const int pu = __builtin_amdgcn_readlane(par, u);
    const bool valid = pu >= 0 && pu < u;
    const int ps = valid ? pu : 0;
    const int d = valid ? __builtin_amdgcn_readlane(depth_v, ps) + 1 : 0;
    depth_v = t == u ? d : depth_v;
    const bool ok = valid && ((okm >> ps) & 1ull) &&
                    __builtin_amdgcn_readlane(dr, u) == __builtin_amdgcn_readlane(gv, ps);
    if (ok) {
      okm |= 1ull << u;
      if (d > dend) {
        end = u;
        dend = d;
      }
    }
  }
  // Lane i < L: the node at depth i + 1 on the root-to-end path; -1 beyond.
  int32_t path_v = -1;
  int u = end;
  for (int i = dend - 1; i >= 0; --i) {
    path_v = t == i ? u : path_v;
    u = __builtin_amdgcn_readlane(par, u);
  }
  if (t == 0) {
    result[0] = end;
    result[1] = dend;
    result[2] = __builtin_amdgcn_readlane(gv, end);
  }
  if (t < n) result[3 + t] = path_v;
}

}  // namespace nvfp4
