// Skinny NVFP4 W4A4 GEMM for gfx950: M <= 16 activation rows against a
// streamed NVFP4 weight matrix.  This is the decode-time product of the page
// "TensorRT Edge-LLM Completes the MLPerf Edge Agentic Benchmark 6.4x Faster
// on Jetson AGX Thor": one row per generated token (section "Using NVFP4
// quantization to accelerate Qwen3.6-27B inference", where low-batch decoding
// is limited by DRAM bandwidth), or 16 rows when the 16-node candidate tree is
// verified in one pass (section "Using tree-based multi-token prediction to
// accelerate LLM inference").  The weight bytes dominate, so the kernel is
// built around streaming them from HBM once with wide coalesced loads and
// enough of them in flight to cover HBM latency.
//
// Work mapping.  A workgroup owns NT tiles of 16 weight rows (output columns)
// and one tile of 16 activation rows; its KW waves split K into interleaved
// "super-steps" of 64*VB elements, and the partial sums are added in a fixed
// order through LDS at the end (deterministic, no atomics).  Inside a wave,
// lane l = r + 16*q streams weight row r of each tile (and activation row r):
// 16*VB contiguous K-elements (8*VB bytes of codes, VB scale bytes) at K
// offset 16*VB*q of the super-step, so the four lanes of a row read one
// contiguous 32*VB-byte run.  Each 8-element slice of a lane's run feeds one
// v_mfma_f32_16x16x32_f16 as that lane's k-group; A and B use the same slice
// for the same MFMA, so the contraction runs over a permutation of K, which
// leaves the sum unchanged.
//
// Latency hiding.  Each wave keeps a ring of D super-steps of loads in flight
// (register slots indexed at compile time): it consumes slot j and refills it
// with the super-step D ahead.  Loads are buffer loads: a load past the end of
// the wave's K range or of the matrix gets an offset outside the buffer, which
// the hardware answers with zeros without touching memory, so the ring needs
// no branches around its loads.
//
// Dequantization: E2M1 -> f16 with the gfx950 packed conversion (unit scale,
// exact), times the E4M3 block scale in f16 (exact: at most 6 significant
// bits in [2^-10, 2688]).  The MFMA products are therefore exact and only the
// fp32 accumulation rounds.  The tensor scales g_a * g_w are applied once in
// the epilogue.
#include <stdlib.h>

#include "device_common.h"
#include "launch.h"

namespace nvfp4 {
namespace {

constexpr int kMaxWavesK = 8;
constexpr uint32_t kOOB = 0x80000000u;  // an offset past every buffer (buffers are < 2^31 bytes)

template <int VB> struct Raw;
template <> struct Raw<2> { u4_t c; uint32_t s; };  // 16 bytes of codes, 2 scale bytes
template <> struct Raw<1> { u2_t c; uint32_t s; };  // 8 bytes of codes, 1 scale byte

// One lane's run: codes at byte offset `co` and scales at `so` of their
// buffers (kOOB for both gives zeros).
template <int VB, int CPOL>
__device__ __forceinline__ Raw<VB> load_run(__amdgpu_buffer_rsrc_t codes, __amdgpu_buffer_rsrc_t scales,
                                            uint32_t co, uint32_t so) {
  Raw<VB> r;
  if constexpr (VB == 2) {
    r.c = __builtin_amdgcn_raw_buffer_load_b128(codes, co, 0, CPOL);
    r.s = __builtin_amdgcn_raw_buffer_load_b16(scales, so, 0, CPOL);
  } else {
    r.c = __builtin_amdgcn_raw_buffer_load_b64(codes, co, 0, CPOL);
    r.s = __builtin_amdgcn_raw_buffer_load_b8(scales, so, 0, CPOL);
  }
  return r;
}

template <int NT, int VB>
struct Slot {
  Raw<VB> a;
  Raw<VB> w[NT];
};

template <int NT, int VB>
__device__ __forceinline__ void mma_slot(const Slot<NT, VB>& s, f4_t (&acc)[NT]) {
  const h2_t sa = e4m3x2_to_h2(s.a.s);
  h2_t sw[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) sw[t] = e4m3x2_to_h2(s.w[t].s);
#pragma unroll
  for (int j = 0; j < 2 * VB; ++j) {
    const h8_t af = dequant8(s.a.c[j], sa[j >> 1]);
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = mfma16x16x32(af, dequant8(s.w[t].c[j], sw[t][j >> 1]), acc[t]);
  }
}

template <int NT, int VB, int D, bool OUT_BF16>
__global__ __launch_bounds__(64 * kMaxWavesK) void gemm_skinny_kernel(GemmArgs p) {
  constexpr int kStep = 64 * VB;  // K-elements per super-step (4 lanes x 16*VB)
  const int lane = threadIdx.x & 63;
  // wave index as a scalar, so that the loop below branches uniformly
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int KW = blockDim.x >> 6;
  const int r = lane & 15, q = lane >> 4;
  const int M = p.M, K = p.K, N = p.N;
  const int n_base = blockIdx.x * (16 * NT);
  const int m_base = blockIdx.y * 16;
  const uint32_t cstride = (uint32_t)K >> 1, sstride = (uint32_t)K >> 4;

  const __amdgpu_buffer_rsrc_t ac = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.ac), (short)0, (int)((uint32_t)M * cstride), 0x00020000);
  const __amdgpu_buffer_rsrc_t as = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.as), (short)0, (int)((uint32_t)M * sstride), 0x00020000);
  const __amdgpu_buffer_rsrc_t wc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.wc), (short)0, (int)((uint32_t)N * cstride), 0x00020000);
  const __amdgpu_buffer_rsrc_t ws = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.ws), (short)0, (int)((uint32_t)N * sstride), 0x00020000);

  // Row bases of this lane (rows outside the matrix read as zeros).
  const int m = m_base + r;
  const bool a_ok = m < M;
  const uint32_t a_cbase = a_ok ? (uint32_t)m * cstride : kOOB;
  const uint32_t a_sbase = a_ok ? (uint32_t)m * sstride : kOOB;
  uint32_t w_cbase[NT], w_sbase[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int n = n_base + 16 * t + r;
    w_cbase[t] = n < N ? (uint32_t)n * cstride : kOOB;
    w_sbase[t] = n < N ? (uint32_t)n * sstride : kOOB;
  }

  // Super-steps of this wave: wave, wave + KW, ...  (the last may be partial).
  const int n_steps = (K + kStep - 1) / kStep;
  const int my_steps = wave < n_steps ? (n_steps - wave + KW - 1) / KW : 0;
  const int lane_k = q * 16 * VB;

  auto load_slot = [&](int i) {
    Slot<NT, VB> s;
    const int k0 = (wave + i * KW) * kStep + lane_k;
    const bool k_ok = i < my_steps && k0 < K;  // K % (16*VB) == 0: a run is all in or all out
    const uint32_t co = (uint32_t)k0 >> 1, so = (uint32_t)k0 >> 4;
    s.a = load_run<VB, 0>(ac, as, k_ok ? a_cbase + co : kOOB, k_ok ? a_sbase + so : kOOB);
#pragma unroll
    for (int t = 0; t < NT; ++t)
      s.w[t] = load_run<VB, 0>(wc, ws, k_ok ? w_cbase[t] + co : kOOB, k_ok ? w_sbase[t] + so : kOOB);
    return s;
  };

  f4_t acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f4_t{0.f, 0.f, 0.f, 0.f};

  // Scheduling fences keep the loads in slot order: loads complete in issue
  // order, so slot j is ready once everything issued before it has returned.
  Slot<NT, VB> ring[D];
#pragma unroll
  for (int j = 0; j < D; ++j) {
    ring[j] = load_slot(j);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int i0 = 0; i0 < my_steps; i0 += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      if (i0 + j < my_steps) mma_slot<NT, VB>(ring[j], acc);
      __builtin_amdgcn_sched_barrier(0);
      ring[j] = load_slot(i0 + j + D);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // Fixed-order reduction of the K-split partial sums.
  __shared__ f4_t red[kMaxWavesK][NT][64];
  if (KW > 1) {
#pragma unroll
    for (int t = 0; t < NT; ++t) red[wave][t][lane] = acc[t];
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      f4_t s = red[0][t][lane];
      for (int w = 1; w < KW; ++w) s += red[w][t][lane];
      acc[t] = s;
    }
  }

  const float gg = (*p.ga) * (*p.gw);
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int n = n_base + 16 * t + r;
    if (n >= N) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int mm = m_base + 4 * q + i;
      if (mm >= M) continue;
      const float v = acc[t][i] * gg;
      const int64_t o = (int64_t)mm * N + n;
      if constexpr (OUT_BF16) {
        reinterpret_cast<uint16_t*>(p.out)[o] = f32_to_bf16_rne(v);
      } else {
        reinterpret_cast<float*>(p.out)[o] = v;
      }
    }
  }
}


// ---------------------------------------------------------------------------
// Fast path for K % 256 == 0: the unit of work is a pair of super-steps (256
// K-elements).  Per unit a lane loads 2 x 16 bytes of codes (its 32 elements
// of each super-step) and ONE 16-byte run of scales covering all 16 blocks of
// the unit (the four lanes of a row load the same 16 bytes, which the memory
// pipeline merges), instead of a 2-byte scale load per super-step: the scale
// requests were as many as the code requests.  Each wave owns a contiguous
// range of units, and a ring of D units of loads is kept in flight.
// ---------------------------------------------------------------------------
struct Unit {
  u4_t c0, c1;  // codes of super-step 0 and 1 (32 elements each)
  u4_t s;       // the 16 scale bytes of the unit
};

template <int NT>
struct USlot {
  Unit a;
  Unit w[NT];
};

__device__ __forceinline__ Unit load_unit(__amdgpu_buffer_rsrc_t codes, __amdgpu_buffer_rsrc_t scales,
                                          uint32_t cbase, uint32_t sbase, bool ok) {
  Unit u;
  u.c0 = __builtin_amdgcn_raw_buffer_load_b128(codes, ok ? cbase : kOOB, 0, 0);
  u.c1 = __builtin_amdgcn_raw_buffer_load_b128(codes, ok ? cbase + 64 : kOOB, 0, 0);
  u.s = __builtin_amdgcn_raw_buffer_load_b128(scales, ok ? sbase : kOOB, 0, 0);
  return u;
}

// Scale bytes of lane group q: blocks 2q, 2q+1 (super-step 0) and 8+2q, 9+2q
// (super-step 1) of the unit's 16.
__device__ __forceinline__ void unit_scales(const u4_t& s, int q, h2_t& s0, h2_t& s1) {
  const uint32_t w0 = (q & 2) ? s.y : s.x;   // bytes 0..7 hold blocks 0..7
  const uint32_t w1 = (q & 2) ? s.w : s.z;   // bytes 8..15 hold blocks 8..15
  const int sh = (q & 1) * 16;
  s0 = e4m3x2_to_h2(w0 >> sh);
  s1 = e4m3x2_to_h2(w1 >> sh);
}

template <int NT>
__device__ __forceinline__ void mma_unit(const USlot<NT>& s, int q, f4_t (&acc)[NT]) {
  h2_t sa0, sa1, sw0[NT], sw1[NT];
  unit_scales(s.a.s, q, sa0, sa1);
#pragma unroll
  for (int t = 0; t < NT; ++t) unit_scales(s.w[t].s, q, sw0[t], sw1[t]);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const h8_t af = dequant8(s.a.c0[j], sa0[j >> 1]);
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = mfma16x16x32(af, dequant8(s.w[t].c0[j], sw0[t][j >> 1]), acc[t]);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const h8_t af = dequant8(s.a.c1[j], sa1[j >> 1]);
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = mfma16x16x32(af, dequant8(s.w[t].c1[j], sw1[t][j >> 1]), acc[t]);
  }
}

template <int NT, int D, bool OUT_BF16>
__global__ __launch_bounds__(64 * kMaxWavesK) void gemm_skinny256_kernel(GemmArgs p) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int KW = blockDim.x >> 6;
  const int r = lane & 15, q = lane >> 4;
  const int M = p.M, K = p.K, N = p.N;
  const int n_base = blockIdx.x * (16 * NT);
  const int m_base = blockIdx.y * 16;
  const uint32_t cstride = (uint32_t)K >> 1, sstride = (uint32_t)K >> 4;

  const __amdgpu_buffer_rsrc_t ac = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.ac), (short)0, (int)((uint32_t)M * cstride), 0x00020000);
  const __amdgpu_buffer_rsrc_t as = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.as), (short)0, (int)((uint32_t)M * sstride), 0x00020000);
  const __amdgpu_buffer_rsrc_t wc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.wc), (short)0, (int)((uint32_t)N * cstride), 0x00020000);
  const __amdgpu_buffer_rsrc_t ws = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.ws), (short)0, (int)((uint32_t)N * sstride), 0x00020000);

  const int m = m_base + r;
  const bool a_ok = m < M;
  const uint32_t a_c = a_ok ? (uint32_t)m * cstride + q * 16 : kOOB;
  const uint32_t a_s = a_ok ? (uint32_t)m * sstride : kOOB;
  uint32_t w_c[NT], w_s[NT];
  bool w_ok[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int n = n_base + 16 * t + r;
    w_ok[t] = n < N;
    w_c[t] = (uint32_t)n * cstride + q * 16;
    w_s[t] = (uint32_t)n * sstride;
  }

  // Contiguous range of units for this wave.
  const int units = K >> 8;
  const int u_begin = (units * wave) / KW, u_end = (units * (wave + 1)) / KW;
  const int my = u_end - u_begin;

  auto load_slot = [&](int i) {
    USlot<NT> s;
    const bool ok = i < my;
    const uint32_t u = (uint32_t)(u_begin + i);
    s.a = load_unit(ac, as, a_c + u * 128, a_s + u * 16, ok && a_ok);
#pragma unroll
    for (int t = 0; t < NT; ++t) s.w[t] = load_unit(wc, ws, w_c[t] + u * 128, w_s[t] + u * 16, ok && w_ok[t]);
    return s;
  };

  f4_t acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f4_t{0.f, 0.f, 0.f, 0.f};

  USlot<NT> ring[D];
#pragma unroll
  for (int j = 0; j < D; ++j) {
    ring[j] = load_slot(j);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int i0 = 0; i0 < my; i0 += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      if (i0 + j < my) mma_unit<NT>(ring[j], q, acc);
      __builtin_amdgcn_sched_barrier(0);
      ring[j] = load_slot(i0 + j + D);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  __shared__ f4_t red[kMaxWavesK][NT][64];
  if (KW > 1) {
#pragma unroll
    for (int t = 0; t < NT; ++t) red[wave][t][lane] = acc[t];
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      f4_t sum = red[0][t][lane];
      for (int w = 1; w < KW; ++w) sum += red[w][t][lane];
      acc[t] = sum;
    }
  }

  const float gg = (*p.ga) * (*p.gw);
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int n = n_base + 16 * t + r;
    if (n >= N) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int mm = m_base + 4 * q + i;
      if (mm >= M) continue;
      const float v = acc[t][i] * gg;
      const int64_t o = (int64_t)mm * N + n;
      if constexpr (OUT_BF16) {
        reinterpret_cast<uint16_t*>(p.out)[o] = f32_to_bf16_rne(v);
      } else {
        reinterpret_cast<float*>(p.out)[o] = v;
      }
    }
  }
}

int env_int(const char* name, int dflt) {
  const char* s = getenv(name);
  return (s && *s) ? atoi(s) : dflt;
}

template <int NT, int VB, int D>
hipError_t launch_cfg(const GemmArgs& a, int kw, hipStream_t stream) {
  const dim3 grid((unsigned)((a.N + 16 * NT - 1) / (16 * NT)), (unsigned)((a.M + 15) / 16));
  const dim3 block(64 * kw);
  if (a.out_bf16) {
    gemm_skinny_kernel<NT, VB, D, true><<<grid, block, 0, stream>>>(a);
  } else {
    gemm_skinny_kernel<NT, VB, D, false><<<grid, block, 0, stream>>>(a);
  }
  return hipGetLastError();
}

template <int VB>
hipError_t launch_vb(const GemmArgs& a, int nt, int kw, hipStream_t stream) {
  switch (nt) {
    case 1: return launch_cfg<1, VB, 8>(a, kw, stream);
    case 2: return launch_cfg<2, VB, 8>(a, kw, stream);
    default: return launch_cfg<4, VB, 4>(a, kw, stream);
  }
}

}  // namespace

template <int NT, int D>
hipError_t launch256(const GemmArgs& a, int kw, hipStream_t stream) {
  const dim3 grid((unsigned)((a.N + 16 * NT - 1) / (16 * NT)), (unsigned)((a.M + 15) / 16));
  const dim3 block(64 * kw);
  if (a.out_bf16) {
    gemm_skinny256_kernel<NT, D, true><<<grid, block, 0, stream>>>(a);
  } else {
    gemm_skinny256_kernel<NT, D, false><<<grid, block, 0, stream>>>(a);
  }
  return hipGetLastError();
}

// Launch choice.  K % 256 == 0 takes the fast path.  Measured on MI355X
// (sweep over NT x D x KW): a few hundred to a few thousand resident waves with
// 2-3 units in flight each do best; deeper rings or more, shorter waves only
// add pressure on the vector L1.  NT = 2 amortizes the activation operand when
// M > 1; KW is the smallest power of two that gives >= 600 waves while every
// wave keeps >= 4 units.  NVFP4_SKINNY_NT, NVFP4_SKINNY_KW and NVFP4_SKINNY_D
// override the choice (tuning knobs; results change only by fp32 summation
// order).  Other K take the general path.
hipError_t launch_gemm_skinny(const GemmArgs& a, hipStream_t stream) {
  const int64_t tiles16 = (a.N + 15) / 16;
  const int64_t mtiles = (a.M + 15) / 16;
  const int e_nt = env_int("NVFP4_SKINNY_NT", 0);
  const int e_kw = env_int("NVFP4_SKINNY_KW", 0);
  const int e_d = env_int("NVFP4_SKINNY_D", 0);
  const bool kw_ok = e_kw == 1 || e_kw == 2 || e_kw == 4 || e_kw == 8;
  if (a.K % 256 == 0) {
    int nt = a.M > 1 ? 2 : 1;
    if (e_nt == 1 || e_nt == 2) nt = e_nt;
    const int64_t wgs = ((tiles16 + nt - 1) / nt) * mtiles;
    const int64_t units = a.K / 256;
    int kw = 1;
    while (kw < kMaxWavesK && wgs * kw < 600 && units / (2 * kw) >= 4) kw *= 2;
    if (kw_ok) kw = e_kw;
    const int d = (e_d == 2 || e_d == 3 || e_d == 4 || e_d == 6) ? e_d : (nt == 1 ? 3 : 2);
    if (nt == 2) {
      switch (d) {
        case 3: return launch256<2, 3>(a, kw, stream);
        case 4: case 6: return launch256<2, 4>(a, kw, stream);
        default: return launch256<2, 2>(a, kw, stream);
      }
    }
    switch (d) {
      case 2: return launch256<1, 2>(a, kw, stream);
      case 4: return launch256<1, 4>(a, kw, stream);
      case 6: return launch256<1, 6>(a, kw, stream);
      default: return launch256<1, 3>(a, kw, stream);
    }
  }
  const int vb = (a.K % 32 == 0) ? 2 : 1;
  int nt = (tiles16 * mtiles >= 1024) ? 2 : 1;
  if (e_nt == 1 || e_nt == 2 || e_nt == 4) nt = e_nt;
  const int64_t wgs = ((tiles16 + nt - 1) / nt) * mtiles;
  const int64_t steps = (a.K + 64 * vb - 1) / (64 * vb);
  int kw = 1;
  while (kw < kMaxWavesK && wgs * kw < 1536 && steps / (2 * kw) >= 4) kw *= 2;
  if (kw_ok) kw = e_kw;
  return vb == 2 ? launch_vb<2>(a, nt, kw, stream) : launch_vb<1>(a, nt, kw, stream);
}

}  // namespace nvfp4
