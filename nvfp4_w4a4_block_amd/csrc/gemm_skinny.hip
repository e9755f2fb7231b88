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

// Fragments of the activation operand read from an f16 copy in LDS (see the
// ALDS mode below): a0 / a1 point at lane (r, q)'s 32 elements of super-step
// 0 / 1 of the unit (K offsets 32*q and 128 + 32*q), the same slices the
// weight lanes use; both point at a 64-byte zero run for rows >= M.
template <int NT>
__device__ __forceinline__ void mma_unit_lds(const Unit (&w)[NT], const _Float16* a0, const _Float16* a1,
                                             int q, f4_t (&acc)[NT]) {
  h2_t sw0[NT], sw1[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) unit_scales(w[t].s, q, sw0[t], sw1[t]);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const h8_t af = *reinterpret_cast<const h8_t*>(a0 + 8 * j);
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = mfma16x16x32(af, dequant8(w[t].c0[j], sw0[t][j >> 1]), acc[t]);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const h8_t af = *reinterpret_cast<const h8_t*>(a1 + 8 * j);
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = mfma16x16x32(af, dequant8(w[t].c1[j], sw1[t][j >> 1]), acc[t]);
  }
}

// ALDS: the activation rows are few (M * K * 2 bytes fit in LDS), so each wave
// dequantizes the rows of its own K range once into LDS as f16, and its lanes
// read ready MFMA fragments (rows >= M read a zero run) instead of converting
// all 16 rows of the activation operand per weight tile.  Without ALDS the
// activation runs travel in the ring with the weights and every wave converts
// them.
template <int NT, int D, bool ALDS, bool OUT_BF16>
__global__ __launch_bounds__(64 * kMaxWavesK) void gemm_skinny256_kernel(GemmArgs p) {
  extern __shared__ __attribute__((aligned(16))) _Float16 a_lds[];
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

  // ALDS fill: rows m_base .. m_base + mrows - 1 of this wave's K range, f16,
  // row-major with a row stride of (max units per wave) * 256 elements.  A
  // 64-byte zero run after all waves' rows serves the rows >= M.
  const int mrows = M - m_base < 16 ? M - m_base : 16;
  const int u_cap = (units + KW - 1) / KW;
  const int row_len = u_cap * 256;
  _Float16* wave_a = a_lds + (size_t)wave * mrows * row_len;
  const _Float16* zero_run = a_lds + (size_t)KW * mrows * row_len;
  if constexpr (ALDS) {
    if (wave == 0 && lane < 16) reinterpret_cast<uint32_t*>(const_cast<_Float16*>(zero_run))[lane] = 0u;
    const int blocks = mrows * my * 16;  // 16-element blocks to convert
    for (int b = lane; b < blocks; b += 64) {
      const int row = b / (my * 16), kb = b - row * (my * 16);
      const uint32_t g_row = (uint32_t)(m_base + row);
      const uint32_t k0 = (uint32_t)(u_begin * 256 + kb * 16);
      const u2_t c = __builtin_amdgcn_raw_buffer_load_b64(ac, g_row * cstride + (k0 >> 1), 0, 0);
      const uint32_t sb = __builtin_amdgcn_raw_buffer_load_b8(as, g_row * sstride + (k0 >> 4), 0, 0);
      const _Float16 sc = (_Float16)e4m3_to_f32(sb);
      h8_t* dst = reinterpret_cast<h8_t*>(wave_a + row * row_len + kb * 16);
      dst[0] = dequant8(c.x, sc);
      dst[1] = dequant8(c.y, sc);
    }
    __syncthreads();  // the zero run is written by wave 0
  }

  auto load_slot = [&](int i) {
    USlot<NT> s;
    const bool ok = i < my;
    const uint32_t u = (uint32_t)(u_begin + i);
    if constexpr (!ALDS) s.a = load_unit(ac, as, a_c + u * 128, a_s + u * 16, ok && a_ok);
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
      if (i0 + j < my) {
        if constexpr (ALDS) {
          const bool live = r < mrows;
          const _Float16* a0 = live ? wave_a + r * row_len + (i0 + j) * 256 + 32 * q : zero_run;
          const _Float16* a1 = live ? a0 + 128 : zero_run;
          mma_unit_lds<NT>(ring[j].w, a0, a1, q, acc);
        } else {
          mma_unit<NT>(ring[j], q, acc);
        }
      }
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

// ---------------------------------------------------------------------------
// Memory-order GEMV for M <= 2 (single-stream decode), K >= 2048, K % 256 == 0.
// Measured on MI355X: reading the weight matrix as many rows at once in
// 256-byte pieces leaves DRAM pages mostly unused (request latency ~3x that
// of a sequential read), so here every wave streams a contiguous run of R
// whole rows in memory order, 1 KB per instruction (lane l takes 16 bytes =
// 32 codes).  Chunk q of the run belongs to row
// q / (K/32) at K offset 32 * (q % (K/32)); its activation values come from
// an f16 copy in LDS.  Its two scale bytes sit at byte 2q of the scale array,
// so the scales of 8 instructions form one contiguous kilobyte, fetched with
// a single 16-byte-per-lane load and staged in LDS (per-lane 2-byte loads
// of the scales cost as much time as the codes themselves).  Each lane accumulates the chunks of its current row
// and, when its row changes, parks the partial sum in a per-row LDS slot;
// the R row sums are then added over the 64 slots in a fixed order, so the
// result does not depend on timing.  Arithmetic as in the other GEMVs: exact
// f16 pairs, v_dot2 into fp32 per 16-block, one FMA with the block scale.
// ---------------------------------------------------------------------------
constexpr int kFlatAB = 8;  // activation blocks per thread in the fill

template <int MR, int CPOL, bool OUT_BF16>
__global__ __launch_bounds__(512) void gemv_flat_kernel(GemmArgs p, int R) {
  // LDS: f16 activations as 4 planes per row, [m][t][chunk][8 values] with
  // plane t holding elements 8t..8t+7 of every 32-element chunk, so that a
  // lane reading its chunk's plane t reads the 16 bytes next to its
  // neighbours' (conflict-free); then the per-wave row slots.
  extern __shared__ __attribute__((aligned(16))) h8_t fa_planes[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int M = p.M, K = p.K, N = p.N;
  const uint32_t cstride = (uint32_t)K >> 1, sstride = (uint32_t)K >> 4;
  const int cpr = K >> 5;                        // 16-byte chunks per row
  const int row0 = (blockIdx.x * (blockDim.x >> 6) + wave) * R;
  const int n_chunks = R * cpr;                  // chunks of this wave's run
  const int n_instr = (n_chunks + 63) >> 6;
  const uint32_t qbase = (uint32_t)row0 * (uint32_t)cpr;

  const __amdgpu_buffer_rsrc_t ac = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.ac), (short)0, (int)((uint32_t)M * cstride), 0x00020000);
  const __amdgpu_buffer_rsrc_t as = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.as), (short)0, (int)((uint32_t)M * sstride), 0x00020000);
  const __amdgpu_buffer_rsrc_t wc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.wc), (short)0, (int)((uint32_t)N * cstride), 0x00020000);
  const __amdgpu_buffer_rsrc_t ws = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.ws), (short)0, (int)((uint32_t)N * sstride), 0x00020000);

  // Chunks past the run (or rows past N, which lie past the buffers) read zeros.
  auto load = [&](int i) {
    const int qi = 64 * i + lane;
    const bool ok = i < n_instr && qi < n_chunks;
    const uint32_t q = qbase + (uint32_t)qi;
    return __builtin_amdgcn_raw_buffer_load_b128(wc, ok ? q * 16 : kOOB, 0, CPOL);
  };
  // The two scale bytes of chunk q sit at byte 2q of the scale array, so the
  // scales of 8 consecutive instructions (512 chunks) are one contiguous
  // kilobyte: one 16-byte load per lane fetches them, and the wave parks them
  // in its own LDS kilobyte.  With K % 256 == 0 every window starts on a
  // 16-byte boundary and the array length is a multiple of 16, so a lane's
  // load lies wholly inside or wholly past the array (the buffer range check
  // zeroes a load that crosses the end, in-range bytes included).
  const uint32_t s_total = (uint32_t)N * sstride;
  auto load_scales = [&](int g) {
    const uint32_t off = 2 * (qbase + 512 * (uint32_t)g) + 16 * lane;
    const bool ok = 512 * g + 8 * lane < n_chunks && off < s_total;
    return __builtin_amdgcn_raw_buffer_load_b128(ws, ok ? off : kOOB, 0, CPOL);
  };

  // Activation blocks of this thread first (straight-line: a fixed number of
  // loads, blocks past the end read zeros), then the weight ring, so that
  // the fill below waits for the activation loads only.
  const int a_blocks = M * (K >> 4);
  u2_t a_code[kFlatAB];
  uint32_t a_sb[kFlatAB];
#pragma unroll
  for (int t = 0; t < kFlatAB; ++t) {
    const uint32_t blk = threadIdx.x + t * blockDim.x;
    const bool ok = (int)blk < a_blocks;
    const uint32_t m = blk / sstride, kb = blk - m * sstride;
    a_code[t] = __builtin_amdgcn_raw_buffer_load_b64(ac, ok ? m * cstride + kb * 8 : kOOB, 0, 0);
    a_sb[t] = __builtin_amdgcn_raw_buffer_load_b8(as, ok ? m * sstride + kb : kOOB, 0, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  u4_t sreg = load_scales(0);
  __builtin_amdgcn_sched_barrier(0);
  u4_t ring[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    ring[j] = load(j);
    __builtin_amdgcn_sched_barrier(0);
  }
  // f16 activation planes (once per workgroup).
#pragma unroll
  for (int t = 0; t < kFlatAB; ++t) {
    const uint32_t blk = threadIdx.x + t * blockDim.x;
    if ((int)blk < a_blocks) {
      const uint32_t m = blk / sstride, kb = blk - m * sstride;
      const _Float16 sc = (_Float16)e4m3_to_f32(a_sb[t]);
      const uint32_t chunk = kb >> 1, t0 = 2 * (kb & 1);
      fa_planes[(m * 4 + t0) * cpr + chunk] = dequant8(a_code[t].x, sc);
      fa_planes[(m * 4 + t0 + 1) * cpr + chunk] = dequant8(a_code[t].y, sc);
    }
  }
  float* slots = reinterpret_cast<float*>(fa_planes + M * 4 * cpr) + wave * (R * MR * 64);
  u4_t* s_stage = reinterpret_cast<u4_t*>(reinterpret_cast<float*>(fa_planes + M * 4 * cpr) + (blockDim.x >> 6) * (R * MR * 64)) + wave * 64;
  const uint16_t* s_bytes = reinterpret_cast<const uint16_t*>(s_stage);
  for (int j = 0; j < R * MR; ++j) slots[j * 64 + lane] = 0.f;
  __syncthreads();

  // Lane state: its current row (local) and K-chunk within that row.
  int row_l = lane / cpr;
  int kc = lane - row_l * cpr;
  float acc[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) acc[m] = 0.f;

  auto consume = [&](const u4_t& c, int j) {
    h8_t av[MR][4];
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
      for (int t = 0; t < 4; ++t) av[m][t] = fa_planes[((m < M ? m : 0) * 4 + t) * cpr + kc];
    const f2_t sw = __builtin_amdgcn_cvt_pk_f32_fp8(s_bytes[64 * j + lane], false);
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      float p0[MR], p1[MR];
#pragma unroll
      for (int m = 0; m < MR; ++m) { p0[m] = 0.f; p1[m] = 0.f; }
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        const uint32_t word = c[2 * b + d];
        const h2_t w0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 0);
        const h2_t w1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 1);
        const h2_t w2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 2);
        const h2_t w3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 3);
#pragma unroll
        for (int m = 0; m < MR; ++m) {
          const h8_t& v = av[m][2 * b + d];   // plane 2b+d: elements 16b + 8d .. +7
          p0[m] = __builtin_amdgcn_fdot2(h2_t{v[0], v[1]}, w0, p0[m], false);
          p1[m] = __builtin_amdgcn_fdot2(h2_t{v[2], v[3]}, w1, p1[m], false);
          p0[m] = __builtin_amdgcn_fdot2(h2_t{v[4], v[5]}, w2, p0[m], false);
          p1[m] = __builtin_amdgcn_fdot2(h2_t{v[6], v[7]}, w3, p1[m], false);
        }
      }
#pragma unroll
      for (int m = 0; m < MR; ++m) acc[m] = __builtin_fmaf(p0[m] + p1[m], b ? sw.y : sw.x, acc[m]);
    }
    // advance to the next instruction's chunk (64 chunks later; cpr >= 64)
    kc += 64;
    if (kc >= cpr) {
      if (row_l < R) {
#pragma unroll
        for (int m = 0; m < MR; ++m) slots[(row_l * MR + m) * 64 + lane] = acc[m];
      }
#pragma unroll
      for (int m = 0; m < MR; ++m) acc[m] = 0.f;
      kc -= cpr;
      ++row_l;
    }
  };

  for (int i0 = 0; i0 < n_instr; i0 += 8) {
    s_stage[lane] = sreg;              // scales of instructions i0 .. i0+7
    sreg = load_scales((i0 >> 3) + 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (i0 + j < n_instr) consume(ring[j], j);
      __builtin_amdgcn_sched_barrier(0);
      ring[j] = load(i0 + j + 8);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if (row_l < R) {  // the last row of this lane, if it did not wrap at the end
#pragma unroll
    for (int m = 0; m < MR; ++m) slots[(row_l * MR + m) * 64 + lane] = acc[m];
  }
  // Same-wave LDS ops are ordered; row (lane / MR, m = lane % MR) sums its 64 slots in order.
  if (lane >= R * MR) return;
  const int row = lane / MR, m = lane % MR;
  const f4_t* sl = reinterpret_cast<const f4_t*>(slots + (row * MR + m) * 64);
  float sum = 0.f;
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    const f4_t v = sl[t];
    sum += v.x; sum += v.y; sum += v.z; sum += v.w;
  }
  const int n = row0 + row;
  if (n < N && m < M) {
    const float v = sum * ((*p.ga) * (*p.gw));
    const int64_t o = (int64_t)m * N + n;
    if constexpr (OUT_BF16) {
      reinterpret_cast<uint16_t*>(p.out)[o] = f32_to_bf16_rne(v);
    } else {
      reinterpret_cast<float*>(p.out)[o] = v;
    }
  }
}


// Compute units of the current device (cached per device).
int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    cus[dev] = v;
  }
  return cus[dev];
}

// Memory-order GEMV launch: 4 waves per workgroup and a grid of one
// workgroup per CU, so that every CU streams the same number of rows (a grid
// of, say, 1.5 workgroups per CU leaves half the CUs idle for the last third
// of the kernel); R rows per wave.
constexpr int kFlatWaves = 4;

int flat_rows_per_wave(const GemmArgs& a) {
  const int64_t waves = (int64_t)device_cus() * kFlatWaves;
  const int64_t r = (a.N + waves - 1) / waves;
  return (int)(r < 1 ? 1 : r);
}

size_t flat_lds_bytes(const GemmArgs& a, int R) {
  return (size_t)a.M * a.K * 2 + (size_t)kFlatWaves * (R * a.M * 64 * 4 + 1024);
}

template <int MR>
hipError_t launch_flat_mr(const GemmArgs& a, int R, hipStream_t stream) {
  const int64_t waves = (a.N + R - 1) / R;
  const dim3 grid((unsigned)((waves + kFlatWaves - 1) / kFlatWaves));
  const size_t lds = flat_lds_bytes(a, R);
  // the weight stream is read once: non-temporal loads
  if (a.out_bf16) gemv_flat_kernel<MR, 2, true><<<grid, 64 * kFlatWaves, lds, stream>>>(a, R);
  else gemv_flat_kernel<MR, 2, false><<<grid, 64 * kFlatWaves, lds, stream>>>(a, R);
  return hipGetLastError();
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

// Dynamic LDS of the ALDS mode: every wave's f16 activation rows plus the
// 64-byte zero run (must match the layout in the kernel).
size_t alds_bytes(const GemmArgs& a, int kw) {
  const int units = a.K / 256;
  const int mrows = a.M < 16 ? a.M : 16;
  return (size_t)kw * mrows * ((units + kw - 1) / kw) * 256 * 2 + 64;
}

template <int NT, int D, bool ALDS>
hipError_t launch256(const GemmArgs& a, int kw, hipStream_t stream) {
  const dim3 grid((unsigned)((a.N + 16 * NT - 1) / (16 * NT)), (unsigned)((a.M + 15) / 16));
  const dim3 block(64 * kw);
  const size_t lds = ALDS ? alds_bytes(a, kw) : 0;
  if (a.out_bf16) {
    gemm_skinny256_kernel<NT, D, ALDS, true><<<grid, block, lds, stream>>>(a);
  } else {
    gemm_skinny256_kernel<NT, D, ALDS, false><<<grid, block, lds, stream>>>(a);
  }
  return hipGetLastError();
}

}  // namespace

// One or two rows, K a multiple of 256 from 2048 on, the f16 activation rows,
// the per-row slots and the fill within the kernel's limits.
bool gemv_flat_supported(const GemmArgs& a) {
  if (a.M < 1 || a.M > 2 || a.K < 2048 || a.K % 256 != 0) return false;
  const int R = flat_rows_per_wave(a);
  return R * a.M <= 64 && flat_lds_bytes(a, R) <= 64 * 1024 &&
         (int64_t)a.M * (a.K / 16) <= (int64_t)64 * kFlatWaves * kFlatAB;
}

hipError_t launch_gemv_flat(const GemmArgs& a, hipStream_t stream) {
  const int R = flat_rows_per_wave(a);
  return a.M == 1 ? launch_flat_mr<1>(a, R, stream) : launch_flat_mr<2>(a, R, stream);
}

// K % 256 == 0, any M (16 rows per grid.y).  Measured on MI355X (sweep over
// tiles per workgroup NT, ring depth D and waves per workgroup KW): a few
// hundred to a few thousand resident waves with 2-3 units in flight each do
// best; deeper rings or more, shorter waves only add pressure on the vector
// L1.  NT = 2 amortizes the activation operand when M > 1; KW is the smallest
// power of two that gives enough waves (>= 4096 with activations in LDS,
// which is faster for M <= 4; >= 600 otherwise) while every wave keeps >= 4
// units.
hipError_t launch_gemm_skinny256(const GemmArgs& a, hipStream_t stream) {
  const int nt = a.M > 1 ? 2 : 1;
  const int64_t wgs = ((a.N + 16 * nt - 1) / (16 * nt)) * ((a.M + 15) / 16);
  const int64_t units = a.K / 256;
  const bool small_m = a.M <= 4;
  int kw = 1;
  while (kw < kMaxWavesK && (small_m ? wgs * kw < 4096 : wgs * kw < 600) && units / (2 * kw) >= 4) kw *= 2;
  const bool alds = small_m && alds_bytes(a, kw) <= 48 * 1024;
  if (nt == 2) return alds ? launch256<2, 2, true>(a, kw, stream) : launch256<2, 2, false>(a, kw, stream);
  return alds ? launch256<1, 3, true>(a, kw, stream) : launch256<1, 3, false>(a, kw, stream);
}

// Any K (a multiple of 16), any M: 64 VB-element super-steps (VB = 2 when the
// rows are 16-byte aligned), two 16-row tiles per workgroup once there are
// 1024 tiles, KW as above for >= 1536 waves.
hipError_t launch_gemm_skinny16(const GemmArgs& a, hipStream_t stream) {
  const int64_t tiles16 = (a.N + 15) / 16, mtiles = (a.M + 15) / 16;
  const int vb = (a.K % 32 == 0) ? 2 : 1;
  const int nt = (tiles16 * mtiles >= 1024) ? 2 : 1;
  const int64_t wgs = ((tiles16 + nt - 1) / nt) * mtiles;
  const int64_t steps = (a.K + 64 * vb - 1) / (64 * vb);
  int kw = 1;
  while (kw < kMaxWavesK && wgs * kw < 1536 && steps / (2 * kw) >= 4) kw *= 2;
  if (vb == 2) return nt == 2 ? launch_cfg<2, 2, 8>(a, kw, stream) : launch_cfg<1, 2, 8>(a, kw, stream);
  return nt == 2 ? launch_cfg<2, 1, 8>(a, kw, stream) : launch_cfg<1, 1, 8>(a, kw, stream);
}

// The weight-streaming path's kernel for a product: the FP4 GEMV (one or two
// rows, K a multiple of 1024 up to 8192), the persistent M=16 stream (3..16
// rows over a tall matrix), the M-tile kernel (3..16 rows where it is faster:
// long K, or many rows), the memory-order GEMV (one or two rows, other K from
// 2048 on), else the skinny kernels.
int skinny_kernel_choice(const GemmArgs& a) {
  if (gemv_fp4_supported(a)) return kKernelGemvFp4;
  if (gemm_m16_stream_preferred(a)) return kKernelM16Stream;
  if (gemm_m16_preferred(a)) return kKernelM16;
  if (gemv_flat_supported(a)) return kKernelGemvFlat;
  return a.K % 256 == 0 ? kKernelSkinny256 : kKernelSkinny16;
}

hipError_t launch_gemm_skinny(const GemmArgs& a, hipStream_t stream) {
  switch (skinny_kernel_choice(a)) {
    case kKernelGemvFp4: return launch_gemv_fp4(a, stream);
    case kKernelM16: return launch_gemm_m16(a, stream);
    case kKernelM16Stream: return launch_gemm_m16_stream(a, stream);
    case kKernelGemvFlat: return launch_gemv_flat(a, stream);
    case kKernelSkinny256: return launch_gemm_skinny256(a, stream);
    default: return launch_gemm_skinny16(a, stream);
  }
}

}  // namespace nvfp4
