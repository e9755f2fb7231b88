// Skinny NVFP4 W4A4 GEMM for gfx950: M <= 16 activation rows against a
// streamed NVFP4 weight matrix.  This is the decode-time product of the page
// "TensorRT Edge-LLM Completes the MLPerf Edge Agentic Benchmark 6.4x Faster
// on Jetson AGX Thor": one row per generated token (section "Using NVFP4
// quantization to accelerate Qwen3.6-27B inference", where low-batch decoding
// is limited by DRAM bandwidth), or 16 rows when the 16-node candidate tree is
// verified in one pass (section "Using tree-based multi-token prediction to
// accelerate LLM inference").  The weight bytes dominate, so the kernel is
// built around streaming them from HBM once with wide coalesced loads.
//
// Work mapping.  A workgroup owns NT tiles of 16 weight rows (output columns)
// and one tile of 16 activation rows; its KW waves split K into interleaved
// "super-steps" of 64*VB elements and the partial sums are added in a fixed
// order through LDS at the end (deterministic, no atomics).  Inside a wave,
// lane l = r + 16*q streams weight row r of each tile (and activation row r):
// 16*VB contiguous K-elements (8*VB bytes of codes, VB scale bytes) at K
// offset 16*VB*q of the super-step, so the four lanes of a row read one
// contiguous 32*VB-byte run.  Each 8-element slice of a lane's run feeds one
// v_mfma_f32_16x16x32_f16 as that lane's k-group; A and B use the same slice
// for the same MFMA, so the contraction runs over a permutation of K, which
// leaves the sum unchanged.
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

template <int VB> struct Raw;
template <> struct Raw<2> { u4_t c; uint32_t s; };  // 16 bytes of codes, 2 scale bytes
template <> struct Raw<1> { u2_t c; uint32_t s; };  // 8 bytes of codes, 1 scale byte

// Loads one lane's run at element k0 of a row; `ok` false gives zero codes and
// zero scales (a row outside the matrix, or a run past K).  Weights are read
// once, so their loads carry the non-temporal hint.
template <int VB, bool NT_HINT>
__device__ __forceinline__ Raw<VB> load_run(const uint8_t* codes_row, const uint8_t* scales_row,
                                            int k0, bool ok) {
  Raw<VB> r;
  if constexpr (VB == 2) {
    r.c = u4_t{0u, 0u, 0u, 0u};
    r.s = 0u;
    if (ok) {
      const u4_t* pc = reinterpret_cast<const u4_t*>(codes_row + (k0 >> 1));
      const uint16_t* ps = reinterpret_cast<const uint16_t*>(scales_row + (k0 >> 4));
      if constexpr (NT_HINT) {
        r.c = __builtin_nontemporal_load(pc);
        r.s = __builtin_nontemporal_load(ps);
      } else {
        r.c = *pc;
        r.s = *ps;
      }
    }
  } else {
    r.c = u2_t{0u, 0u};
    r.s = 0u;
    if (ok) {
      const u2_t* pc = reinterpret_cast<const u2_t*>(codes_row + (k0 >> 1));
      const uint8_t* ps = scales_row + (k0 >> 4);
      if constexpr (NT_HINT) {
        r.c = __builtin_nontemporal_load(pc);
        r.s = __builtin_nontemporal_load(ps);
      } else {
        r.c = *pc;
        r.s = *ps;
      }
    }
  }
  return r;
}

template <int NT, int VB>
__device__ __forceinline__ void mma_run(const Raw<VB>& a, const Raw<VB> (&w)[NT], f4_t (&acc)[NT]) {
  const h2_t sa = e4m3x2_to_h2(a.s);
  h2_t sw[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) sw[t] = e4m3x2_to_h2(w[t].s);
#pragma unroll
  for (int j = 0; j < 2 * VB; ++j) {
    const h8_t af = dequant8(a.c[j], sa[j >> 1]);
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = mfma16x16x32(af, dequant8(w[t].c[j], sw[t][j >> 1]), acc[t]);
  }
}

template <int NT, int VB, bool OUT_BF16>
__global__ __launch_bounds__(64 * kMaxWavesK) void gemm_skinny_kernel(GemmArgs p) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int KW = blockDim.x >> 6;
  const int r = lane & 15, q = lane >> 4;
  const int M = p.M, K = p.K, N = p.N;
  const int n_base = blockIdx.x * (16 * NT);
  const int m_base = blockIdx.y * 16;
  const int64_t cstride = K >> 1, sstride = K >> 4;

  // Rows streamed by this lane; rows outside the matrix are clamped to a
  // valid address and read as zeros.
  const int m = m_base + r;
  const bool a_ok = m < M;
  const int64_t a_row = a_ok ? m : M - 1;
  const uint8_t* a_c = p.ac + a_row * cstride;
  const uint8_t* a_s = p.as + a_row * sstride;
  const uint8_t* w_c[NT];
  const uint8_t* w_s[NT];
  bool w_ok[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int n = n_base + 16 * t + r;
    w_ok[t] = n < N;
    const int64_t row = w_ok[t] ? n : N - 1;
    w_c[t] = p.wc + row * cstride;
    w_s[t] = p.ws + row * sstride;
  }

  constexpr int kStep = 64 * VB;  // K-elements per super-step (4 lanes x 16*VB)
  const int s_full = K / kStep;
  const int lane_k = q * 16 * VB;

  f4_t acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f4_t{0.f, 0.f, 0.f, 0.f};

  Raw<VB> a_cur, w_cur[NT];
  int ss = wave;
  if (ss < s_full) {
    const int k0 = ss * kStep + lane_k;
    a_cur = load_run<VB, false>(a_c, a_s, k0, a_ok);
#pragma unroll
    for (int t = 0; t < NT; ++t) w_cur[t] = load_run<VB, true>(w_c[t], w_s[t], k0, w_ok[t]);
  }
  while (ss < s_full) {
    const int sn = ss + KW;
    Raw<VB> a_nxt, w_nxt[NT];
    if (sn < s_full) {  // issue the next super-step's loads before using this one
      const int k0 = sn * kStep + lane_k;
      a_nxt = load_run<VB, false>(a_c, a_s, k0, a_ok);
#pragma unroll
      for (int t = 0; t < NT; ++t) w_nxt[t] = load_run<VB, true>(w_c[t], w_s[t], k0, w_ok[t]);
    }
    mma_run<NT, VB>(a_cur, w_cur, acc);
    a_cur = a_nxt;
#pragma unroll
    for (int t = 0; t < NT; ++t) w_cur[t] = w_nxt[t];
    ss = sn;
  }
  // Ragged end of K: a partial super-step, taken by the wave whose turn it is.
  if (s_full * kStep < K && wave == s_full % KW) {
    const int k0 = s_full * kStep + lane_k;
    const bool k_ok = k0 < K;  // K % (16*VB) == 0, so a lane's run is all in or all out
    a_cur = load_run<VB, false>(a_c, a_s, k0, a_ok && k_ok);
#pragma unroll
    for (int t = 0; t < NT; ++t) w_cur[t] = load_run<VB, true>(w_c[t], w_s[t], k0, w_ok[t] && k_ok);
    mma_run<NT, VB>(a_cur, w_cur, acc);
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

int env_int(const char* name, int dflt) {
  const char* s = getenv(name);
  return (s && *s) ? atoi(s) : dflt;
}

template <int NT, int VB>
hipError_t launch_nt_vb(const GemmArgs& a, int kw, hipStream_t stream) {
  const dim3 grid((unsigned)((a.N + 16 * NT - 1) / (16 * NT)), (unsigned)((a.M + 15) / 16));
  const dim3 block(64 * kw);
  if (a.out_bf16) {
    gemm_skinny_kernel<NT, VB, true><<<grid, block, 0, stream>>>(a);
  } else {
    gemm_skinny_kernel<NT, VB, false><<<grid, block, 0, stream>>>(a);
  }
  return hipGetLastError();
}

}  // namespace

// Picks the tile count per wave (NT) and the K-split (KW waves per
// workgroup) so that the grid holds a few thousand waves: enough loads in
// flight to cover HBM latency on 256 CUs, with each wave still streaming
// several super-steps.  NVFP4_SKINNY_NT / NVFP4_SKINNY_KW override the choice
// (tuning knobs; values outside {1,2} / {1,2,4,8} are ignored).
hipError_t launch_gemm_skinny(const GemmArgs& a, hipStream_t stream) {
  const int vb = (a.K % 32 == 0) ? 2 : 1;
  const int64_t tiles16 = (a.N + 15) / 16;
  const int64_t mtiles = (a.M + 15) / 16;
  int nt = (tiles16 * mtiles >= 1024) ? 2 : 1;
  const int e_nt = env_int("NVFP4_SKINNY_NT", 0);
  if (e_nt == 1 || e_nt == 2) nt = e_nt;
  const int64_t wgs = ((tiles16 + nt - 1) / nt) * mtiles;
  const int64_t steps = (a.K + 64 * vb - 1) / (64 * vb);
  int kw = 1;
  while (kw < kMaxWavesK && wgs * kw < 2048 && steps / (2 * kw) >= 2) kw *= 2;
  const int e_kw = env_int("NVFP4_SKINNY_KW", 0);
  if (e_kw == 1 || e_kw == 2 || e_kw == 4 || e_kw == 8) kw = e_kw;
  if (nt == 2) return vb == 2 ? launch_nt_vb<2, 2>(a, kw, stream) : launch_nt_vb<2, 1>(a, kw, stream);
  return vb == 2 ? launch_nt_vb<1, 2>(a, kw, stream) : launch_nt_vb<1, 1>(a, kw, stream);
}

}  // namespace nvfp4
