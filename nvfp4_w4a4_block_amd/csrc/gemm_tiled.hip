// LDS-tiled NVFP4 W4A4 GEMM for gfx950 (large M).  This is the product of a
// suffix prefill, where a few hundred new tokens pass through every NVFP4
// linear layer at once (page "TensorRT Edge-LLM Completes the MLPerf Edge
// Agentic Benchmark 6.4x Faster on Jetson AGX Thor", section "Reusing KV cache
// across agent turns"), so the contraction is dense and runs on the matrix
// cores.
//
// gfx950's block-scaled FP4 MFMA takes power-of-two (E8M0) scales per 32
// elements; NVFP4 carries E4M3 scales per 16.  Instead, each 16-block is
// dequantized exactly to f16 (E2M1 value times E4M3 scale: at most 6
// significant bits, range [2^-10, 2688]) and multiplied with the f16 MFMA,
// accumulating in fp32; g_a * g_w is applied in the epilogue.
//
// Tile: 128 x 128 outputs per workgroup of 4 waves (2 x 2, 64 x 64 each, 16
// accumulator tiles of 16 x 16 per wave), K advanced 64 at a time.  Each
// thread loads 32 packed codes (16 bytes) plus 2 scale bytes of one A row and
// one B row per K-step, dequantizes them in registers and stores f16 rows to
// a double-buffered LDS tile; the next step's global loads are in flight
// while the current tile is multiplied.
#include "device_common.h"
#include "launch.h"

namespace nvfp4 {
namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDS_STRIDE = BK + 8;  // f16 per LDS row; 16 bytes of padding spread the banks
constexpr int kThreads = 256;

struct RawRun {
  u4_t c;      // 32 codes
  uint32_t s;  // 2 scale bytes (low 16 bits)
};

// One thread's run of a row at element k (k % 32 == 0): up to two 16-blocks,
// each present only if inside K and the row is inside the matrix.
template <bool K32>
__device__ __forceinline__ RawRun load_run(const uint8_t* codes_row, const uint8_t* scales_row,
                                           int k, int K, bool row_ok) {
  RawRun r;
  r.c = u4_t{0u, 0u, 0u, 0u};
  r.s = 0u;
  if (!row_ok || k >= K) return r;
  if constexpr (K32) {  // rows are 16-byte aligned and both blocks are inside K
    r.c = *reinterpret_cast<const u4_t*>(codes_row + (k >> 1));
    r.s = *reinterpret_cast<const uint16_t*>(scales_row + (k >> 4));
  } else {              // rows are 8-byte aligned; the second block may be past K
    const u2_t lo = *reinterpret_cast<const u2_t*>(codes_row + (k >> 1));
    r.c.x = lo.x;
    r.c.y = lo.y;
    r.s = scales_row[k >> 4];
    if (k + 16 < K) {
      const u2_t hi = *reinterpret_cast<const u2_t*>(codes_row + (k >> 1) + 8);
      r.c.z = hi.x;
      r.c.w = hi.y;
      r.s |= (uint32_t)scales_row[(k >> 4) + 1] << 8;
    }
  }
  return r;
}

__device__ __forceinline__ void store_run(_Float16* dst, const RawRun& r) {
  const h2_t s = e4m3x2_to_h2(r.s);
  h8_t* d = reinterpret_cast<h8_t*>(dst);
  d[0] = dequant8(r.c.x, s.x);
  d[1] = dequant8(r.c.y, s.x);
  d[2] = dequant8(r.c.z, s.y);
  d[3] = dequant8(r.c.w, s.y);
}

template <bool K32, bool OUT_BF16>
__global__ __launch_bounds__(kThreads) void gemm_tiled_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) _Float16 lds[2][2][BM][LDS_STRIDE];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int M = p.M, K = p.K, N = p.N;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int64_t cstride = K >> 1, sstride = K >> 4;

  // Loader role: row lr of the A and B tiles, K sub-range [32*h, 32*h + 32).
  const int lr = tid >> 1, h = tid & 1;
  const bool a_ok = m0 + lr < M, b_ok = n0 + lr < N;
  const int64_t a_row = a_ok ? m0 + lr : M - 1, b_row = b_ok ? n0 + lr : N - 1;
  const uint8_t* a_c = p.ac + a_row * cstride;
  const uint8_t* a_s = p.as + a_row * sstride;
  const uint8_t* b_c = p.wc + b_row * cstride;
  const uint8_t* b_s = p.ws + b_row * sstride;

  f4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f4_t{0.f, 0.f, 0.f, 0.f};

  const int KT = (K + BK - 1) / BK;
  RawRun ra = load_run<K32>(a_c, a_s, 32 * h, K, a_ok);
  RawRun rb = load_run<K32>(b_c, b_s, 32 * h, K, b_ok);
  store_run(&lds[0][0][lr][32 * h], ra);
  store_run(&lds[0][1][lr][32 * h], rb);

  const int fr = lane & 15, fk = 8 * (lane >> 4);
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    const bool more = kt + 1 < KT;
    if (more) {
      const int k = (kt + 1) * BK + 32 * h;
      ra = load_run<K32>(a_c, a_s, k, K, a_ok);
      rb = load_run<K32>(b_c, b_s, k, K, b_ok);
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      h8_t af[4], bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const h8_t*>(&lds[buf][0][wm * 64 + 16 * i + fr][kk + fk]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bf[j] = *reinterpret_cast<const h8_t*>(&lds[buf][1][wn * 64 + 16 * j + fr][kk + fk]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(af[i], bf[j], acc[i][j]);
    }
    if (more) {
      store_run(&lds[buf ^ 1][0][lr][32 * h], ra);
      store_run(&lds[buf ^ 1][1][lr][32 * h], rb);
    }
  }

  const float gg = (*p.ga) * (*p.gw);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + wn * 64 + 16 * j + fr;
      if (n >= N) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = m0 + wm * 64 + 16 * i + 4 * (lane >> 4) + e;
        if (m >= M) continue;
        const float v = acc[i][j][e] * gg;
        const int64_t o = (int64_t)m * N + n;
        if constexpr (OUT_BF16) {
          reinterpret_cast<uint16_t*>(p.out)[o] = f32_to_bf16_rne(v);
        } else {
          reinterpret_cast<float*>(p.out)[o] = v;
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_tiled(const GemmArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)((a.N + BN - 1) / BN), (unsigned)((a.M + BM - 1) / BM));
  const bool k32 = a.K % 32 == 0;
  if (k32) {
    if (a.out_bf16) gemm_tiled_kernel<true, true><<<grid, kThreads, 0, stream>>>(a);
    else gemm_tiled_kernel<true, false><<<grid, kThreads, 0, stream>>>(a);
  } else {
    if (a.out_bf16) gemm_tiled_kernel<false, true><<<grid, kThreads, 0, stream>>>(a);
    else gemm_tiled_kernel<false, false><<<grid, kThreads, 0, stream>>>(a);
  }
  return hipGetLastError();
}

}  // namespace nvfp4
