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


// ---------------------------------------------------------------------------
// Wave-tiled path for K % 128 == 0 (prefill shapes).  Every wave owns a
// 128 x 80 output tile (8 x 5 MFMA tiles of 16 x 16, 160 accumulators per
// lane) over a quarter of K; the four waves of a workgroup hold the same tile
// and split K, and their partial sums are added in a fixed order through LDS
// at the end.  A 128 x 80 tile makes both prefill GEMMs (512 x 25600 and
// 512 x 5120 outputs) exact multiples of 256 workgroups, one per CU per round.
//
// Operands come from global memory (mostly L2) in the MFMA lane layout: lane
// l = r + 16*q of a 16-row tile takes 16 bytes (32 codes) of row r at K
// offset 32*q of a 128-K step and the 2 scale bytes of those two blocks; each
// 8-code slice feeds one 16x16x32 f16 MFMA (the same K permutation on both
// operands, so the sum is unchanged).  Dequantization is per wave: 208 rows
// converted per K-step for 10240 outputs.
//
// Latency hiding with one wave per SIMD: the codes of the next two K-steps
// stream into a private 3-slot LDS ring through buffer->LDS loads (no
// registers held in flight); at the start of a step the wave reads its codes
// back (each lane its own 16 bytes per tile, conflict-free) and the scale
// bytes, loaded into a small register ring, are already there.  Rows past M
// or N lie past the end of their buffers and read as zeros.
//
// Workgroup order: consecutive workgroups go to different XCDs; the tile
// index is remapped so that each XCD walks a contiguous range of tiles with
// the M-tiles innermost, and the four M-tiles that share a weight tile run on
// the same XCD and meet it in that XCD's L2.
// ---------------------------------------------------------------------------
constexpr int WTM = 8, WTN = 5, WKS = 4;       // 16-row A tiles, 16-row B tiles, K split
constexpr int WT = WTM + WTN;                   // 16-row tiles per wave
constexpr int kSlots = 3;                       // LDS ring depth (K-steps)
constexpr int kSlotBytes = WT * 1024;           // codes of one K-step: 64 lanes x 16 bytes per tile
constexpr int kWaveLds = kSlots * kSlotBytes;

#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

// s_waitcnt immediate for "at most n vector-memory operations outstanding".
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

template <bool OUT_BF16>
__global__ __launch_bounds__(64 * WKS) void gemm_wave_tiled_kernel(GemmArgs p, int tiles_m, int tiles_n) {
  extern __shared__ __attribute__((aligned(16))) uint8_t wt_lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, q = lane >> 4;
  const int M = p.M, K = p.K, N = p.N;

  const int total = tiles_m * tiles_n;
  const int bid = blockIdx.x;
  const int L = (total % 8 == 0) ? (bid % 8) * (total / 8) + bid / 8 : bid;
  const int tm = L % tiles_m, tn = L / tiles_m;
  const int m0 = tm * 16 * WTM, n0 = tn * 16 * WTN;

  const uint32_t cstride = (uint32_t)K >> 1, sstride = (uint32_t)K >> 4;
  const __amdgpu_buffer_rsrc_t ac = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.ac), (short)0, (int)((uint32_t)M * cstride), 0x00020000);
  const __amdgpu_buffer_rsrc_t as = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.as), (short)0, (int)((uint32_t)M * sstride), 0x00020000);
  const __amdgpu_buffer_rsrc_t wc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.wc), (short)0, (int)((uint32_t)N * cstride), 0x00020000);
  const __amdgpu_buffer_rsrc_t ws = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.ws), (short)0, (int)((uint32_t)N * sstride), 0x00020000);

  constexpr uint32_t OOB = 0x80000000u;
  const uint32_t a_c0 = (uint32_t)(m0 + r) * cstride + 16 * q, a_s0 = (uint32_t)(m0 + r) * sstride + 2 * q;
  const uint32_t b_c0 = (uint32_t)(n0 + r) * cstride + 16 * q, b_s0 = (uint32_t)(n0 + r) * sstride + 2 * q;
  const uint32_t tc = 16 * cstride, ts = 16 * sstride;  // bytes between consecutive 16-row tiles

  const int steps = K >> 7;
  const int s_begin = (steps * wave) / WKS, s_end = (steps * (wave + 1)) / WKS;
  const int my = s_end - s_begin;

  uint8_t* ring = wt_lds + wave * kWaveLds;

  // Codes of step i -> LDS slot (i % kSlots): WT buffer->LDS loads.
  auto dma_step = [&](int i) {
    const bool ok = i < my;
    const uint32_t co = (uint32_t)(s_begin + i) * 64;
    uint8_t* slot = ring + (i % kSlots) * kSlotBytes;
#pragma unroll
    for (int t = 0; t < WTM; ++t)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ac, LDS_PTR(slot + t * 1024), 16,
                                               ok ? a_c0 + t * tc + co : OOB, 0, 0, 0);
#pragma unroll
    for (int t = 0; t < WTN; ++t)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wc, LDS_PTR(slot + (WTM + t) * 1024), 16,
                                               ok ? b_c0 + t * tc + co : OOB, 0, 0, 0);
  };
  // Scale bytes of step i: one 16-bit load per tile (2 blocks of the lane's run).
  struct Scales { uint32_t v[WT]; };
  auto load_scales = [&](int i) {
    Scales sc;
    const bool ok = i < my;
    const uint32_t so = (uint32_t)(s_begin + i) * 8;
#pragma unroll
    for (int t = 0; t < WTM; ++t)
      sc.v[t] = __builtin_amdgcn_raw_buffer_load_b16(as, ok ? a_s0 + t * ts + so : OOB, 0, 0);
#pragma unroll
    for (int t = 0; t < WTN; ++t)
      sc.v[WTM + t] = __builtin_amdgcn_raw_buffer_load_b16(ws, ok ? b_s0 + t * ts + so : OOB, 0, 0);
    return sc;
  };

  f4_t acc[WTM][WTN];
#pragma unroll
  for (int i = 0; i < WTM; ++i)
#pragma unroll
    for (int j = 0; j < WTN; ++j) acc[i][j] = f4_t{0.f, 0.f, 0.f, 0.f};

  // Prologue: steps 0 and 1 in flight.  Per step the issue order is (codes,
  // scales), 2*WT operations; at the top of step i the operations of step
  // i+1 (issued after step i's) may stay outstanding.  The loop is unrolled
  // by the ring depth so that every slot (LDS and scale registers) is named
  // statically: a scale register is never copied while its load is in flight.
  auto step = [&](int i, const Scales& sc, Scales& sc_next2, uint8_t* slot, uint8_t* slot_next2) {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * WT));
    u4_t code[WT];
#pragma unroll
    for (int t = 0; t < WT; ++t) code[t] = *reinterpret_cast<const u4_t*>(slot + t * 1024 + 16 * lane);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * WT) & ~(15 << 8));  // LDS reads of this slot done
    __builtin_amdgcn_sched_barrier(0);
    {  // step i + 2 -> the slot and scale registers that step i - 1 used
      const int i2 = i + 2;
      const bool ok = i2 < my;
      const uint32_t co = (uint32_t)(s_begin + i2) * 64, so = (uint32_t)(s_begin + i2) * 8;
#pragma unroll
      for (int t = 0; t < WTM; ++t)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ac, LDS_PTR(slot_next2 + t * 1024), 16,
                                                 ok ? a_c0 + t * tc + co : OOB, 0, 0, 0);
#pragma unroll
      for (int t = 0; t < WTN; ++t)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wc, LDS_PTR(slot_next2 + (WTM + t) * 1024), 16,
                                                 ok ? b_c0 + t * tc + co : OOB, 0, 0, 0);
#pragma unroll
      for (int t = 0; t < WTM; ++t)
        sc_next2.v[t] = __builtin_amdgcn_raw_buffer_load_b16(as, ok ? a_s0 + t * ts + so : OOB, 0, 0);
#pragma unroll
      for (int t = 0; t < WTN; ++t)
        sc_next2.v[WTM + t] = __builtin_amdgcn_raw_buffer_load_b16(ws, ok ? b_s0 + t * ts + so : OOB, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (i < my) {
      h2_t sp[WT];  // the two block scales of every tile, converted once per step
#pragma unroll
      for (int t = 0; t < WT; ++t) sp[t] = e4m3x2_to_h2(sc.v[t]);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        h8_t bf[WTN];
#pragma unroll
        for (int j = 0; j < WTN; ++j) bf[j] = dequant8(code[WTM + j][kk], sp[WTM + j][kk >> 1]);
#pragma unroll
        for (int ti = 0; ti < WTM; ++ti) {
          const h8_t af = dequant8(code[ti][kk], sp[ti][kk >> 1]);
#pragma unroll
          for (int j = 0; j < WTN; ++j) acc[ti][j] = mfma16x16x32(af, bf[j], acc[ti][j]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  uint8_t* slot0 = ring;
  uint8_t* slot1 = ring + kSlotBytes;
  uint8_t* slot2 = ring + 2 * kSlotBytes;
  Scales sc0, sc1, sc2;
  dma_step(0);
  sc0 = load_scales(0);
  dma_step(1);
  sc1 = load_scales(1);
  for (int i0 = 0; i0 < my; i0 += 3) {
    step(i0, sc0, sc2, slot0, slot2);
    step(i0 + 1, sc1, sc0, slot1, slot0);
    step(i0 + 2, sc2, sc1, slot2, slot1);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();  // every wave is done with its ring; the LDS is reused below

  // Reduction of the four K-quarters, in phases of two A tiles (32 rows):
  // every wave dumps its 2 x 5 accumulator tiles (lane-major), then wave w
  // adds tiles p = w, w+4, w+8 of the phase over waves 0..3 in order and
  // stores them.
  f4_t* red_lds = reinterpret_cast<f4_t*>(wt_lds);
  const float gg = (*p.ga) * (*p.gw);
#pragma unroll
  for (int ph = 0; ph < WTM / 2; ++ph) {
#pragma unroll
    for (int ii = 0; ii < 2; ++ii)
#pragma unroll
      for (int j = 0; j < WTN; ++j)
        red_lds[((wave * 2 + ii) * WTN + j) * 64 + lane] = acc[2 * ph + ii][j];
    __syncthreads();
    for (int pidx = wave; pidx < 2 * WTN; pidx += WKS) {
      const int ii = pidx / WTN, j = pidx % WTN;
      f4_t sum = red_lds[((0 * 2 + ii) * WTN + j) * 64 + lane];
#pragma unroll
      for (int w = 1; w < WKS; ++w) sum += red_lds[((w * 2 + ii) * WTN + j) * 64 + lane];
      const int n = n0 + 16 * j + r;
      if (n < N) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = m0 + 16 * (2 * ph + ii) + 4 * q + e;
          if (m < M) {
            const float v = sum[e] * gg;
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
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_gemm_tiled(const GemmArgs& a, hipStream_t stream) {
  if (a.K % 128 == 0 && a.K >= 128 * WKS) {
    const int tiles_m = (a.M + 16 * WTM - 1) / (16 * WTM), tiles_n = (a.N + 16 * WTN - 1) / (16 * WTN);
    const size_t lds = (size_t)WKS * kWaveLds;  // >= the reduction buffer (WKS * 2 * WTN KiB)
    const dim3 grid((unsigned)(tiles_m * tiles_n));
    // more than the default 64 KiB of dynamic LDS: raise the kernels' limit once
    static const hipError_t attr = [] {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_wave_tiled_kernel<true>),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, WKS * kWaveLds);
      if (e == hipSuccess)
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_wave_tiled_kernel<false>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, WKS * kWaveLds);
      return e;
    }();
    if (attr != hipSuccess) return attr;
    if (a.out_bf16) gemm_wave_tiled_kernel<true><<<grid, 64 * WKS, lds, stream>>>(a, tiles_m, tiles_n);
    else gemm_wave_tiled_kernel<false><<<grid, 64 * WKS, lds, stream>>>(a, tiles_m, tiles_n);
    return hipGetLastError();
  }
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
