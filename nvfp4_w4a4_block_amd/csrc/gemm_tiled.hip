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
// Persistent workgroup-tiled path for K % 1024 == 0 (prefill shapes).
//
// Output tile 64 x 160 per workgroup (2 x 5 MFMA tiles of 32 x 32, f16
// 32x32x16 matrix instructions).  Both prefill GEMMs (512 x 25600 and
// 512 x 5120 outputs) are exact multiples of 256 such tiles.  One workgroup per
// CU walks its tiles in turn, and the load pipeline runs on across tile
// boundaries.  Eight waves (two per SIMD: while one waits on its matrix
// instruction the other issues its dequantization) each hold the whole tile
// (160 accumulators per lane) over an eighth of every 256-K step and add their
// partial sums in a fixed order through LDS when the tile is done.  A wave
// dequantizes only its own eighth, so every operand element is converted to
// f16 exactly once per workgroup.
//
// Loads: the workgroup stages each 256-K step (14 tiles of 16 rows x 128 code
// bytes: 4 of A, 10 of B) in a 3-slot LDS ring with buffer->LDS loads, each
// instruction 8 rows x 128 bytes, so that every four consecutive lanes read 64
// contiguous bytes: the L1 cache then takes 16 accesses per instruction, not
// one per lane.  Scale bytes (16 per row and step) come 4 steps at a time into
// a 2-slot LDS buffer, 16 rows x 64 bytes per instruction.  The 16-byte chunks
// of a row are XOR-swizzled by the row index inside LDS, so the MFMA-layout
// reads spread over the banks.  Rows past M or N lie past the end of their
// buffers and read as zeros.
//
// Schedule of step g: wait for this wave's loads of step g + 1, barrier (no
// memory fence), issue the loads of step g + 3 into the slot step g used
// (every wave is past its reads) and, at a group start, the next scale group;
// then multiply step g with the LDS reads of step g + 1's codes and scale
// bytes (into the other register set) spread among its matrix instructions.
// Reading them all right after the barrier stalled every wave at once on LDS
// issue (the eight waves' reads arrive together); spread out they wait about a
// third as long.  The step loop is unrolled by a scale group (4 steps), so each
// step's expected wait count is a constant; anything else (a tile or stream
// boundary) waits for all loads.
// ---------------------------------------------------------------------------
typedef float f32x16_t __attribute__((ext_vector_type(16)));
template <int P> struct StepPos { static constexpr int value = P; };  // step index & 3

constexpr int MT = 2, NT = 5;                // 32 x 32 MFMA tiles per workgroup tile
constexpr int FT = MT + NT;                  // MFMA operand tiles
constexpr int BMW = 32 * MT, BNW = 32 * NT;  // 64 x 160 outputs
constexpr int TA = BMW / 16, TT = TA + BNW / 16;  // 16-row load tiles: 4 of A, 14 in all
constexpr int kWaves = 8;
constexpr int kStepK = 256;                  // 128 code bytes per row per step
constexpr int kTileStep = 16 * 128;          // one 16-row tile of one step
constexpr int kSlotBytes = TT * kTileStep;   // 28 KiB
constexpr int kSlots = 3;
constexpr int kGroup = 4;                    // steps per scale group
constexpr int kScaleTile = 16 * 64;          // 16 rows x 64 scale bytes
constexpr int kScaleBuf = TT * kScaleTile;   // 14 KiB
constexpr int kRedBytes = kWaves * 64 * 64;  // one accumulator tile of every wave
constexpr int kScaleOff = kSlots * kSlotBytes;
constexpr int kRedOff = kScaleOff + 2 * kScaleBuf;
constexpr int kLdsBytes = kRedOff + kRedBytes;  // 144 KiB
constexpr int kCodeLoadsMax = 4;             // per wave and step: 4 (waves 0-3) or 3 (waves 4-7)
constexpr int kScaleLoads = 2;               // per wave and group
static_assert(kWaves * 3 + 4 == 2 * TT, "every half of every load tile is issued once per step");

#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

// s_waitcnt immediates: "at most n vector-memory operations outstanding", and
// "all LDS operations done".
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int kLgkm0 = 15 | (3 << 14) | (7 << 4);

__device__ __forceinline__ void wait_vm(int n) {
  switch (n) {
#define W_(k) case k: __builtin_amdgcn_s_waitcnt(vmcnt_imm(k)); break;
    W_(1) W_(2) W_(3) W_(4) W_(5) W_(6) W_(7) W_(8) W_(9) W_(10) W_(11) W_(12)
#undef W_
    default: __builtin_amdgcn_s_waitcnt(vmcnt_imm(0)); break;  // also safe for any other count
  }
}

// Workgroup barrier for LDS traffic only: this wave's LDS operations are done,
// no wait on vector memory (loads of later steps stay in flight), and the
// compiler moves no memory access across it.
__device__ __forceinline__ void barrier_lds() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(kLgkm0);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// E4M3FN byte (finite) -> f16, exact, one instruction (every finite E4M3
// value, subnormals included, is an f16 value; unit scale).
__device__ __forceinline__ _Float16 e4m3_to_f16(uint32_t byte) {
  return (_Float16)__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(byte, 1.0f, false)[0];
}

__device__ __forceinline__ f32x16_t mfma32x32x16(h8_t a, h8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

template <bool OUT_BF16, bool QOUT>
__global__ __launch_bounds__(64 * kWaves) void gemm_wg_tiled_kernel(GemmArgs p, int tiles_m, int tiles_n) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r32 = lane & 31, kq = lane >> 5;
  const int M = p.M, K = p.K, N = p.N;
  const int total = tiles_m * tiles_n;
  const int grid = gridDim.x, b = blockIdx.x;
  const int my_tiles = (total - b + grid - 1) / grid;
  const int steps = K / kStepK;  // a multiple of kGroup
  const int groups = steps / kGroup;
  const int total_steps = my_tiles * steps;

  const uint32_t cstride = (uint32_t)K >> 1, sstride = (uint32_t)K >> 4;
  const __amdgpu_buffer_rsrc_t rac = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.ac), (short)0, (int)((uint32_t)M * cstride), 0x00020000);
  const __amdgpu_buffer_rsrc_t ras = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.as), (short)0, (int)((uint32_t)M * sstride), 0x00020000);
  const __amdgpu_buffer_rsrc_t rwc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.wc), (short)0, (int)((uint32_t)N * cstride), 0x00020000);
  const __amdgpu_buffer_rsrc_t rws = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.ws), (short)0, (int)((uint32_t)N * sstride), 0x00020000);

  // Tile it of this workgroup -> first output row and column.  Consecutive
  // workgroups run on different XCDs; with total % 8 == 0 each XCD walks a
  // contiguous range of tiles, M-tiles innermost, so the M-tiles that share a
  // weight tile meet it in one L2.
  auto coords = [&](int it, int& mb, int& nb) {
    const int idx = it * grid + b;
    const int L = (total % 8 == 0) ? (idx % 8) * (total / 8) + idx / 8 : idx;
    mb = (L % tiles_m) * BMW;
    nb = (L / tiles_m) * BNW;
  };

  // This wave's loads.  Codes: load k (k < 4 for waves 0-3, k < 3 for waves
  // 4-7) takes rows 8h..8h+7 (h = w & 1) of load tile (w >> 1) + 4k (tiles 0-3
  // are A rows, 4-13 B rows).  Lane l reads row 8h + l/8, 16-byte chunk
  // (l % 8) ^ (l / 8) of the step and lands at LDS byte 16 l of the
  // instruction: chunk c of row j sits at 16 * (8 j + (c ^ (j & 7))) inside its
  // tile.  Scales: load k = 0, 1 takes load tile min(w + 8k, 13) (waves 6-7
  // repeat wave 5's second load: the same bytes to the same place); lane l
  // reads row l/4, chunk (l % 4) ^ ((l / 8) & 3) of the group's 64 bytes, so
  // chunk c (step c of the group) of row j sits at 16 * (4 j + (c ^ ((j >> 1) & 3))).
  const int h = w & 1, wp = w >> 1;
  const int n_code = w < 4 ? 4 : 3;
  const uint32_t lane_c = (uint32_t)(8 * h + (lane >> 3)) * cstride + 16u * (uint32_t)((lane & 7) ^ (lane >> 3));
  const uint32_t lane_s = (uint32_t)(lane >> 2) * sstride + 16u * (uint32_t)((lane & 3) ^ ((lane >> 3) & 3));
  uint32_t coff[kCodeLoadsMax], soff[kScaleLoads];
  auto set_code_tile = [&](int mb, int nb) {
#pragma unroll
    for (int k = 0; k < kCodeLoadsMax; ++k) {
      const int t = wp + 4 * k;
      const int row = t < TA ? mb + 16 * t : nb + 16 * (t - TA);
      coff[k] = (uint32_t)row * cstride + lane_c;
    }
  };
  auto set_scale_tile = [&](int mb, int nb) {
#pragma unroll
    for (int k = 0; k < kScaleLoads; ++k) {
      const int t = min(w + 8 * k, TT - 1);
      const int row = t < TA ? mb + 16 * t : nb + 16 * (t - TA);
      soff[k] = (uint32_t)row * sstride + lane_s;
    }
  };
  auto issue_codes = [&](int i, int slot) {
    uint8_t* base = lds + slot * kSlotBytes + h * 1024;
    const uint32_t so = (uint32_t)i * 128u;
#pragma unroll
    for (int k = 0; k < kCodeLoadsMax; ++k)
      if (k < 3 || w < 4)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(k == 0 ? rac : rwc, LDS_PTR(base + (wp + 4 * k) * kTileStep), 16,
                                                 coff[k] + so, 0, 0, 0);
  };
  auto issue_scales = [&](int gi, int buf) {
    uint8_t* base = lds + kScaleOff + buf * kScaleBuf;
    const uint32_t so = (uint32_t)gi * 64u;
#pragma unroll
    for (int k = 0; k < kScaleLoads; ++k) {
      const int t = min(w + 8 * k, TT - 1);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(t < TA ? ras : rws, LDS_PTR(base + t * kScaleTile), 16,
                                               soff[k] + so, 0, 0, 0);
    }
  };

  // Consumer side: lane (r32, kq) of wave w takes the 8 code bytes
  // [16w + 8kq, 16w + 8kq + 8) of row r32 of every 32-row MFMA tile, i.e.
  // K = 32w + 16kq + 0..15 of the step: one 16-block, whose scale is byte
  // 2w + kq of the step's 16.  Its first dword feeds slice 0 (one MFMA), the
  // second slice 1 (the same permutation of K on both operands, so the sum is
  // unchanged).  MFMA tile t of the workgroup (0-1 A, 2-6 B) is load tiles 2t
  // and 2t + 1.
  const int jr = r32 & 15;
  const int rd_code = kTileStep * (r32 >> 4) + 128 * jr + 16 * (w ^ (jr & 7)) + 8 * kq;
  const int rd_scale = kScaleTile * (r32 >> 4) + 64 * jr + 2 * w + kq;
  const int sw_r = (jr >> 1) & 3;
  struct Ops {
    u2_t c[FT];
    uint32_t s[FT];
  };
  auto read_ops = [&](int slot, int buf, int i, Ops& o) {
    const uint8_t* cs = lds + slot * kSlotBytes + rd_code;
    const uint8_t* ss = lds + kScaleOff + buf * kScaleBuf + rd_scale + 16 * ((i & 3) ^ sw_r);
#pragma unroll
    for (int t = 0; t < FT; ++t) o.c[t] = *reinterpret_cast<const u2_t*>(cs + t * 2 * kTileStep);
#pragma unroll
    for (int t = 0; t < FT; ++t) o.s[t] = ss[t * 2 * kScaleTile];
  };
  auto multiply = [&](const Ops& o, f32x16_t (&acc)[MT][NT]) {
    // one conversion per scale byte; the packed multiplies broadcast its low half
    _Float16 sv[FT];
#pragma unroll
    for (int t = 0; t < FT; ++t) sv[t] = e4m3_to_f16(o.s[t]);
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
      h8_t af[MT];
#pragma unroll
      for (int ti = 0; ti < MT; ++ti) af[ti] = dequant8(o.c[ti][sl], sv[ti]);
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const h8_t bf = dequant8(o.c[MT + j][sl], sv[MT + j]);
#pragma unroll
        for (int ti = 0; ti < MT; ++ti) acc[ti][j] = mfma32x32x16(af[ti], bf, acc[ti][j]);
      }
    }
    // Interleave: each matrix instruction followed by (at first) one LDS read
    // of the next step and a run of dequantization.
#pragma unroll
    for (int q = 0; q < 2 * MT * NT; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);           // MFMA
      if (q < 12) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);           // VALU
    }
  };

  const float gg = (*p.ga) * (*p.gw);
  [[maybe_unused]] const float gy = QOUT ? *p.y_global : 0.0f;

  // Load pointers: codes run three steps ahead of the multiplies, scales one
  // group ahead; both continue into the next tile.
  int c_it = 0, c_i = 0, s_it = 0, s_gi = 0;
  bool s_valid = true;
  auto advance_codes = [&]() {
    if (++c_i == steps) {
      c_i = 0;
      if (++c_it < my_tiles) {
        int mb, nb;
        coords(c_it, mb, nb);
        set_code_tile(mb, nb);
      }
    }
  };
  auto advance_scales = [&]() {
    if (++s_gi == groups) {
      s_gi = 0;
      if (++s_it < my_tiles) {
        int mb, nb;
        coords(s_it, mb, nb);
        set_scale_tile(mb, nb);
      } else {
        s_valid = false;
      }
    }
  };

  // Loads issued (by this wave) after the codes of the step the next wait is
  // for: the scale group issued with them, and the codes and scales of the
  // step after.  With every group 4 steps long, a step's scale group was
  // issued before its codes.
  int c_prev1 = 0, s_prev1 = 0, s_prev2 = 0;
  Ops opa, opb;
  {
    int mb, nb;
    coords(0, mb, nb);
    set_code_tile(mb, nb);
    set_scale_tile(mb, nb);
    issue_scales(0, 0);
    advance_scales();
    const int n_pro = total_steps < 3 ? total_steps : 3;
    for (int j = 0; j < n_pro; ++j) {
      issue_codes(c_i, j);
      advance_codes();
    }
    wait_vm(n_code * (n_pro - 1));
    barrier_lds();
    read_ops(0, 0, 0, opa);
    c_prev1 = n_pro == 3 ? n_code : 0;
  }

  // Top of step g: make step g + 1's operands ready in `nxt` and keep the
  // loads three steps ahead.  i is g's index inside its tile, it its tile.
  int slot = 0, sb = 0, g = 0;
  auto advance = [&](auto pos, int i, int it, Ops& nxt) {
    constexpr int P = decltype(pos)::value;  // == i & 3
    const int ni = (i + 1 == steps) ? 0 : i + 1;
    const int nslot = slot == 2 ? 0 : slot + 1;
    const int nsb = (ni & 3) == 0 ? sb ^ 1 : sb;
    if (g + 1 < total_steps) {
      // Loads issued after step g + 1's codes: the scale group of the step
      // before last (P == 2), the last step's codes, the last step's scale
      // group (P == 1).  After a tile's epilogue its output stores are
      // outstanding too, and near the end of the stream fewer loads were
      // issued: there (any other count) wait for all.
      const int nw = i == 0 && it > 0 ? 0 : s_prev2 + c_prev1 + s_prev1;
      constexpr int off = (P == 1 || P == 2) ? kScaleLoads : 0;
      if (nw == 4 + off) __builtin_amdgcn_s_waitcnt(vmcnt_imm(4 + off));
      else if (nw == 3 + off) __builtin_amdgcn_s_waitcnt(vmcnt_imm(3 + off));
      else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      barrier_lds();
      int c_cur = 0, s_cur = 0;
      if (g + 3 < total_steps) {
        issue_codes(c_i, slot);
        advance_codes();
        c_cur = n_code;
      }
      if (P == 0 && s_valid) {
        issue_scales(s_gi, sb ^ 1);
        advance_scales();
        s_cur = kScaleLoads;
      }
      s_prev2 = s_prev1;
      s_prev1 = s_cur;
      c_prev1 = c_cur;
    }
    // Step g + 1's operands (none are used after the last step: there the
    // read is of a slot no load writes any more).  The slots loaded above are
    // not the ones read here.
    read_ops(nslot, nsb, ni, nxt);
    slot = nslot;
    sb = nsb;
    ++g;
  };

  for (int it = 0; it < my_tiles; ++it) {
    int m0, n0;
    coords(it, m0, n0);
    f32x16_t acc[MT][NT];
#pragma unroll
    for (int ti = 0; ti < MT; ++ti)
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[ti][j][e] = 0.0f;

    // steps is a multiple of 4: every tile starts with its operands in opa
    for (int i = 0; i < steps; i += 4) {
      advance(StepPos<0>{}, i, it, opb);
      multiply(opa, acc);
      __builtin_amdgcn_sched_barrier(0);
      advance(StepPos<1>{}, i + 1, it, opa);
      multiply(opb, acc);
      __builtin_amdgcn_sched_barrier(0);
      advance(StepPos<2>{}, i + 2, it, opb);
      multiply(opa, acc);
      __builtin_amdgcn_sched_barrier(0);
      advance(StepPos<3>{}, i + 3, it, opa);
      multiply(opb, acc);
      __builtin_amdgcn_sched_barrier(0);
    }

    // Tile done: reduce the eight K-eighths one accumulator tile at a time.
    // Every wave dumps its tile (element pair e2 of lane l at
    // (w * 8 + e2) * 64 + l), then wave w adds pair e2 = w over waves 0..7 in
    // order and stores it: elements 2w, 2w + 1 of lane l are rows
    // 8(w / 2) + 4(l / 32) + 2(w % 2) + 0..1, column l % 32 of the tile.
    f2_t* red = reinterpret_cast<f2_t*>(lds + kRedOff);
    [[maybe_unused]] uint32_t qv[MT * NT];  // bf16 output quantization: this lane's two stored values per tile
#pragma unroll
    for (int tix = 0; tix < MT * NT; ++tix) {
      const f32x16_t a = acc[tix / NT][tix % NT];
#pragma unroll
      for (int e2 = 0; e2 < 8; ++e2) red[(w * 8 + e2) * 64 + lane] = f2_t{a[2 * e2], a[2 * e2 + 1]};
      barrier_lds();
      f2_t sum = red[(0 * 8 + w) * 64 + lane];
#pragma unroll
      for (int v = 1; v < kWaves; ++v) sum += red[(v * 8 + w) * 64 + lane];
      const int n = n0 + 32 * (tix % NT) + r32;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int m = m0 + 32 * (tix / NT) + 8 * (w >> 1) + 4 * kq + 2 * (w & 1) + e;
        const bool ok = n < N && m < M;
        const float v = sum[e] * gg;
        if constexpr (OUT_BF16) {
          const uint16_t bits = f32_to_bf16_rne(v);
          // with output quantization the tile is stored from the LDS staging
          // below, eight values (16 bytes) per store
          if (!QOUT && ok) reinterpret_cast<uint16_t*>(p.out)[(int64_t)m * N + n] = bits;
          if constexpr (QOUT) {  // quantized after the tile, from LDS (below)
            if (e == 0) qv[tix] = bits;
            else qv[tix] |= (uint32_t)bits << 16;
          }
        } else {
          if (ok) reinterpret_cast<float*>(p.out)[(int64_t)m * N + n] = v;
        }
        if constexpr (QOUT && !OUT_BF16) {
          const float x = v;  // the value as stored
          // The 16 lanes 16c .. 16c+15 of a half-wave hold one 16-column
          // block of row m (N % 16 == 0: a block is wholly inside or wholly
          // outside the matrix).  The same fp32 steps as every quantizer here:
          // amax, s = (amax / 6) / g, scale byte, d = sv * g, inv = 1 / d,
          // codes of x * inv; element 2j in the low nibble of byte j.
          float amax = __builtin_fabsf(x);
#pragma unroll
          for (int sh = 1; sh < 16; sh <<= 1) amax = __builtin_fmaxf(amax, __shfl_xor(amax, sh));
          const float s = (gy == 0.0f) ? 0.0f : (amax / 6.0f) / gy;
          const uint32_t sbyte = e4m3_from_nonneg(s);
          const float d = e4m3_to_f32(sbyte) * gy;
          const float inv = (d == 0.0f) ? 0.0f : 1.0f / d;
          uint32_t word = e2m1_from_f32(x * inv) << (4 * (r32 & 7));
#pragma unroll
          for (int sh = 1; sh < 8; sh <<= 1) word |= __shfl_xor(word, sh);
          if (ok) {
            const int64_t blk = (int64_t)m * (N >> 4) + (n >> 4);
            if ((r32 & 7) == 0) reinterpret_cast<uint32_t*>(p.y_codes)[2 * blk + ((r32 >> 3) & 1)] = word;
            if ((r32 & 15) == 0) p.y_scales[blk] = (uint8_t)sbyte;
          }
        }
      }
      barrier_lds();
    }
    if constexpr (QOUT && OUT_BF16) {
      // The tile's bf16 values, [64 rows][160 columns], staged in the
      // reduction area, then stored and quantized as quant_blocks_kernel
      // quantizes them: two adjacent threads per 16-column block, eight values
      // each (one 16-byte store of the output; measured 1.3% faster at the
      // up-projection than two-byte stores from the reduction), the same fp32
      // steps (amax, s = (amax / 6) / g, scale byte, d = sv * g, inv = 1 / d,
      // codes of x * inv), element 2j in the low nibble of byte j.
      uint16_t* stage = reinterpret_cast<uint16_t*>(lds + kRedOff);
#pragma unroll
      for (int tix = 0; tix < MT * NT; ++tix) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int row = 32 * (tix / NT) + 8 * (w >> 1) + 4 * kq + 2 * (w & 1) + e;
          stage[row * BNW + 32 * (tix % NT) + r32] = (uint16_t)(qv[tix] >> (16 * e));
        }
      }
      barrier_lds();
      constexpr int kHalves = BMW * (BNW / 8);  // 1280 runs of 8 values
#pragma unroll
      for (int i = 0; i < (kHalves + 64 * kWaves - 1) / (64 * kWaves); ++i) {
        const int hb = (int)threadIdx.x + 64 * kWaves * i;
        const bool valid = hb < kHalves;
        const int row = hb / (BNW / 8), rem = hb - row * (BNW / 8), blk = rem >> 1, half = rem & 1;
        u4_t raw = u4_t{0u, 0u, 0u, 0u};
        if (valid) raw = *reinterpret_cast<const u4_t*>(stage + row * BNW + 16 * blk + 8 * half);
        float x[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          x[2 * k] = __uint_as_float(raw[k] << 16);
          x[2 * k + 1] = __uint_as_float(raw[k] & 0xFFFF0000u);
        }
        float amax = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) amax = __builtin_fmaxf(amax, __builtin_fabsf(x[k]));
        amax = __builtin_fmaxf(amax, __shfl_xor(amax, 1));  // the block's other half: thread ^ 1
        const float s = (gy == 0.0f) ? 0.0f : (amax / 6.0f) / gy;
        const uint32_t sbyte = e4m3_from_nonneg(s);
        const float d = e4m3_to_f32(sbyte) * gy;
        const float inv = (d == 0.0f) ? 0.0f : 1.0f / d;
#pragma unroll
        for (int k = 0; k < 8; ++k) x[k] *= inv;
        const uint32_t word = e2m1x8_from_f32(x);
        const int m = m0 + row, n = n0 + 16 * blk;
        if (valid && m < M && n < N) {  // N % 16 == 0: the whole block is inside
          *reinterpret_cast<u4_t*>(reinterpret_cast<uint16_t*>(p.out) + (int64_t)m * N + n + 8 * half) = raw;
          const int64_t b16 = (int64_t)m * (N >> 4) + (n >> 4);
          reinterpret_cast<uint32_t*>(p.y_codes)[2 * b16 + half] = word;
          if (half == 0) p.y_scales[b16] = (uint8_t)sbyte;
        }
      }
      barrier_lds();  // the staging is read before the next tile reduces through the same LDS
    }
  }
}

}  // namespace

static int tiled_cus() {
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

namespace {

bool persistent_ok(const GemmArgs& a) {
  // buffer offsets are 32-bit: rows up to one tile past the end must stay below 2^31 bytes
  const int64_t rows = (int64_t)(a.M > a.N ? a.M : a.N) + BNW;
  return a.K % (kStepK * kGroup) == 0 && a.K > 0 && rows * (a.K / 2) < ((int64_t)1 << 31);
}

template <bool OUT_BF16, bool QOUT>
hipError_t launch_persistent(const GemmArgs& a, hipStream_t stream) {
  const int tiles_m = (a.M + BMW - 1) / BMW, tiles_n = (a.N + BNW - 1) / BNW;
  const int total = tiles_m * tiles_n;
  const int cus = tiled_cus();
  const dim3 grid((unsigned)(total < cus ? total : cus));
  // more than the default 64 KiB of dynamic LDS: raise this kernel's limit once
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&gemm_wg_tiled_kernel<OUT_BF16, QOUT>),
      hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
  if (attr != hipSuccess) return attr;
  gemm_wg_tiled_kernel<OUT_BF16, QOUT><<<grid, 64 * kWaves, kLdsBytes, stream>>>(a, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace

bool gemm_tiled_persistent_supported(const GemmArgs& a) { return persistent_ok(a); }

bool gemm_tiled_quant_out_supported(const GemmArgs& a) { return persistent_ok(a) && a.N % 16 == 0; }

hipError_t launch_gemm_tiled_persistent(const GemmArgs& a, hipStream_t stream) {
  const bool q = a.y_codes != nullptr && a.N % 16 == 0;
  if (a.out_bf16) return q ? launch_persistent<true, true>(a, stream) : launch_persistent<true, false>(a, stream);
  return q ? launch_persistent<false, true>(a, stream) : launch_persistent<false, false>(a, stream);
}

hipError_t launch_gemm_tiled_simple(const GemmArgs& a, hipStream_t stream) {
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

hipError_t launch_gemm_tiled(const GemmArgs& a, hipStream_t stream) {
  return persistent_ok(a) ? launch_gemm_tiled_persistent(a, stream) : launch_gemm_tiled_simple(a, stream);
}

}  // namespace nvfp4
