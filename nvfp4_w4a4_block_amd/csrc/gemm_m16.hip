// Weight-streaming GEMM for up to 16 activation rows: the verification pass
// of a 16-node candidate tree, and the language-model head over it (page
// "TensorRT Edge-LLM Completes the MLPerf Edge Agentic Benchmark 6.4x Faster
// on Jetson AGX Thor", sections "Using tree-based multi-token prediction to
// accelerate LLM inference" and "Using NVFP4 quantization to accelerate
// Qwen3.6-27B inference").  At these sizes the product reads every weight
// once and little else, so the kernel is a weight stream feeding f16 matrix
// cores:
//
//   - a line is 128 K-elements: 64 code bytes and 8 scale bytes of a row;
//   - one 16-byte load per lane covers a line of 16 weight rows: lane
//     j + 16q holds bytes 16q .. 16q+15 of row j's line (elements 32q ..
//     32q+31, blocks 2q and 2q+1), a 64-byte run per row;
//   - the codes are dequantized exactly to f16 with their E4M3 scale (E2M1 x
//     E4M3 has at most 6 significant bits and lies in [2^-10, 2688]) and are
//     the B operand of v_mfma_f32_16x16x32_f16, column j = weight row j.  For
//     piece p (elements 32q + 8p .. +7 of every lane) the MFMA's k = 8q + e
//     is element 32q + 8p + e, so four MFMAs cover the line and every column
//     of every MFMA is used;
//   - the A operand is the 16 activation rows (rows past M read zeros), laid
//     out the same way (lane i + 16q: row i, elements 32q .. 32q+31), staged
//     once per workgroup in LDS as codes and scales for the workgroup's K
//     range and dequantized per line, once for the G row groups of a wave.
//     Every product is exact; the fp32 accumulation is the only rounding.
//
// Work split: a workgroup has RB x KS waves; each wave owns G groups of 16
// rows and one of KS slices of the workgroup's lines, with D lines of weight
// loads in flight.  The KS partial sums are added through LDS in a fixed
// order.  When K is long and N small (tree verification of a down-
// projection: N = 5120 rows, K = 25600) the lines are also split over KZ
// workgroups (grid.y): each writes its fp32 partial tile to a caller-owned
// workspace, and the last of the KZ workgroups of a row block to arrive (a
// counter per row block) adds the KZ partials in the order kz = 0, 1, ... and
// writes the result, then resets the counter to zero.  The sum does not
// depend on which workgroup arrives last, so results are bit-identical from
// run to run.
#include "device_common.h"
#include "launch.h"

namespace nvfp4 {
namespace {

constexpr uint32_t kOOB = 0x80000000u;  // buffer offset past any array: loads read zeros
constexpr int kLine = 128;              // K-elements per line
constexpr int kMaxLdsM16 = 64 * 1024;   // LDS budget of one workgroup
constexpr int kFillBatch = 8;           // staged pieces loaded per thread before they are stored

// Two consecutive lines (a 128-byte run of each row), loaded back to back so
// that both halves of a row's 128-byte segment are requested together.
template <int G>
struct Pair {
  u4_t w[2][G];  // weight codes of each half and row group
};

// Weight scales are fetched a block of 8 lines (4 pairs) at a time: lane
// j + 16c loads 16 bytes of row j (lines 2c and 2c + 1 of the block), so one
// load covers 16 rows x 64 contiguous bytes, and the block is parked in a
// per-wave LDS slot of 16 rows x 64 bytes whose dwords are XOR-swizzled by
// row (dword d of row j at 4 (d ^ j)), so the 2-byte reads of a quarter-wave
// (16 rows, one offset) hit distinct banks.  Per-lane 2-byte scale loads from
// memory touch 16 cache lines for 128 bytes and cost as much time as the
// codes (measured: the code stream alone runs at 5.5 TB/s, with such scale
// loads at 3.6 TB/s).
constexpr uint32_t kScaleSlot = 16u * 64u;  // LDS bytes per wave and row group

// LDS layout of the staged activations for LS lines: 16 rows of codes
// (stride 64 LS + 16 bytes: 16-byte units per row step = 4 LS + 1, odd, so the
// 16 rows read by a quarter-wave fall in distinct banks), then 16 rows of
// scales (stride 8 LS + 4 bytes: an odd number of words).
__host__ __device__ constexpr uint32_t cstride(int LS) { return 64u * (uint32_t)LS + 16u; }
__host__ __device__ constexpr uint32_t sstride(int LS) { return 8u * (uint32_t)LS + 4u; }
__host__ __device__ constexpr uint32_t alds_bytes(int LS) { return 16u * (cstride(LS) + sstride(LS)); }
// Shared activation window (AW mode): the workgroup dequantizes 4 lines of the
// 16 activation rows at a time into f16 in LDS, double-buffered (row stride
// 1040 bytes = 65 16-byte units, odd, so a quarter-wave's 16 rows hit
// distinct banks), and every wave reads its A operand from there instead of
// dequantizing it itself.
constexpr int kWin = 4;                                  // lines per window
constexpr uint32_t kWinRow = kWin * kLine * 2 + 16;      // bytes per row of a window
constexpr uint32_t kWinSlot = 16u * kWinRow;             // one window
constexpr int kAwThreads = 512;                          // AW workgroups: 8 waves, one 16-block each
static_assert(16 * kWin * kLine / 16 == kAwThreads, "one 16-element block per thread and window");

__host__ __device__ constexpr uint32_t a_region(bool aw, int LS) { return aw ? 2u * kWinSlot : alds_bytes(LS); }
// Whole-range weight scales (SB, with AW): each wave stages the scale bytes of
// its 16 rows for all the workgroup's lines once, in 16-byte chunks of two
// lines; row stride 16 ceil(LS / 2) + 4 bytes (whole chunks, and an odd
// number of words: the 16 rows of a quarter-wave hit distinct banks).
constexpr int kSbMaxLines = 64;        // lines whose scales one wave stages (8 loads per lane)
constexpr int kSbMaxLds = 160 * 1024;  // LDS a workgroup may allocate on gfx950 (static included)
__host__ __device__ constexpr uint32_t sb_stride(int LS) { return 16u * (((uint32_t)LS + 1u) >> 1) + 4u; }
// LDS of a workgroup: the activations, then the weight scales of every wave.
__host__ __device__ constexpr uint32_t lds_bytes(int LS, int waves, int G, bool aw = false, bool sb = false) {
  return a_region(aw, LS) + (sb ? (uint32_t)waves * 16u * sb_stride(LS) : (uint32_t)waves * (uint32_t)G * kScaleSlot);
}

// Workgroup barrier for LDS traffic only: this wave's LDS operations are done,
// vector-memory loads stay in flight, and the compiler moves no memory access
// across it.
__device__ __forceinline__ void barrier_lds() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));  // lgkmcnt(0) only
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

struct Plan {
  int G;   // 16-row groups per wave
  int RB;  // row blocks (waves with distinct rows) per workgroup
  int KS;  // K slices per workgroup (waves splitting its lines)
  int KZ;  // K splits over workgroups (grid.y); > 1 needs the workspace
  int LS;  // lines per K split (the last split may have fewer)
  int D;   // pairs of lines of weight loads in flight per wave
  int CP;  // cache policy of the weight loads (2: non-temporal)
  bool AW; // shared activation window (G = 1, RB = 8, KS = 1)
  bool SB; // with AW: each wave stages its weight scales for all its lines once (LS <= 64)
};

struct Split {
  float* part;    // [KZ][M][N] fp32 partial sums (KZ > 1)
  uint32_t* cnt;  // [row blocks] arrival counters, zero between calls
};

template <int G, int D, int CP, bool OUT_BF16, int MAXT = 512, bool AW = false, bool SB = false>
__global__ __launch_bounds__(MAXT) void gemm_m16_kernel(GemmArgs p, int KS, int LS, Split sp) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds_m16[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = blockDim.x >> 6;
  const int RB = nw / KS;
  const int rb = wave / KS, kc = wave - rb * KS;
  const int M = p.M, K = p.K, N = p.N;
  const int KZ = gridDim.y, kz = blockIdx.y;
  const uint32_t row_bytes = (uint32_t)K >> 1, srow = (uint32_t)K >> 4;
  const int L = K / kLine;
  // the workgroup's lines [l0, l0 + Lr)
  const int l0 = kz * LS;
  const int Lr = (L - l0 < LS) ? L - l0 : LS;
  // this wave's pairs of lines [u0, u1): lines [2 u0, t1)
  const int Pr = (Lr + 1) >> 1;
  const int PW = (Pr + KS - 1) / KS;
  const int u0 = kc * PW < Pr ? kc * PW : Pr;
  const int u1 = u0 + PW < Pr ? u0 + PW : Pr;
  const int t1 = 2 * u1 < Lr ? 2 * u1 : Lr;
  const uint32_t row0 = ((uint32_t)blockIdx.x * RB + rb) * 16u * G;

  const __amdgpu_buffer_rsrc_t ac = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.ac), (short)0, (int)((uint32_t)M * row_bytes), 0x00020000);
  const __amdgpu_buffer_rsrc_t as = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.as), (short)0, (int)((uint32_t)M * srow), 0x00020000);
  const __amdgpu_buffer_rsrc_t wc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.wc), (short)0, (int)((uint32_t)N * row_bytes), 0x00020000);
  const __amdgpu_buffer_rsrc_t ws = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.ws), (short)0, (int)((uint32_t)N * srow), 0x00020000);

  const int j = lane & 15, q = lane >> 4;
  // weight row row0 + j (+ 16g): 16 code bytes at 64 t + 16 q of line t
  const uint32_t w_off = (row0 + (uint32_t)j) * row_bytes + 16u * (uint32_t)q;

  // pair u: lines 2u and 2u + 1 relative to l0 (l0 is even)
  auto load = [&](int u) {
    Pair<G> d;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int t = 2 * u + h;
      const bool ok = t < t1;
      const uint32_t tl = (uint32_t)(l0 + t);
#pragma unroll
      for (int g = 0; g < G; ++g)
        d.w[h][g] = __builtin_amdgcn_raw_buffer_load_b128(wc, ok ? w_off + 16u * g * row_bytes + 64u * tl : kOOB, 0, CP);
    }
    return d;
  };
  // scale block starting at pair ub: lane j + 16c gets row j's scale bytes of
  // lines 2ub + 2c and 2ub + 2c + 1
  const uint32_t sb_off = (row0 + (uint32_t)j) * srow + 16u * (uint32_t)q;
  auto load_scales = [&](int ub, u4_t (&sb)[G]) {
    const int t = 2 * ub + 2 * q;
    const bool ok = t < t1;
#pragma unroll
    for (int g = 0; g < G; ++g)
      sb[g] = __builtin_amdgcn_raw_buffer_load_b128(ws, ok ? sb_off + 16u * g * srow + 8u * (uint32_t)(l0 + 2 * ub) : kOOB, 0, CP);
  };
  uint8_t* const w_slot = SB ? lds_m16 + a_region(AW, LS) + ((uint32_t)wave * 16u + (uint32_t)j) * sb_stride(LS)
                             : lds_m16 + a_region(AW, LS) + (uint32_t)wave * G * kScaleSlot + 64u * (uint32_t)j;
  auto park_scales = [&](const u4_t (&sb)[G]) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<uint32_t*>(w_slot + g * kScaleSlot + 4u * ((4u * q + i) ^ (uint32_t)j)) = sb[g][i];
    }
  };

  u4_t sX[G], sY[G];
  if constexpr (SB) {
    // this wave's 16 rows x lines [l0, l0 + Lr) of scale bytes: chunk c of row
    // r (16 bytes, lines 2c and 2c + 1) -> slot row r at 16 c (as dwords)
    const uint32_t nch = (uint32_t)(Lr + 1) >> 1, total = 16u * nch;
    u4_t v[8];
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8) {
      const uint32_t c = (uint32_t)lane + 64u * s8;
      const uint32_t r = c / nch, k = c - r * nch;
      v[s8] = __builtin_amdgcn_raw_buffer_load_b128(
          ws, c < total ? (row0 + r) * srow + 8u * (uint32_t)l0 + 16u * k : kOOB, 0, 0);
    }
    uint8_t* const slot0 = lds_m16 + a_region(AW, LS) + (uint32_t)wave * 16u * sb_stride(LS);
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8) {
      const uint32_t c = (uint32_t)lane + 64u * s8;
      const uint32_t r = c / nch, k = c - r * nch;
      if (c < total) {
#pragma unroll
        for (int i = 0; i < 4; ++i) *reinterpret_cast<uint32_t*>(slot0 + r * sb_stride(LS) + 16u * k + 4u * i) = v[s8][i];
      }
    }
  } else {
    load_scales(u0, sX);
    load_scales(u0 + 4, sY);
  }
  __builtin_amdgcn_sched_barrier(0);
  Pair<G> buf[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    buf[d] = load(u0 + d);
    __builtin_amdgcn_sched_barrier(0);
  }

  // AW: thread i dequantizes 16-element block i of each window: row i / 32,
  // block i % 32 (line (i % 32) / 8 of the window, block i % 8 of that line).
  const uint32_t aw_r = threadIdx.x >> 5, aw_b = threadIdx.x & 31;
  u2_t aw_c = {0u, 0u};
  uint32_t aw_s = 0;
  auto aw_load = [&](int w) {  // window w: lines 4w .. 4w+3 relative to l0
    const int t = kWin * w + (int)(aw_b >> 3);
    const bool ok = aw_r < (uint32_t)M && t < Lr;
    const uint32_t k16 = 8u * (uint32_t)(l0 + kWin * w) + aw_b;  // 16-element block index in the row
    aw_c = __builtin_amdgcn_raw_buffer_load_b64(ac, ok ? aw_r * row_bytes + 8u * k16 : kOOB, 0, 0);
    aw_s = __builtin_amdgcn_raw_buffer_load_b8(as, ok ? aw_r * srow + k16 : kOOB, 0, 0);
  };
  auto aw_store = [&](int w) {
    const _Float16 sc = (_Float16)e4m3_to_f32(aw_s);
    uint8_t* dst = lds_m16 + (uint32_t)(w & 1) * kWinSlot + aw_r * kWinRow + 32u * aw_b;
    *reinterpret_cast<h8_t*>(dst) = dequant8(aw_c.x, sc);
    *reinterpret_cast<h8_t*>(dst + 16) = dequant8(aw_c.y, sc);
  };
  if constexpr (AW) {
    aw_load(0);
    aw_store(0);
    aw_load(1);
    barrier_lds();
  } else {
  // Stage the activations of lines [l0, l0 + Lr): 16-byte code pieces and
  // 4-byte scale pieces, rows past M as zeros, a batch of loads per thread
  // before its stores.
  {
    const uint32_t cs = cstride(LS), ss = sstride(LS);
    const uint32_t cpr = 4u * (uint32_t)Lr, spr = 2u * (uint32_t)Lr;  // pieces per row
    const uint32_t cpieces = 16u * cpr, spieces = 16u * spr;
    for (uint32_t base = 0; base < cpieces; base += kFillBatch * blockDim.x) {
      u4_t v[kFillBatch];
#pragma unroll
      for (int s = 0; s < kFillBatch; ++s) {
        const uint32_t pc = base + threadIdx.x + blockDim.x * s;
        const uint32_t r = pc / cpr, c = pc - r * cpr;
        const bool ok = pc < cpieces && r < (uint32_t)M;
        v[s] = __builtin_amdgcn_raw_buffer_load_b128(ac, ok ? r * row_bytes + 64u * l0 + 16u * c : kOOB, 0, 0);
      }
#pragma unroll
      for (int s = 0; s < kFillBatch; ++s) {
        const uint32_t pc = base + threadIdx.x + blockDim.x * s;
        const uint32_t r = pc / cpr, c = pc - r * cpr;
        if (pc < cpieces) *reinterpret_cast<u4_t*>(lds_m16 + r * cs + 16u * c) = v[s];
      }
    }
    for (uint32_t base = 0; base < spieces; base += kFillBatch * blockDim.x) {
      uint32_t v[kFillBatch];
#pragma unroll
      for (int s = 0; s < kFillBatch; ++s) {
        const uint32_t pc = base + threadIdx.x + blockDim.x * s;
        const uint32_t r = pc / spr, c = pc - r * spr;
        const bool ok = pc < spieces && r < (uint32_t)M;
        v[s] = __builtin_amdgcn_raw_buffer_load_b32(as, ok ? r * srow + 8u * l0 + 4u * c : kOOB, 0, 0);
      }
#pragma unroll
      for (int s = 0; s < kFillBatch; ++s) {
        const uint32_t pc = base + threadIdx.x + blockDim.x * s;
        const uint32_t r = pc / spr, c = pc - r * spr;
        if (pc < spieces) *reinterpret_cast<uint32_t*>(lds_m16 + 16u * cs + r * ss + 4u * c) = v[s];
      }
    }
    __syncthreads();
    // Every load issued so far has landed (the staging stores waited for
    // them, and they are younger than the first weight loads).  Saying so
    // explicitly lets the compiler's wait-count analysis start the main loop
    // from an empty state; otherwise it cannot prove the staging loads done and
    // drains the whole prefetch ring at the top of every iteration.
    __builtin_amdgcn_s_waitcnt(0);
  }

  }

  f4_t acc[G][2];
#pragma unroll
  for (int g = 0; g < G; ++g) acc[g][0] = acc[g][1] = f4_t{0.f, 0.f, 0.f, 0.f};

  // activation row j, elements 32q .. 32q+31 of each line
  [[maybe_unused]] const uint8_t* a_lds = lds_m16 + (uint32_t)j * cstride(LS) + 16u * q;
  [[maybe_unused]] const uint8_t* as_lds = lds_m16 + 16u * cstride(LS) + (uint32_t)j * sstride(LS) + 2u * q;
  // line r of the current scale block: this lane's two scale bytes 2q, 2q+1
  auto w_scale = [&](int g, int r) {
    const uint32_t dw = 2u * (uint32_t)r + ((uint32_t)q >> 1);
    return (uint32_t)*reinterpret_cast<const uint16_t*>(w_slot + g * kScaleSlot + 4u * (dw ^ (uint32_t)j) +
                                                        2u * ((uint32_t)q & 1u));
  };
  auto compute = [&](const Pair<G>& d, int u, int p) {  // p: pair within the scale block
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int t = 2 * u + h;
      if (h == 1 && t >= t1) break;  // odd line count: no second half
      h8_t av[4];
      if constexpr (AW) {
        const uint8_t* src = lds_m16 + (uint32_t)((t / kWin) & 1) * kWinSlot + (uint32_t)j * kWinRow +
                             2u * (uint32_t)(kLine * (t % kWin) + 32 * q);
#pragma unroll
        for (int pc = 0; pc < 4; ++pc) av[pc] = *reinterpret_cast<const h8_t*>(src + 16 * pc);
      } else {
        const u4_t a = *reinterpret_cast<const u4_t*>(a_lds + 64u * t);
        const h2_t sa = e4m3x2_to_h2(*reinterpret_cast<const uint16_t*>(as_lds + 8u * t));
#pragma unroll
        for (int pc = 0; pc < 4; ++pc) av[pc] = dequant8(a[pc], pc < 2 ? sa.x : sa.y);
      }
      h2_t sw[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        if constexpr (SB) {
          sw[g] = e4m3x2_to_h2(*reinterpret_cast<const uint16_t*>(w_slot + 8u * (uint32_t)t + 2u * (uint32_t)q));
        } else {
          sw[g] = e4m3x2_to_h2(w_scale(g, 2 * p + h));
        }
      }
#pragma unroll
      for (int pc = 0; pc < 4; ++pc) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const h8_t wv = dequant8(d.w[h][g][pc], pc < 2 ? sw[g].x : sw[g].y);
          acc[g][pc & 1] = mfma16x16x32(av[pc], wv, acc[g][pc & 1]);
        }
      }
    }
  };

  // One scale block = 4 pairs; D (1, 2 or 4) divides it, so ring slot p % D
  // holds pair ub + p.  Two blocks per iteration alternate the scale
  // registers: park block k, request block k + 2, compute block k.
  auto block = [&](int ub, u4_t (&sb)[G]) {
    if constexpr (!SB) {
      park_scales(sb);
      load_scales(ub + 8, sb);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      if constexpr (AW) {
        if ((p & 1) == 0) {  // window w = (ub + p) / 2 begins: store window w + 1, request w + 2
          const int w = (ub + p) >> 1;
          aw_store(w + 1);
          aw_load(w + 2);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if (ub + p < u1) compute(buf[p % D], ub + p, p);
      __builtin_amdgcn_sched_barrier(0);
      buf[p % D] = load(ub + p + D);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (AW) {
        if (p & 1) barrier_lds();  // window w done everywhere; window w + 1 stored everywhere
      }
    }
  };
  for (int ub = u0; ub < u1; ub += 8) {
    block(ub, sX);
    if (ub + 4 < u1) block(ub + 4, sY);
  }

  // D[i][j] sits in lane j + 16(i/4), element i%4: activation row m = 4q + e,
  // weight row n = row0 + 16g + j.
  f4_t v[G];
#pragma unroll
  for (int g = 0; g < G; ++g) v[g] = acc[g][0] + acc[g][1];

  if (KS > 1) {  // add the K slices of the workgroup in order kc = 0, 1, ...
    __syncthreads();  // the staged activations are dead; reuse the LDS
    f4_t* part = reinterpret_cast<f4_t*>(lds_m16);
    if (kc != 0) {
#pragma unroll
      for (int g = 0; g < G; ++g) part[(wave * G + g) * 64 + lane] = v[g];
    }
    __syncthreads();
    if (kc == 0) {
      for (int k2 = 1; k2 < KS; ++k2) {
#pragma unroll
        for (int g = 0; g < G; ++g) v[g] += part[((wave + k2) * G + g) * 64 + lane];
      }
    }
  }

  if (KZ > 1) {  // add the KZ partial tiles of this row block in order kz = 0, 1, ...
    // The partials are written and read with device-scope (write-through,
    // coherent across the XCDs' L2s) stores and loads; each thread waits for
    // its stores to complete before the barrier after which one thread takes
    // the ticket, so no L2-wide write-back or invalidation is needed.
    __shared__ uint32_t ticket;
    if (kc == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const uint32_t n = row0 + 16u * g + j;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = 4 * q + e;
          if (n < (uint32_t)N && m < M)
            __hip_atomic_store(sp.part + ((int64_t)kz * M + m) * N + n, v[g][e], __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);  // this thread's stores have completed
    __syncthreads();
    if (threadIdx.x == 0)
      ticket = __hip_atomic_fetch_add(sp.cnt + blockIdx.x, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (ticket != (uint32_t)(KZ - 1)) return;
    if (kc == 0) {
      // Four splits' partials are requested at once (one round trip each
      // four), then added in the order z = 0, 1, ...
      f4_t tot[G];
#pragma unroll
      for (int g = 0; g < G; ++g) tot[g] = f4_t{0.f, 0.f, 0.f, 0.f};
      for (int z0 = 0; z0 < KZ; z0 += 4) {
        f4_t r[4][G];
#pragma unroll
        for (int zz = 0; zz < 4; ++zz) {
#pragma unroll
          for (int g = 0; g < G; ++g) {
            const uint32_t n = row0 + 16u * g + j;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int m = 4 * q + e;
              r[zz][g][e] = (z0 + zz < KZ && n < (uint32_t)N && m < M)
                                ? __hip_atomic_load(sp.part + ((int64_t)(z0 + zz) * M + m) * N + n, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT)
                                : 0.f;
            }
          }
        }
#pragma unroll
        for (int zz = 0; zz < 4; ++zz) {
          if (z0 + zz < KZ) {
#pragma unroll
            for (int g = 0; g < G; ++g) tot[g] += r[zz][g];
          }
        }
      }
#pragma unroll
      for (int g = 0; g < G; ++g) v[g] = tot[g];
    }
    if (threadIdx.x == 0) __hip_atomic_store(sp.cnt + blockIdx.x, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (kc != 0) return;

  const float gscale = (*p.ga) * (*p.gw);
  uint64_t best[4] = {0, 0, 0, 0};
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const uint32_t n = row0 + 16u * g + j;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = 4 * q + e;
      if (n < (uint32_t)N && m < M) {
        const float val = v[g][e] * gscale;
        if (p.argmax_keys) {
          const uint64_t key = argmax_key(val, n);
          best[e] = key > best[e] ? key : best[e];
        }
        if (p.out) {
          const int64_t o = (int64_t)m * N + n;
          if constexpr (OUT_BF16) {
            reinterpret_cast<uint16_t*>(p.out)[o] = f32_to_bf16_rne(val);
          } else {
            reinterpret_cast<float*>(p.out)[o] = val;
          }
        }
      }
    }
  }
  if (p.argmax_keys) {
    // the 16 lanes of a quarter share rows 4q .. 4q+3; the maximum key does
    // not depend on the order in which workgroups merge theirs.  Keys are
    // spread over kKeySlots slots per row to keep same-address atomics few.
    const uint32_t slot = blockIdx.x % kKeySlots;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint64_t b = best[e];
#pragma unroll
      for (int x = 1; x < 16; x <<= 1) {
        const uint64_t o = __shfl_xor(b, x);
        b = o > b ? o : b;
      }
      const int m = 4 * q + e;
      if (j == 0 && m < M && b != 0)
        atomicMax(reinterpret_cast<unsigned long long*>(p.argmax_keys) + slot * 16u + m, b);
    }
  }
}

int env_int(const char* name, int dflt) {
  const char* v = getenv(name);
  return v && *v ? atoi(v) : dflt;
}

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

// The most lines whose staged activations fit the LDS budget next to the
// scale slots of `slots` (waves x row groups): 49 for eight single-group waves.
constexpr int max_ls(int slots) {
  return (int)(((uint32_t)kMaxLdsM16 / 16u - 4u * kScaleSlot / 64u * (uint32_t)slots - 20u) / 72u);
}
static_assert(lds_bytes(max_ls(8), 8, 1) <= (uint32_t)kMaxLdsM16 && max_ls(32) >= 1, "LDS budget");
// the most dynamic LDS an SB launch asks for, well below the hardware limit
constexpr int kSbLds = (int)lds_bytes(kSbMaxLines, 8, 1, true, true);
static_assert(kSbLds + 1024 <= kSbMaxLds, "SB LDS budget");

// Launch plan, from a sweep over G x RB x KS x KZ x D x AW on MI355X at the
// LM head (16 x 5120 x 151936) and the tree-verification down-projection (16 x
// 25600 x 5120): one 16-row group per wave, eight waves with distinct rows per
// workgroup sharing one dequantized activation window (AW), each wave's weight
// scales for all its lines staged once (SB), two pairs of lines in flight,
// cached loads.  K
// is split over workgroups when the rows alone give fewer than ~4 waves per
// CU (up to about 7.5 waves per CU in all, at least 6 lines per split; below)
// or when the staged activations would not fit the LDS.
// NVFP4_M16_{G,RB,KS,KZ,D,CP}, NVFP4_M16_AW and NVFP4_M16_SB override the
// choice (tuning knobs; results change only by fp32 summation order).
// Without a workspace, a starved product with a long K goes to the skinny
// kernel instead (gemm_m16_preferred): more than twice this many lines.
constexpr int kSplitLines = 34;

Plan make_plan(const GemmArgs& a, bool can_split) {
  const int L = a.K / kLine;
  const int64_t cus = device_cus();
  Plan pl;
  pl.G = 1;
  const int e_g = env_int("NVFP4_M16_G", 0);
  if (e_g == 1 || e_g == 2 || e_g == 4) pl.G = e_g;
  // up to 16 waves per workgroup with one row group per wave (<= 128 VGPRs), else 8
  const int max_waves = pl.G == 1 ? 16 : 8;
  pl.RB = 8;
  const int e_rb = env_int("NVFP4_M16_RB", 0);
  if (e_rb >= 1 && e_rb <= max_waves) pl.RB = e_rb;
  pl.KS = 1;
  const int e_ks = env_int("NVFP4_M16_KS", 0);
  if (e_ks >= 1 && e_ks <= 8 && e_ks * pl.RB <= max_waves) pl.KS = e_ks;
  const int64_t waves_per_split = ((a.N + 16 * pl.G - 1) / (16 * pl.G)) * pl.KS;
  int KZ = 1;
  if (can_split) {
    if (waves_per_split < 4 * cus) {
      // Too few row groups to fill the GPU: split K until there are about 7.5
      // waves per compute unit in all, keeping at least 6 lines per split.
      // Measured at M = 16: K = 25600, N = 5120 is best at 6 splits (34
      // lines); at K = 5120, N = 1024 .. 8192 this takes 13.2-13.6 us down to
      // 9.8-11.7 us against the former ~34 lines per split (2 splits).
      const int64_t want = (15 * cus / 2 + waves_per_split - 1) / waves_per_split;
      const int cap = L / 6 > 1 ? L / 6 : 1;
      KZ = (int)(want < cap ? want : cap);
    }
    const int e_kz = env_int("NVFP4_M16_KZ", 0);
    if (e_kz >= 1) KZ = e_kz < L ? e_kz : L;
  }
  const bool aw = env_int("NVFP4_M16_AW", 1) == 1 && pl.G == 1 && pl.RB == 8 && pl.KS == 1 &&
                  env_int("NVFP4_M16_CP", 0) != 2;
  const int mls = aw ? 1 << 20 : max_ls(pl.RB * pl.KS * pl.G);  // AW stages no whole K range
  while ((L + KZ - 1) / KZ > mls) ++KZ;
  pl.LS = (L + KZ - 1) / KZ;
  pl.LS += pl.LS & (L > pl.LS ? 1 : 0);  // splits start on an even line (whole 128-byte runs)
  pl.KZ = (L + pl.LS - 1) / pl.LS;       // no split without lines
  pl.D = env_int("NVFP4_M16_D", 2);
  if (pl.D != 1 && pl.D != 2 && pl.D != 4) pl.D = 2;
  if (pl.G == 4 && pl.D == 4) pl.D = 2;  // would spill registers
  pl.CP = env_int("NVFP4_M16_CP", 0) == 2 ? 2 : 0;
  pl.AW = env_int("NVFP4_M16_AW", 1) == 1 && pl.G == 1 && pl.RB == 8 && pl.KS == 1 && pl.CP == 0;
  pl.SB = pl.AW && pl.LS <= kSbMaxLines && env_int("NVFP4_M16_SB", 1) == 1;
  return pl;
}

int64_t row_blocks(const GemmArgs& a, const Plan& pl) {
  return (a.N + 16 * pl.G * pl.RB - 1) / (16 * pl.G * pl.RB);
}

// Workspace layout: arrival counters (one per row block, rounded up to 256
// bytes), then the fp32 partial sums [KZ][M][N].
int64_t split_bytes(const GemmArgs& a, const Plan& pl) {
  if (pl.KZ <= 1) return 0;
  const int64_t cnt = (row_blocks(a, pl) * 4 + 255) / 256 * 256;
  return cnt + (int64_t)pl.KZ * a.M * a.N * 4;
}

template <int G, int D, int CP>
hipError_t launch_gd(const GemmArgs& a, const Plan& pl, Split sp, hipStream_t stream) {
  const dim3 grid((unsigned)row_blocks(a, pl), (unsigned)pl.KZ);
  const int nw = pl.RB * pl.KS;
  const uint32_t lds = lds_bytes(pl.LS, nw, G, pl.AW, pl.SB);  // >= the KS partial sums (nw * G KiB)
  if constexpr (G == 1 && CP == 0) {
    if (pl.SB) {
      static const hipError_t attr = [] {  // may exceed the default 64 KiB of dynamic LDS
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_m16_kernel<G, D, CP, true, 512, true, true>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, kSbLds);
        if (e == hipSuccess)
          e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_m16_kernel<G, D, CP, false, 512, true, true>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, kSbLds);
        return e;
      }();
      if (attr != hipSuccess) return attr;
      if (a.out_bf16) gemm_m16_kernel<G, D, CP, true, 512, true, true><<<grid, 64 * nw, lds, stream>>>(a, pl.KS, pl.LS, sp);
      else gemm_m16_kernel<G, D, CP, false, 512, true, true><<<grid, 64 * nw, lds, stream>>>(a, pl.KS, pl.LS, sp);
      return hipGetLastError();
    }
    if (pl.AW) {
      if (a.out_bf16) gemm_m16_kernel<G, D, CP, true, 512, true><<<grid, 64 * nw, lds, stream>>>(a, pl.KS, pl.LS, sp);
      else gemm_m16_kernel<G, D, CP, false, 512, true><<<grid, 64 * nw, lds, stream>>>(a, pl.KS, pl.LS, sp);
      return hipGetLastError();
    }
  }
  if constexpr (G == 1) {
    if (nw > 8) {
      if (a.out_bf16) gemm_m16_kernel<G, D, CP, true, 1024><<<grid, 64 * nw, lds, stream>>>(a, pl.KS, pl.LS, sp);
      else gemm_m16_kernel<G, D, CP, false, 1024><<<grid, 64 * nw, lds, stream>>>(a, pl.KS, pl.LS, sp);
      return hipGetLastError();
    }
  }
  if (a.out_bf16) gemm_m16_kernel<G, D, CP, true><<<grid, 64 * nw, lds, stream>>>(a, pl.KS, pl.LS, sp);
  else gemm_m16_kernel<G, D, CP, false><<<grid, 64 * nw, lds, stream>>>(a, pl.KS, pl.LS, sp);
  return hipGetLastError();
}

template <int G>
hipError_t launch_g(const GemmArgs& a, const Plan& pl, Split sp, hipStream_t stream) {
  if (pl.CP == 2) return launch_gd<G, 2, 2>(a, pl, sp, stream);
  switch (pl.D) {
    case 1: return launch_gd<G, 1, 0>(a, pl, sp, stream);
    case 4: return launch_gd<G, 4, 0>(a, pl, sp, stream);
    default: return launch_gd<G, 2, 0>(a, pl, sp, stream);
  }
}

bool have_workspace(const GemmArgs& a) { return a.workspace != nullptr && a.workspace_bytes > 0; }

}  // namespace

int64_t gemm_m16_workspace_bytes(const GemmArgs& a) {
  if (a.M < 1 || a.M > 16 || a.K % kLine != 0 || a.N < 1) return 0;
  return split_bytes(a, make_plan(a, true));
}

// Any K that is a multiple of 128: with a large enough workspace the lines
// are split over workgroups as needed; without one, the default plan (shared
// activation window) takes any K in one pass, and plans that stage the
// activations of the whole K range need them to fit the LDS (K <= 6272).
bool gemm_m16_supported(const GemmArgs& a) {
  if (a.M < 1 || a.M > 16 || a.K % kLine != 0) return false;
  const bool split = have_workspace(a) && a.workspace_bytes >= gemm_m16_workspace_bytes(a);
  return split || make_plan(a, false).KZ == 1;
}

// The weight-streaming GEMM picks this kernel unless, with no workspace to
// split K, it would leave most CUs idle on a long K (fewer than half as many
// workgroups as CUs and more than two splits' worth of lines: the tree-
// verification down-projection, 5120 x 25600, runs 67 us unsplit here against
// 31 us in the older skinny kernel and 21 us split).
// Short K (up to 8192, a multiple of 256) and at most 16384 rows: the skinny
// kernel, with fewer dependent memory round trips per wave, is faster than
// this one even split (same-process measurements at M = 16: K = 5120 and N =
// 1024 / 5120 / 8192 / 16384 12-19% / 16% / 19% / 4% faster, K = 2560 30%,
// K = 8192 4%; at N = 25600, K = 12288 or K = 25600 this kernel is 25-48%
// faster).  NVFP4_M16_SMALL=0 turns the rule off.
bool gemm_m16_small_prefers_skinny(const GemmArgs& a) {
  return a.M >= 3 && a.M <= 16 && a.K <= 8192 && a.K % 256 == 0 && a.N <= 16384 &&
         env_int("NVFP4_M16_SMALL", 1) == 1;
}

bool gemm_m16_preferred(const GemmArgs& a) {
  if (!gemm_m16_supported(a)) return false;
  if (gemm_m16_small_prefers_skinny(a)) return false;
  const bool split = have_workspace(a) && a.workspace_bytes >= gemm_m16_workspace_bytes(a);
  if (split) return true;
  const Plan pl = make_plan(a, false);
  return !(row_blocks(a, pl) * 2 < device_cus() && a.K / kLine > 2 * kSplitLines);
}

hipError_t launch_gemm_m16(const GemmArgs& a, hipStream_t stream) {
  const bool split = have_workspace(a) && a.workspace_bytes >= gemm_m16_workspace_bytes(a);
  const Plan pl = make_plan(a, split);
  if (pl.KZ > 1 && !split) return hipErrorInvalidValue;  // callers check gemm_m16_supported() first
  Split sp{nullptr, nullptr};
  if (pl.KZ > 1) {
    const int64_t cnt = (row_blocks(a, pl) * 4 + 255) / 256 * 256;
    sp.cnt = reinterpret_cast<uint32_t*>(a.workspace);
    sp.part = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(a.workspace) + cnt);
  }
  return pl.G == 4 ? launch_g<4>(a, pl, sp, stream) : pl.G == 2 ? launch_g<2>(a, pl, sp, stream)
                                                              : launch_g<1>(a, pl, sp, stream);
}

}  // namespace nvfp4
