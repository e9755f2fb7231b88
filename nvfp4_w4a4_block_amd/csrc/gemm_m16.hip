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
//     32q+31, blocks 2q and 2q+1), a 64-byte run per row; the two lines of a
//     128-byte run are requested back to back;
//   - the codes are dequantized exactly to f16 with their E4M3 scale (E2M1 x
//     E4M3 has at most 6 significant bits and lies in [2^-10, 2688]) and are
//     the B operand of v_mfma_f32_16x16x32_f16, column j = weight row j.  For
//     piece p (elements 32q + 8p .. +7 of every lane) the MFMA's k = 8q + e
//     is element 32q + 8p + e, so four MFMAs cover the line and every column
//     of every MFMA is used;
//   - the A operand is the 16 activation rows (rows past M read zeros), laid
//     out the same way.  The eight waves of a workgroup (one 16-row group of
//     weights each, all on the same lines) share a double-buffered window of
//     4 lines x 16 activation rows, dequantized to f16 in LDS once per
//     workgroup: each thread converts one 16-element block per window.
//     Every product is exact; the fp32 accumulation is the only rounding.
//
// Weight scales: each wave stages the scale bytes of its 16 rows for all its
// lines once, at the start, in whole 16-byte chunks (up to 64 lines); for
// more lines it fetches them 8 lines at a time into a per-wave LDS slot.
// Per-lane 2-byte scale loads from memory touch 16 cache lines per 128 bytes
// and cost as much time as the codes (measured: the code stream alone runs at
// 5.5 TB/s, with such scale loads at 3.6 TB/s).
//
// When K is long and N small (tree verification of a down-projection:
// N = 5120 rows, K = 25600) the lines are also split over KZ workgroups
// (grid.y): each writes its fp32 partial tile to a caller-owned workspace,
// and the last of the KZ workgroups of a row block to arrive (a counter per
// row block) adds the KZ partials in the order kz = 0, 1, ... and writes the
// result, then resets the counter to zero.  The sum does not depend on which
// workgroup arrives last, so results are bit-identical from run to run.
#include "device_common.h"
#include "launch.h"

namespace nvfp4 {
namespace {

constexpr uint32_t kOOB = 0x80000000u;  // buffer offset past any array: loads read zeros
constexpr int kLine = 128;              // K-elements per line
constexpr int kWaves = 8;               // waves per workgroup, one 16-row group of weights each
constexpr int kThreads = 64 * kWaves;
constexpr int kD = 2;                   // pairs of lines of weight loads in flight per wave

// Two consecutive lines (a 128-byte run of each row), loaded back to back so
// that both halves of a row's 128-byte segment are requested together.
struct Pair {
  u4_t w[2];  // weight codes of each half
};

// 8-line scale blocks (more than kSbMaxLines lines per wave): lane j + 16c
// loads 16 bytes of row j (lines 2c and 2c + 1 of the block), so one load
// covers 16 rows x 64 contiguous bytes, and the block is parked in a per-wave
// LDS slot of 16 rows x 64 bytes whose dwords are XOR-swizzled by row (dword d
// of row j at 4 (d ^ j)), so the 2-byte reads of a quarter-wave (16 rows, one
// offset) hit distinct banks.
constexpr uint32_t kScaleSlot = 16u * 64u;  // LDS bytes per wave

// Shared activation window: 4 lines of the 16 activation rows in f16,
// double-buffered (row stride 1040 bytes = 65 16-byte units, odd, so a
// quarter-wave's 16 rows hit distinct banks).
constexpr int kWin = 4;                                  // lines per window
constexpr uint32_t kWinRow = kWin * kLine * 2 + 16;      // bytes per row of a window
constexpr uint32_t kWinSlot = 16u * kWinRow;             // one window
static_assert(16 * kWin * kLine / 16 == kThreads, "one 16-element block per thread and window");
constexpr uint32_t kARegion = 2u * kWinSlot;

// Whole-range weight scales (SB): each wave stages the scale bytes of its 16
// rows for all the workgroup's lines once, in 16-byte chunks of two lines;
// row stride 16 ceil(LS / 2) + 4 bytes (whole chunks, and an odd number of
// words: the 16 rows of a quarter-wave hit distinct banks).
constexpr int kSbMaxLines = 64;        // lines whose scales one wave stages (8 loads per lane)
constexpr int kLdsMax = 160 * 1024;    // LDS a workgroup may allocate on gfx950 (static included)
__host__ __device__ constexpr uint32_t sb_stride(int LS) { return 16u * (((uint32_t)LS + 1u) >> 1) + 4u; }
// LDS of a workgroup: the activation windows, then the weight scales of every wave.
__host__ __device__ constexpr uint32_t lds_bytes(int LS, bool sb) {
  return kARegion + (sb ? (uint32_t)kWaves * 16u * sb_stride(LS) : (uint32_t)kWaves * kScaleSlot);
}
constexpr int kSbLds = (int)lds_bytes(kSbMaxLines, true);  // the most dynamic LDS a launch asks for
static_assert(kSbLds + 1024 <= kLdsMax, "SB LDS budget");

// Workgroup barrier for LDS traffic only: this wave's LDS operations are done,
// vector-memory loads stay in flight, and the compiler moves no memory access
// across it.
__device__ __forceinline__ void barrier_lds() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));  // lgkmcnt(0) only
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

struct Split {
  float* part;    // [KZ][M][N] fp32 partial sums (KZ > 1)
  uint32_t* cnt;  // [row blocks] arrival counters, zero between calls
};

template <bool OUT_BF16, bool SB>
__global__ __launch_bounds__(kThreads) void gemm_m16_kernel(GemmArgs p, int LS, Split sp) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds_m16[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int M = p.M, K = p.K, N = p.N;
  const int KZ = gridDim.y, kz = blockIdx.y;
  const uint32_t row_bytes = (uint32_t)K >> 1, srow = (uint32_t)K >> 4;
  const int L = K / kLine;
  // the workgroup's lines [l0, l0 + Lr), as pairs [0, u1)
  const int l0 = kz * LS;
  const int Lr = (L - l0 < LS) ? L - l0 : LS;
  const int u1 = (Lr + 1) >> 1;
  const uint32_t row0 = ((uint32_t)blockIdx.x * kWaves + wave) * 16u;

  const __amdgpu_buffer_rsrc_t ac = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.ac), (short)0, (int)((uint32_t)M * row_bytes), 0x00020000);
  const __amdgpu_buffer_rsrc_t as = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.as), (short)0, (int)((uint32_t)M * srow), 0x00020000);
  const __amdgpu_buffer_rsrc_t wc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.wc), (short)0, (int)((uint32_t)N * row_bytes), 0x00020000);
  const __amdgpu_buffer_rsrc_t ws = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.ws), (short)0, (int)((uint32_t)N * srow), 0x00020000);

  const int j = lane & 15, q = lane >> 4;
  // weight row row0 + j: 16 code bytes at 64 t + 16 q of line t
  const uint32_t w_off = (row0 + (uint32_t)j) * row_bytes + 16u * (uint32_t)q;

  // pair u: lines 2u and 2u + 1 relative to l0 (l0 is even)
  auto load = [&](int u) {
    Pair d;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int t = 2 * u + h;
      const uint32_t tl = (uint32_t)(l0 + t);
      d.w[h] = __builtin_amdgcn_raw_buffer_load_b128(wc, t < Lr ? w_off + 64u * tl : kOOB, 0, 0);
    }
    return d;
  };
  // 8-line scale block starting at pair ub: lane j + 16c gets row j's scale
  // bytes of lines 2ub + 2c and 2ub + 2c + 1
  const uint32_t sb_off = (row0 + (uint32_t)j) * srow + 16u * (uint32_t)q;
  auto load_scales = [&](int ub) {
    const int t = 2 * ub + 2 * q;
    return __builtin_amdgcn_raw_buffer_load_b128(ws, t < Lr ? sb_off + 8u * (uint32_t)(l0 + 2 * ub) : kOOB, 0, 0);
  };
  uint8_t* const w_slot = SB ? lds_m16 + kARegion + ((uint32_t)wave * 16u + (uint32_t)j) * sb_stride(LS)
                             : lds_m16 + kARegion + (uint32_t)wave * kScaleSlot + 64u * (uint32_t)j;
  auto park_scales = [&](const u4_t& sb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<uint32_t*>(w_slot + 4u * ((4u * q + i) ^ (uint32_t)j)) = sb[i];
  };

  u4_t sX = {0u, 0u, 0u, 0u}, sY = {0u, 0u, 0u, 0u};
  // Thread i dequantizes 16-element block i of each window: row i / 32,
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
  // Set-up in one memory round trip: the weight scales (or the first two
  // 8-line scale blocks), the first activation window and the first weight
  // loads are all requested before anything waits; the scale staging and the
  // window store then wait only for their own loads, which are earlier in the
  // in-order load counter (measured: the K-split down-projection 4.7% faster,
  // the LM head unchanged).
  u4_t sbv[8];
  [[maybe_unused]] const uint32_t nch = (uint32_t)(Lr + 1) >> 1, total = 16u * nch;
  if constexpr (SB) {
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8) {
      const uint32_t c = (uint32_t)lane + 64u * s8;
      const uint32_t r = c / nch, k = c - r * nch;
      sbv[s8] = __builtin_amdgcn_raw_buffer_load_b128(
          ws, c < total ? (row0 + r) * srow + 8u * (uint32_t)l0 + 16u * k : kOOB, 0, 0);
    }
  } else {
    sX = load_scales(0);
    sY = load_scales(4);
  }
  aw_load(0);
  __builtin_amdgcn_sched_barrier(0);
  Pair buf[kD];
#pragma unroll
  for (int d = 0; d < kD; ++d) {
    buf[d] = load(d);
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (SB) {
    // this wave's 16 rows x lines [l0, l0 + Lr) of scale bytes: chunk c of row
    // r (16 bytes, lines 2c and 2c + 1) -> slot row r at 16 c (as dwords)
    uint8_t* const slot0 = lds_m16 + kARegion + (uint32_t)wave * 16u * sb_stride(LS);
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8) {
      const uint32_t c = (uint32_t)lane + 64u * s8;
      const uint32_t r = c / nch, k = c - r * nch;
      if (c < total) {
#pragma unroll
        for (int i = 0; i < 4; ++i) *reinterpret_cast<uint32_t*>(slot0 + r * sb_stride(LS) + 16u * k + 4u * i) = sbv[s8][i];
      }
    }
  }
  aw_store(0);
  aw_load(1);
  barrier_lds();

  f4_t acc[2] = {f4_t{0.f, 0.f, 0.f, 0.f}, f4_t{0.f, 0.f, 0.f, 0.f}};

  // line r of the current 8-line scale block: this lane's two scale bytes 2q, 2q+1
  auto w_scale = [&](int r) {
    const uint32_t dw = 2u * (uint32_t)r + ((uint32_t)q >> 1);
    return (uint32_t)*reinterpret_cast<const uint16_t*>(w_slot + 4u * (dw ^ (uint32_t)j) + 2u * ((uint32_t)q & 1u));
  };
  auto compute = [&](const Pair& d, int u, int pb) {  // pb: pair within the scale block
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int t = 2 * u + h;
      if (h == 1 && t >= Lr) break;  // odd line count: no second half
      h8_t av[4];
      const uint8_t* src = lds_m16 + (uint32_t)((t / kWin) & 1) * kWinSlot + (uint32_t)j * kWinRow +
                           2u * (uint32_t)(kLine * (t % kWin) + 32 * q);
#pragma unroll
      for (int pc = 0; pc < 4; ++pc) av[pc] = *reinterpret_cast<const h8_t*>(src + 16 * pc);
      h2_t sw;
      if constexpr (SB) {
        sw = e4m3x2_to_h2(*reinterpret_cast<const uint16_t*>(w_slot + 8u * (uint32_t)t + 2u * (uint32_t)q));
      } else {
        sw = e4m3x2_to_h2(w_scale(2 * pb + h));
      }
#pragma unroll
      for (int pc = 0; pc < 4; ++pc) {
        const h8_t wv = dequant8(d.w[h][pc], pc < 2 ? sw.x : sw.y);
        acc[pc & 1] = mfma16x16x32(av[pc], wv, acc[pc & 1]);
      }
    }
  };

  // One scale block = 4 pairs; kD divides it, so ring slot pb % kD holds
  // pair ub + pb.  Without SB, two blocks per iteration alternate the scale
  // registers: park block k, request block k + 2, compute block k.  Every
  // second pair starts a window: store window w + 1, request window w + 2,
  // and one LDS barrier per window orders the ring.
  auto block = [&](int ub, u4_t& sb) {
    if constexpr (!SB) {
      park_scales(sb);
      sb = load_scales(ub + 8);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int pb = 0; pb < 4; ++pb) {
      if ((pb & 1) == 0) {  // window w = (ub + pb) / 2 begins
        const int w = (ub + pb) >> 1;
        aw_store(w + 1);
        aw_load(w + 2);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (ub + pb < u1) compute(buf[pb % kD], ub + pb, pb);
      __builtin_amdgcn_sched_barrier(0);
      buf[pb % kD] = load(ub + pb + kD);
      __builtin_amdgcn_sched_barrier(0);
      if (pb & 1) barrier_lds();  // window w done everywhere; window w + 1 stored everywhere
    }
  };
  for (int ub = 0; ub < u1; ub += 8) {
    block(ub, sX);
    if (ub + 4 < u1) block(ub + 4, sY);
  }

  // D[i][j] sits in lane j + 16(i/4), element i%4: activation row m = 4q + e,
  // weight row n = row0 + j.
  f4_t v = acc[0] + acc[1];
  const uint32_t n = row0 + (uint32_t)j;

  if (KZ > 1) {  // add the KZ partial tiles of this row block in order kz = 0, 1, ...
    // Ordering: every thread writes its partials with agent-scope stores and
    // waits for them to complete (the workgroup barrier alone compiles to no
    // wait on other waves' stores); after the barrier the thread that takes
    // the arrival ticket issues an agent-scope release fence, so everything
    // that happens before the barrier happens before the ticket; the last
    // workgroup to arrive takes an agent-scope acquire fence before it reads
    // the partials, with agent-scope loads.
    __shared__ uint32_t ticket;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = 4 * q + e;
      if (n < (uint32_t)N && m < M)
        __hip_atomic_store(sp.part + ((int64_t)kz * M + m) * N + n, v[e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_s_waitcnt(0);  // this thread's stores have completed
    __syncthreads();
    if (threadIdx.x == 0) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      const uint32_t t = __hip_atomic_fetch_add(sp.cnt + blockIdx.x, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (t == (uint32_t)(KZ - 1)) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      ticket = t;
    }
    __syncthreads();
    if (ticket != (uint32_t)(KZ - 1)) return;
    // Four splits' partials are requested at once (one round trip each
    // four), then added in the order z = 0, 1, ...
    f4_t tot = {0.f, 0.f, 0.f, 0.f};
    for (int z0 = 0; z0 < KZ; z0 += 4) {
      f4_t r[4];
#pragma unroll
      for (int zz = 0; zz < 4; ++zz) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = 4 * q + e;
          r[zz][e] = (z0 + zz < KZ && n < (uint32_t)N && m < M)
                         ? __hip_atomic_load(sp.part + ((int64_t)(z0 + zz) * M + m) * N + n, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT)
                         : 0.f;
        }
      }
#pragma unroll
      for (int zz = 0; zz < 4; ++zz) {
        if (z0 + zz < KZ) tot += r[zz];
      }
    }
    v = tot;
    if (threadIdx.x == 0) __hip_atomic_store(sp.cnt + blockIdx.x, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  const float gscale = (*p.ga) * (*p.gw);
  uint64_t best[4] = {0, 0, 0, 0};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int m = 4 * q + e;
    if (n < (uint32_t)N && m < M) {
      const float val = v[e] * gscale;
      if (p.argmax_keys) best[e] = argmax_key(val, n);
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

struct Plan {
  int KZ;   // K splits over workgroups (grid.y); > 1 needs the workspace
  int LS;   // lines per K split (the last split may have fewer)
  bool SB;  // each wave stages its weight scales for all its lines once (LS <= kSbMaxLines)
};

// Launch plan (from a sweep on MI355X at the LM head, 16 x 5120 x 151936, and
// the tree-verification down-projection, 16 x 25600 x 5120, over row groups
// per wave, waves per workgroup, K slices, loads in flight, cache policy and
// activation staging: one 16-row group per wave, eight waves sharing one
// dequantized activation window, two pairs of lines in flight, cached loads).
// With a workspace, K is split over workgroups when the row groups alone give
// fewer than 4 waves per CU: until there are about 7.5 waves per CU in all,
// with at least 6 lines per split.  Measured at M = 16: K = 25600, N = 5120 is
// best at 6 splits (34 lines, the best of 2-20); at K = 5120 and N = 1024 ..
// 8192 this takes 13.2-13.6 us down to 9.8-11.7 us against the former ~34
// lines per split.
Plan make_plan(const GemmArgs& a, bool can_split) {
  const int L = a.K / kLine;
  const int64_t cus = device_cus();
  const int64_t waves = (a.N + 15) / 16;
  int KZ = 1;
  if (can_split && waves < 4 * cus) {
    const int64_t want = (15 * cus / 2 + waves - 1) / waves;
    const int cap = L / 6 > 1 ? L / 6 : 1;
    KZ = (int)(want < cap ? want : cap);
  }
  Plan pl;
  pl.LS = (L + KZ - 1) / KZ;
  pl.LS += pl.LS & (L > pl.LS ? 1 : 0);  // splits start on an even line (whole 128-byte runs)
  pl.KZ = (L + pl.LS - 1) / pl.LS;       // no split without lines
  pl.SB = pl.LS <= kSbMaxLines;
  return pl;
}

int64_t row_blocks(const GemmArgs& a) { return (a.N + 16 * kWaves - 1) / (16 * kWaves); }

// Workspace layout: arrival counters (one per row block, rounded up to 256
// bytes), then the fp32 partial sums [KZ][M][N].
int64_t split_bytes(const GemmArgs& a, const Plan& pl) {
  if (pl.KZ <= 1) return 0;
  const int64_t cnt = (row_blocks(a) * 4 + 255) / 256 * 256;
  return cnt + (int64_t)pl.KZ * a.M * a.N * 4;
}

template <bool OUT_BF16, bool SB>
hipError_t launch_plan(const GemmArgs& a, const Plan& pl, Split sp, hipStream_t stream) {
  auto kern = &gemm_m16_kernel<OUT_BF16, SB>;
  if constexpr (SB) {
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, kSbLds);
    if (attr != hipSuccess) return attr;  // may exceed the default 64 KiB of dynamic LDS
  }
  const dim3 grid((unsigned)row_blocks(a), (unsigned)pl.KZ);
  kern<<<grid, kThreads, lds_bytes(pl.LS, SB), stream>>>(a, pl.LS, sp);
  return hipGetLastError();
}

bool have_workspace(const GemmArgs& a) { return a.workspace != nullptr && a.workspace_bytes > 0; }

// Without a workspace, a starved product with a long K goes to the skinny
// kernel instead: fewer than half as many workgroups as CUs and more than
// this many lines (the tree-verification down-projection, 5120 x 25600, runs
// 67 us unsplit here against 31 us in the skinny kernel and 21 us split).
constexpr int kStarvedLines = 68;

}  // namespace

int64_t gemm_m16_workspace_bytes(const GemmArgs& a) {
  if (a.M < 1 || a.M > 16 || a.K % kLine != 0 || a.N < 1) return 0;
  return split_bytes(a, make_plan(a, true));
}

// Any M in 1..16 and K a multiple of 128: the shared activation window takes
// any K in one pass, and a large enough workspace lets it split.
bool gemm_m16_supported(const GemmArgs& a) { return a.M >= 1 && a.M <= 16 && a.K % kLine == 0 && a.N >= 1; }

// Short K (a multiple of 256 up to 8192) and at most 16384 rows: the skinny
// kernel, with fewer dependent memory round trips per wave, is faster than
// this one even split (same-process measurements at M = 16: K = 5120 and N =
// 1024 / 5120 / 8192 / 16384 12-19% / 16% / 19% / 4% faster, K = 2560 30%,
// K = 8192 4%; at N = 25600, K = 12288 or K = 25600 this kernel is 25-48%
// faster).
bool gemm_m16_small_prefers_skinny(const GemmArgs& a) {
  return a.M >= 3 && a.M <= 16 && a.K <= 8192 && a.K % 256 == 0 && a.N <= 16384;
}

bool gemm_m16_preferred(const GemmArgs& a) {
  if (a.M < 3 || !gemm_m16_supported(a) || gemm_m16_small_prefers_skinny(a)) return false;
  const bool split = have_workspace(a) && a.workspace_bytes >= gemm_m16_workspace_bytes(a);
  if (split) return true;
  return !(row_blocks(a) * 2 < device_cus() && a.K / kLine > kStarvedLines);
}

hipError_t launch_gemm_m16(const GemmArgs& a, hipStream_t stream) {
  const bool split = have_workspace(a) && a.workspace_bytes >= gemm_m16_workspace_bytes(a);
  const Plan pl = make_plan(a, split);
  Split sp{nullptr, nullptr};
  if (pl.KZ > 1) {
    const int64_t cnt = (row_blocks(a) * 4 + 255) / 256 * 256;
    sp.cnt = reinterpret_cast<uint32_t*>(a.workspace);
    sp.part = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(a.workspace) + cnt);
  }
  if (pl.SB) return a.out_bf16 ? launch_plan<true, true>(a, pl, sp, stream) : launch_plan<false, true>(a, pl, sp, stream);
  return a.out_bf16 ? launch_plan<true, false>(a, pl, sp, stream) : launch_plan<false, false>(a, pl, sp, stream);
}

}  // namespace nvfp4
