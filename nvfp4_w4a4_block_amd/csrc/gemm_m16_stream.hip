// Weight-streaming GEMM for up to 16 activation rows over a tall weight
// matrix: the language-model head applied to every node of a 16-node
// candidate tree (page "TensorRT Edge-LLM Completes the MLPerf Edge Agentic
// Benchmark 6.4x Faster on Jetson AGX Thor", sections "Using tree-based
// multi-token prediction to accelerate LLM inference" and "Using NVFP4
// quantization to accelerate Qwen3.6-27B inference").  The product reads
// every weight once, so it is organised like a read stream:
//
//   - one workgroup of 8 waves per CU, resident for the whole product; the
//     16-row weight groups are dealt out in contiguous runs, one run per wave
//     (4-5 groups per wave at the LM head), so every wave reads as much as
//     every other and no workgroup starts late;
//   - each wave keeps D loads in flight (a load is 128-byte runs of 8 of its
//     16 rows: two lines of 128 K-elements; the two loads of a pair of lines
//     are exchanged by half-rows into the MFMA operand layout), and the ring
//     runs on from one group to the next and from one K chunk to the next, so
//     the loads never stop;
//   - K is walked in chunks of C lines.  The activation rows of the current
//     chunk (all 16 rows, rows past M zero) are dequantized exactly to f16
//     once per workgroup into LDS and read by every wave as the A operand of
//     v_mfma_f32_16x16x32_f16; the codes of the next chunk are already in
//     registers when the chunk ends, so a chunk change costs two workgroup
//     barriers and a few LDS stores while the weight loads stay in flight;
//   - the weight scale bytes of a (chunk, group) block, 16 rows x 8C bytes,
//     are copied into a per-wave LDS slot by buffer->LDS loads one block
//     ahead; the codes are dequantized exactly to f16 with them (E2M1 x E4M3
//     has at most 6 significant bits and lies in [2^-10, 2688]) and are the B
//     operand, column j = weight row j.  Piece p of a lane's 32 elements is
//     MFMA k-range 8q .. 8q+7, the same permutation of K on both operands.
//
// Every product is exact; the only roundings are the fp32 accumulation, in a
// fixed order (per line, alternating two accumulators; per block, added to
// the group's sum in chunk order), so results are identical from run to run.
// Output: the same epilogue as the M-tile kernel (x g_a g_w, bf16 or fp32,
// and the row-argmax keys when asked).  For the verification of a candidate
// tree the last workgroup to finish also folds the argmax keys and runs the
// greedy acceptance (no separate launch after the product).
#include "device_common.h"
#include "launch.h"

namespace nvfp4 {
namespace {

constexpr uint32_t kOOB = 0x80000000u;  // buffer offset past any array: loads read zeros
constexpr int kLine = 128;              // K-elements per line
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxG = 8;                // 16-row groups per wave (one accumulator tile each)

// f16 bytes of one activation row of a chunk in LDS: C lines, plus 16 bytes
// so that the 16 rows of a quarter-wave (an odd number of 16-byte units
// apart) fall in distinct banks.
template <int C> constexpr uint32_t a_row_bytes() { return (uint32_t)C * kLine * 2u + 16u; }
// One weight-scale slot: 16 rows x 8C bytes, in whole 1 KiB load instructions.
template <int C> constexpr uint32_t scale_slot_bytes() { return ((16u * 8u * C + 1023u) / 1024u) * 1024u; }
// Staging of the next chunk's activation codes (16 rows x 64C bytes) and
// scale bytes (16 rows x 8C bytes), in whole 1 KiB load instructions.
template <int C> constexpr uint32_t stage_code_bytes() { return 16u * 64u * C; }
template <int C> constexpr uint32_t stage_scale_bytes() { return ((16u * 8u * C + 1023u) / 1024u) * 1024u; }
template <int C> constexpr uint32_t stream_lds_bytes() {
  return 16u * a_row_bytes<C>() + (uint32_t)kWaves * 2u * scale_slot_bytes<C>() + stage_code_bytes<C>() +
         stage_scale_bytes<C>();
}
static_assert(stream_lds_bytes<20>() <= 160u * 1024u, "LDS budget");

#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

__device__ __forceinline__ void barrier_lds() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));  // lgkmcnt(0) only
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// "At most n vector-memory operations outstanding" (n < 64).
template <int n> __device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int C, int D, bool OUT_BF16>
__global__ __launch_bounds__(kThreads) void gemm_m16_stream_kernel(GemmArgs p, int NG) {
  static_assert(C % D == 0 && C % 4 == 0, "ring depth divides the chunk; 4 threads per activation line");
  extern __shared__ __attribute__((aligned(16))) uint8_t lds_s[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int M = p.M, K = p.K, N = p.N;
  const uint32_t row_bytes = (uint32_t)K >> 1, srow = (uint32_t)K >> 4;
  const int NC = K / (kLine * C);

  // This wave's groups [g0, g0 + Gw): contiguous runs of equal length +-1.
  const int64_t W = (int64_t)gridDim.x * kWaves, w = (int64_t)blockIdx.x * kWaves + wave;
  const int g0 = (int)(w * NG / W);
  const int Gw = (int)((w + 1) * NG / W) - g0;

  const __amdgpu_buffer_rsrc_t ac = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.ac), (short)0, (int)((uint32_t)M * row_bytes), 0x00020000);
  const __amdgpu_buffer_rsrc_t as = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.as), (short)0, (int)((uint32_t)M * srow), 0x00020000);
  const __amdgpu_buffer_rsrc_t wc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.wc), (short)0, (int)((uint32_t)N * row_bytes), 0x00020000);
  const __amdgpu_buffer_rsrc_t ws = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.ws), (short)0, (int)((uint32_t)N * srow), 0x00020000);

  uint8_t* const a_lds = lds_s;
  uint8_t* const slots = lds_s + 16u * a_row_bytes<C>() + (uint32_t)wave * 2u * scale_slot_bytes<C>();

  uint8_t* const stage_c = lds_s + 16u * a_row_bytes<C>() + (uint32_t)kWaves * 2u * scale_slot_bytes<C>();
  uint8_t* const stage_s = stage_c + stage_code_bytes<C>();

  // ---- activation chunk c: the workgroup's waves copy its codes and scale
  // bytes into the staging area with buffer->LDS loads (load instruction i,
  // of 16-byte units 64 i .. 64 i + 63, is issued by wave i % 8), then
  // thread i dequantizes 16-element blocks i + 512 s of the chunk (row
  // b / 8C, block b % 8C of that row's chunk) into the f16 A region ----
  constexpr int kCI = (int)(stage_code_bytes<C>() / 1024u), kSIa = (int)(stage_scale_bytes<C>() / 1024u);
  auto a_issue = [&](int c) {
    for (int i = wave; i < kCI; i += kWaves) {
      const uint32_t pos = 64u * i + (uint32_t)lane;
      const uint32_t r = pos / (4u * C), u = pos % (4u * C);
      const uint32_t off = r < (uint32_t)M ? r * row_bytes + 64u * C * (uint32_t)c + 16u * u : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ac, LDS_PTR(stage_c + 1024u * i), 16, off, 0, 0, 0);
    }
    for (int i = wave; i < kSIa; i += kWaves) {
      const uint32_t pos = 64u * i + (uint32_t)lane;
      const uint32_t r = pos / (C / 2u), u = pos % (C / 2u);
      const uint32_t off = r < (uint32_t)M ? r * srow + 8u * C * (uint32_t)c + 16u * u : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(as, LDS_PTR(stage_s + 1024u * i), 16, off, 0, 0, 0);
    }
  };
  constexpr int kAB = C / 4;  // 16-element activation blocks per thread and chunk
  auto a_store = [&]() {
#pragma unroll
    for (int s = 0; s < kAB; ++s) {
      const uint32_t b = threadIdx.x + (uint32_t)kThreads * s;
      const uint32_t r = b / (8u * C), k16 = b % (8u * C);
      const u2_t codes = *reinterpret_cast<const u2_t*>(stage_c + r * 64u * C + 8u * k16);
      const _Float16 sc = (_Float16)e4m3_to_f32(stage_s[r * 8u * C + k16]);
      uint8_t* dst = a_lds + r * a_row_bytes<C>() + 32u * k16;
      *reinterpret_cast<h8_t*>(dst) = dequant8(codes.x, sc);
      *reinterpret_cast<h8_t*>(dst + 16) = dequant8(codes.y, sc);
    }
  };

  // ---- weight scales of block (chunk c, group g) into slot `sl`: position
  // 16 x (64 i + lane) holds 16-byte piece k of row j (j = pos / (C/2),
  // k = pos % (C/2)), so row j's bytes sit at 8C j .. 8C j + 8C - 1 ----
  constexpr uint32_t kSC = C / 2;  // 16-byte pieces per row
  constexpr int kSI = (int)(scale_slot_bytes<C>() / 1024u);
  auto s_issue = [&](int c, int g, int sl) {
    uint8_t* base = slots + (uint32_t)sl * scale_slot_bytes<C>();
#pragma unroll
    for (int i = 0; i < kSI; ++i) {
      const uint32_t pos = 64u * i + (uint32_t)lane;
      const uint32_t jj = pos / kSC, k = pos % kSC;
      const uint32_t off = jj < 16u ? ((uint32_t)g * 16u + jj) * srow + 8u * C * (uint32_t)c + 16u * k : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ws, LDS_PTR(base + 1024u * i), 16, off, 0, 0, 0);
    }
  };

  const int j = lane & 15, q = lane >> 4;
  // Weight loads come in pairs per pair of lines (2u, 2u + 1) of a block:
  // load 2u covers rows 0-7, load 2u + 1 rows 8-15, each row's whole 128-byte
  // run of the two lines (8 rows x 128 bytes per instruction: whole cache
  // lines; measured faster than 16 rows x 64 bytes).  Lane j + 16q of load
  // 2u + h reads row (j & 7) + 8h, line 2u + (j >> 3), bytes 16q .. 16q+15.
  // wbase is the lane's address of load 0 of the block starting at line c*C
  // of group g; load v adds woff(v).  Non-temporal: the weights are read once.
  auto wbase = [&](int c, int g) {
    return ((uint32_t)g * 16u + (uint32_t)(j & 7)) * row_bytes + 64u * C * (uint32_t)c + 64u * (uint32_t)(j >> 3) +
           16u * (uint32_t)q;
  };
  auto woff = [&](int v) { return 8u * row_bytes * (uint32_t)(v & 1) + 64u * (uint32_t)(v & ~1); };
  auto wload = [&](uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b128(wc, off, 0, 2); };
  // Loads 2u (a) and 2u + 1 (b) -> the B operand layout of lines 2u and
  // 2u + 1 (lane j + 16q: row j, bytes 16q .. 16q+15 of the line).  Rows 0-7
  // of line 2u already sit in a's lanes j < 8, rows 8-15 of line 2u + 1 in b's
  // lanes j >= 8; the other halves move by 8 lanes within each 16-lane row:
  // line 2u takes b's lanes j - 8 into lanes j >= 8 (row_shr:8, banks 2-3),
  // line 2u + 1 takes a's lanes j + 8 into lanes j < 8 (row_shl:8, banks 0-1).
  auto transpose_pair = [](const u4_t& a, const u4_t& b, u4_t& l0, u4_t& l1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      l0[i] = (uint32_t)__builtin_amdgcn_update_dpp((int)a[i], (int)b[i], 0x118, 0xF, 0xC, false);
      l1[i] = (uint32_t)__builtin_amdgcn_update_dpp((int)b[i], (int)a[i], 0x108, 0xF, 0x3, false);
    }
  };

  // ---- set-up: scales of the first block, the first activation chunk, the
  // first D lines.  Buffer->LDS loads are waited for explicitly, by counting
  // the loads issued after them (vmcnt is in order); the issue order below
  // and in the loop is what the counts assume. ----
  if (Gw > 0) s_issue(0, g0, 0);
  a_issue(0);
  __builtin_amdgcn_sched_barrier(0);
  u4_t ring[D];
  const uint32_t first = Gw > 0 ? wbase(0, g0) : kOOB;
#pragma unroll
  for (int t = 0; t < D; ++t) {
    ring[t] = wload(first + woff(t));
    __builtin_amdgcn_sched_barrier(0);
  }
  wait_vm<D>();  // this wave's copies of the first scales and activation chunk have landed
  barrier_lds();
  a_store();
  barrier_lds();
  if (NC > 1) a_issue(1);
  __builtin_amdgcn_sched_barrier(0);

  f4_t acc[kMaxG];
#pragma unroll
  for (int s = 0; s < kMaxG; ++s) acc[s] = f4_t{0.f, 0.f, 0.f, 0.f};

  const uint8_t* const a_lane = a_lds + (uint32_t)j * a_row_bytes<C>() + 64u * (uint32_t)q;
  int sl = 0;
  for (int c = 0; c < NC; ++c) {
    if (c > 0) {
      // This wave's copies of chunk c were issued before the line loads of
      // its blocks of chunk c - 1 (at least C of them when it has any).
      __builtin_amdgcn_sched_barrier(0);
      if (Gw > 0) wait_vm<C>();
      else wait_vm<0>();
      barrier_lds();  // every wave is done with chunk c - 1; chunk c is staged
      a_store();
      barrier_lds();  // chunk c is in the A region; the staging area is free
      if (c + 1 < NC) a_issue(c + 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    for (int gi = 0; gi < Gw; ++gi) {
      // This block's scales were requested before the C line loads of the
      // previous block (in the set-up: before at least C other loads).
      __builtin_amdgcn_sched_barrier(0);
      wait_vm<C>();
      __builtin_amdgcn_sched_barrier(0);
      const bool last_g = gi + 1 == Gw;
      const bool has_next = !last_g || c + 1 < NC;
      const int nc = last_g ? c + 1 : c, ng = last_g ? g0 : g0 + gi + 1;
      if (has_next) s_issue(nc, ng, sl ^ 1);
      __builtin_amdgcn_sched_barrier(0);
      const uint32_t cb = wbase(c, g0 + gi);
      const uint32_t nb = has_next ? wbase(nc, ng) : kOOB;
      const uint8_t* sslot = slots + (uint32_t)sl * scale_slot_bytes<C>() + 8u * C * (uint32_t)j + 2u * (uint32_t)q;
      f4_t a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < C; t += 2) {
        u4_t lines[2];
        transpose_pair(ring[t % D], ring[(t + 1) % D], lines[0], lines[1]);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          h8_t av[4];
#pragma unroll
          for (int pc = 0; pc < 4; ++pc)
            av[pc] = *reinterpret_cast<const h8_t*>(a_lane + 256u * (t + h) + 16u * pc);
          const h2_t sw = e4m3x2_to_h2(*reinterpret_cast<const uint16_t*>(sslot + 8u * (t + h)));
#pragma unroll
          for (int pc = 0; pc < 4; ++pc) {
            const h8_t bv = dequant8(lines[h][pc], pc < 2 ? sw.x : sw.y);
            if (pc & 1) a1 = mfma16x16x32(av[pc], bv, a1);
            else a0 = mfma16x16x32(av[pc], bv, a0);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int v = t + h + D;
          ring[(t + h) % D] = wload(v < C ? cb + woff(v) : nb + woff(v - C));
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      const f4_t v = a0 + a1;
#pragma unroll
      for (int s = 0; s < kMaxG; ++s)
        if (s == gi) acc[s] += v;
      sl ^= 1;
    }
  }

  // ---- epilogue: D[i][j] of group g sits in lane j + 16(i/4), element i%4:
  // activation row m = 4q + e, weight row n = 16g + j ----
  const float gscale = (*p.ga) * (*p.gw);
  uint64_t best[4] = {0, 0, 0, 0};
#pragma unroll
  for (int s = 0; s < kMaxG; ++s) {
    if (s >= Gw) break;
    const uint32_t n = (uint32_t)(g0 + s) * 16u + (uint32_t)j;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = 4 * q + e;
      if (n < (uint32_t)N && m < M) {
        const float val = acc[s][e] * gscale;
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
    // rows 4q .. 4q+3 are shared by the 16 lanes of a quarter; the maximum
    // key does not depend on the order in which waves merge theirs.  Slot
    // kKeySlots - 1 takes no key: its first word is the arrival counter of
    // the fused tree acceptance.
    const uint32_t slot = (uint32_t)w % (kKeySlots - 1);
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

  if (p.tree_result) {
    // ---- fused tree acceptance, in the last workgroup to finish.  Ordering
    // as for a split-K ticket: every thread waits for its key maxima to
    // complete; after the barrier the ticket's thread issues an agent-scope
    // release fence, so every key of this workgroup happens before its
    // ticket; the last workgroup takes an agent-scope acquire fence before
    // it reads the keys, with agent-scope loads. ----
    static_assert(kKeySlots * 16 == 2 * kThreads, "two key words per thread");
    __shared__ uint32_t ticket;
    uint64_t* const keys = p.argmax_keys;
    __builtin_amdgcn_s_waitcnt(0);  // this thread's key maxima have completed
    __syncthreads();
    if (threadIdx.x == 0) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      uint32_t* const cnt = reinterpret_cast<uint32_t*>(keys + (kKeySlots - 1) * 16);
      const uint32_t t = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (t == gridDim.x - 1) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      ticket = t;
    }
    __syncthreads();
    if (ticket != gridDim.x - 1) return;
    // Lane v < M of wave 0: node v's parent and draft token (requested
    // before the fold, which they overlap).
    const uint32_t t = threadIdx.x;
    int32_t par = -1, dr = 0;
    if (t < (uint32_t)M) {
      par = p.tree_parent[t];
      dr = p.tree_draft[t];
    }
    // Thread t holds words t and t + 512 (row t % 16 of slots t / 16 and
    // t / 16 + 32; slot kKeySlots - 1 is the counter) and resets both to
    // zero, the counter with them; rows fold over the slots in LDS (the
    // activation region, which no wave reads any more).
    uint64_t* const kb = reinterpret_cast<uint64_t*>(lds_s);
    const uint64_t k0 = __hip_atomic_load(keys + t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t k1 = t + kThreads < (uint32_t)(kKeySlots - 1) * 16u
                            ? __hip_atomic_load(keys + t + kThreads, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                            : 0ull;
    __hip_atomic_store(keys + t, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(keys + t + kThreads, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    kb[t] = k0 > k1 ? k0 : k1;
    __syncthreads();
    for (uint32_t half = kKeySlots / 4; half >= 1; half >>= 1) {
      if (t < half * 16u) kb[t] = kb[t] > kb[t + half * 16u] ? kb[t] : kb[t + half * 16u];
      __syncthreads();
    }
    if (t >= 64) return;  // no barrier follows
    const int32_t gv = t < (uint32_t)M ? (int32_t)(0xFFFFFFFFu - (uint32_t)kb[t]) : 0;
    if (t < (uint32_t)M) p.tree_greedy[t] = gv;
    tree_walk_wave(M, par, dr, gv, p.tree_result);
  }
}

int stream_chunk_lines(int K) {
  if (K % kLine != 0) return 0;
  const int L = K / kLine;
  for (int C : {20, 16, 12, 8})
    if (L % C == 0) return C;
  return 0;
}

int device_cus_stream() {
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

// One workgroup per CU while that gives every wave at most kMaxG groups;
// more workgroups (queued behind the first ones) for taller matrices.
int64_t stream_grid(const GemmArgs& a) {
  const int64_t NG = ((int64_t)a.N + 15) / 16;
  const int64_t need = (NG + (int64_t)kWaves * kMaxG - 1) / ((int64_t)kWaves * kMaxG);
  const int64_t cus = device_cus_stream();
  return need > cus ? need : cus;
}

template <int C, int D, bool OUT_BF16>
hipError_t launch_stream(const GemmArgs& a, hipStream_t stream) {
  auto kern = &gemm_m16_stream_kernel<C, D, OUT_BF16>;
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     (int)stream_lds_bytes<C>());
  if (attr != hipSuccess) return attr;
  const int NG = (int)(((int64_t)a.N + 15) / 16);
  kern<<<dim3((unsigned)stream_grid(a)), kThreads, stream_lds_bytes<C>(), stream>>>(a, NG);
  return hipGetLastError();
}

template <bool OUT_BF16>
hipError_t launch_stream_c(const GemmArgs& a, hipStream_t stream) {
  switch (stream_chunk_lines(a.K)) {
    case 20: return launch_stream<20, 10, OUT_BF16>(a, stream);
    case 16: return launch_stream<16, 8, OUT_BF16>(a, stream);
    case 12: return launch_stream<12, 6, OUT_BF16>(a, stream);
    default: return launch_stream<8, 8, OUT_BF16>(a, stream);
  }
}

}  // namespace

// 1 <= M <= 16; K a multiple of 1024 or of 128 x (20, 16 or 12); 32-bit
// buffer offsets over the weight codes.
bool gemm_m16_stream_supported(const GemmArgs& a) {
  return a.M >= 1 && a.M <= 16 && a.N >= 1 && stream_chunk_lines(a.K) > 0 &&
         (int64_t)a.N * (a.K / 2) < ((int64_t)1 << 31);
}

// Tall matrices: from 10 groups of 16 rows per CU on (measured on MI355X at
// M = 16, K = 5120, against the M-tile kernel: N = 32768 20.4 vs 20.2 us,
// 40960 29.7 vs 31.7, 49152 30.6 vs 33.1, 65536 34.8 vs 36.5, 151936 79.6
// vs 90.5; at K = 2560, N = 65536 19.3 vs 20.4).
bool gemm_m16_stream_preferred(const GemmArgs& a) {
  return gemm_m16_stream_supported(a) && a.M >= 3 &&
         ((int64_t)a.N + 15) / 16 >= (int64_t)10 * device_cus_stream();
}

hipError_t launch_gemm_m16_stream(const GemmArgs& a, hipStream_t stream) {
  return a.out_bf16 ? launch_stream_c<true>(a, stream) : launch_stream_c<false>(a, stream);
}

}  // namespace nvfp4
