// GEMV for one or two activation rows on the FP4 matrix cores of gfx950.
//
// Decode multiplies an NVFP4 weight matrix by one activation row (two for a
// batch of two), so the kernel must stream the weights at HBM speed with as
// little arithmetic per byte as possible; the page "TensorRT Edge-LLM
// Completes the MLPerf Edge Agentic Benchmark 6.4x Faster on Jetson AGX Thor"
// (section "Using NVFP4 quantization to accelerate Qwen3.6-27B inference")
// gives the bandwidth bound of low-batch decode as the reason for NVFP4.
//
// Each weight byte goes from the load straight into the E2M1 operand of
// v_mfma_scale_f32_16x16x128_f8f6f4 with unit (E8M0 = 1) block scales, so no
// weight is converted on the vector ALU.  The hardware's block scales are
// powers of two over 32 elements and cannot carry NVFP4's E4M3 scales over
// 16 elements; instead every MFMA output is made the exact partial dot
// product of one (weight row, 16-block) pair, and the E4M3 scales are applied
// to those partials in fp32:
//
//   B operand (weights): column j = weight row j/2, half c = j%2 of a
//     256-element line; lane j + 16g holds bytes 64c + 16g .. +15 of that row's
//     128-byte line, so one load instruction covers 8 rows x 128 bytes.
//   A operand (activations, block-diagonal): row i holds activation block i
//     of the line (16 values) at MFMA k-positions 32((i%8)/2) + 16(i%2) .. +15
//     and zeros elsewhere.
//   D[i][j] = sum over those 16 positions = (row j/2, block i) partial when
//     i/8 == j%2 (the k-positions of row i then meet the weights of block i);
//     the other half of D are unused cross terms.
//
// With D[i][j] in lane j + 16(i/4), element i%4, lane L (j = L%16, q = L/16)
// is active when q/2 == j%2 and then holds the partials of row j/2, blocks
// 4q .. 4q+3: one dword of weight scales and four consecutive activation
// scales.  E2M1 products and their 16-term sums are exact in fp32, the scale
// product s_w * s_a of two E4M3 values is exact, so each partial is rounded
// once when scaled and once when accumulated.  Row sums are reduced over the
// four active lanes of a row in a fixed butterfly order: results do not
// depend on timing.
#include "device_common.h"
#include "launch.h"

namespace nvfp4 {
namespace {

typedef int v8i_t __attribute__((ext_vector_type(8)));

constexpr uint32_t kOOB = 0x80000000u;  // buffer offset past any array: loads read zeros
constexpr int kWaves = 4;               // waves per workgroup
constexpr int kScaleLoads = 8;          // 16-byte weight-scale loads per lane (<= 8 KiB per wave)

// 16x16x128 E2M1 x E2M1 product with unit block scales (E8M0 127 = 2^0).
__device__ __forceinline__ f4_t mfma_e2m1(const u4_t& a, const u4_t& b) {
  const v8i_t A = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  const v8i_t B = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, f4_t{0.f, 0.f, 0.f, 0.f}, 4, 4, 0, 127, 0,
                                                          127);
}

// LDS bytes of one workgroup: the activation operands of every line, the
// activation scales as fp32, then per wave its weight scales and row sums.
size_t fp4_lds_bytes(int MR, int K, int G) {
  return (size_t)MR * (K / 256) * 1024 + (size_t)MR * (K / 16) * 4 +
         (size_t)kWaves * ((size_t)G * K / 2 + (size_t)G * 8 * MR * 4);
}

// Wave w of the W in the grid owns the contiguous run of groups of 8
// consecutive weight rows [floor(w NG / W), floor((w + 1) NG / W)) (NG =
// ceil(N / 8); rows past N read zeros and are not stored): the longer runs are
// spread evenly over the grid, so every CU gets the same share; with no more
// groups than waves, group w.  W NG < 2^32 (N <= 2^18), so 32-bit arithmetic
// is exact.  G bounds the run length and sizes the per-wave LDS areas.  K = 256 L is a template parameter: the L lines of a
// group are unrolled, so every load, LDS and scale offset is an immediate and
// a line costs one weight load, three LDS reads, one MFMA per activation row
// and the scale arithmetic.  D weight loads are in flight per wave (D divides
// L, so ring slots are static across groups).
//
// FUSE = 0 reads pre-quantized activation codes and scales; FUSE = 1 (bf16)
// or 2 (fp32) reads the raw activation rows and quantizes their 16-blocks in
// the set-up (quantize_block16, bit-identical to the activation quantizer),
// every workgroup for itself; workgroup 0 also stores the codes and scales.
// With p.ga_dynamic set, the tensor scale is computed there too: the largest
// magnitude over the raw rows (each workgroup holds all of them), reduced
// across the workgroup, g_a = fl32(amax / 2688), as the standalone scale
// kernel computes it.
template <int MR, int L, int D, bool OUT_BF16, int FUSE>
__global__ __launch_bounds__(256) void gemv_fp4_kernel(GemmArgs p, int G, uint32_t NG) {
  static_assert(L % D == 0 && D <= L, "ring depth must divide the line count");
  constexpr int K = 256 * L;
  constexpr uint32_t row_bytes = 128u * L;
  constexpr uint32_t srow = 16u * L;
  constexpr int kFillPerThread = (MR * L + kWaves - 1) / kWaves;
  extern __shared__ __attribute__((aligned(16))) u4_t lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int N = p.N;
  const uint32_t wsc_bytes = (uint32_t)G * 8u * srow;  // per-wave LDS area for G groups
  u4_t* tiles = lds;                                                      // [MR][L][64]
  float* asc = reinterpret_cast<float*>(tiles + MR * L * 64);             // [MR][K/16]
  uint8_t* wsc_all = reinterpret_cast<uint8_t*>(asc + MR * (K >> 4));
  uint8_t* wsc = wsc_all + wave * wsc_bytes;                              // [8G][K/16]
  float* slots = reinterpret_cast<float*>(wsc_all + kWaves * wsc_bytes) + wave * (G * 8 * MR);

  const uint32_t W = gridDim.x * (uint32_t)kWaves, wv = blockIdx.x * (uint32_t)kWaves + (uint32_t)wave;
  int g0w, Gw;  // Gw <= G
  if (NG <= W) {  // at most one group per wave: no division
    g0w = (int)wv;
    Gw = wv < NG ? 1 : 0;
  } else {
    g0w = (int)(wv * NG / W);
    Gw = (int)((wv + 1u) * NG / W) - g0w;
  }
  const uint32_t wsc_need = (uint32_t)Gw * 8u * srow;
  const uint32_t row0 = (uint32_t)g0w * 8u;

  const __amdgpu_buffer_rsrc_t ac = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.ac), (short)0, (int)(MR * row_bytes), 0x00020000);
  const __amdgpu_buffer_rsrc_t as = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.as), (short)0, (int)(MR * srow), 0x00020000);
  const __amdgpu_buffer_rsrc_t wc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.wc), (short)0, (int)((uint32_t)N * row_bytes), 0x00020000);
  const __amdgpu_buffer_rsrc_t ws = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.ws), (short)0, (int)((uint32_t)N * srow), 0x00020000);

  // ---- loads of the set-up, issued before the weight ring ----
  // Activation operand entry (tile tau = m * L + t, lane) for tau = wave + 4s:
  // lane i + 16g of line t carries block i's 8 code bytes when g == (i%8)/2.
  const int ti = lane & 15, tg = lane >> 4;
  const bool nz = tg == ((ti & 7) >> 1);
  constexpr int kFillLoads = FUSE == 0 ? kFillPerThread : 1;
  u2_t fa[kFillLoads];
  uint32_t asb = 0;
  const uint32_t a_dw = (uint32_t)threadIdx.x;  // activation scales, 4 bytes per thread
  // Fused: 16-blocks tid, tid + 256, ... of the raw rows, 16-byte pieces.
  constexpr int kRawBlocks = MR * L * 16;
  constexpr int kRawPerThread = (kRawBlocks + 255) / 256;
  constexpr int kRawVec = FUSE == 2 ? 4 : 2;  // 16-byte loads per block (fp32 : bf16)
  u4_t xr[FUSE == 0 ? 1 : kRawPerThread][kRawVec];
  [[maybe_unused]] float ga_used = 0.0f;  // fused: the tensor scale the rows were quantized with
  if constexpr (FUSE == 0) {
#pragma unroll
    for (int s = 0; s < kFillPerThread; ++s) {
      const int tau = wave + kWaves * s;
      const int m = tau >= L ? 1 : 0;
      const int t = tau - m * L;
      const bool ok = nz && tau < MR * L;
      fa[s] = __builtin_amdgcn_raw_buffer_load_b64(ac, ok ? m * row_bytes + (16u * t + ti) * 8u : kOOB, 0, 0);
    }
    asb = __builtin_amdgcn_raw_buffer_load_b32(as, a_dw * 4u < MR * srow ? a_dw * 4u : kOOB, 0, 0);
  } else {
    const __amdgpu_buffer_rsrc_t ar = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(p.a_raw), (short)0, (int)(kRawBlocks * 16 * kRawVec), 0x00020000);
#pragma unroll
    for (int s = 0; s < kRawPerThread; ++s) {
      const uint32_t b = threadIdx.x + 256u * s;
#pragma unroll
      for (int v = 0; v < kRawVec; ++v)
        xr[s][v] = __builtin_amdgcn_raw_buffer_load_b128(ar, b < (uint32_t)kRawBlocks ? (b * kRawVec + v) * 16u : kOOB,
                                                          0, 0);
    }
  }
  // This wave's weight scales: rows row0 .. row0 + 8Gw - 1, contiguous.
  u4_t sreg[kScaleLoads];
#pragma unroll
  for (int s = 0; s < kScaleLoads; ++s) {
    const uint32_t rel = 1024u * s + 16u * lane;
    const uint32_t off = row0 * srow + rel;
    sreg[s] = __builtin_amdgcn_raw_buffer_load_b128(ws, rel < wsc_need && off < (uint32_t)N * srow ? off : kOOB,
                                                     0, 2);
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- weight ring: instruction (group g, line t) of lane j + 16q reads
  // row 8g + j/2, bytes 128t + 64(j%2) + 16q of the row ----
  const int j = lane & 15, q = lane >> 4;
  const bool active = (q >> 1) == (j & 1);
  const uint32_t b_lane = (uint32_t)(j >> 1) * row_bytes + 64u * (j & 1) + 16u * q;
  auto wload = [&](uint32_t vo, int t) {
    return __builtin_amdgcn_raw_buffer_load_b128(wc, vo + 128u * t, 0, 2);
  };
  const uint32_t vo_first = Gw > 0 ? b_lane + row0 * row_bytes : kOOB;
  u4_t ring[D];
#pragma unroll
  for (int t = 0; t < D; ++t) {
    ring[t] = wload(vo_first, t);
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- set-up stores (wait for the set-up loads only) ----
  if constexpr (FUSE == 0) {
#pragma unroll
    for (int s = 0; s < kFillPerThread; ++s) {
      const int tau = wave + kWaves * s;
      if (tau < MR * L)
        tiles[tau * 64 + lane] = (ti & 1) ? u4_t{0u, 0u, fa[s].x, fa[s].y} : u4_t{fa[s].x, fa[s].y, 0u, 0u};
    }
    if (a_dw * 4u < MR * srow) {
      const f2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8(asb, false);
      const f2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8(asb, true);
      *reinterpret_cast<f4_t*>(asc + 4 * a_dw) = f4_t{lo.x, lo.y, hi.x, hi.y};
    }
  } else {
    // raw value e (0..15) of this thread's block s, as fp32
    // (The vector element is copied to a scalar before the bit cast: a bit
    // cast applied to the element expression itself compiled to a read of
    // the vector's first element.)
    auto raw = [&](int s, int e) {
      if constexpr (FUSE == 2) {
        const uint32_t w = xr[s][e >> 2][e & 3];
        return __builtin_bit_cast(float, w);
      } else {  // two bf16 per word: element 2c in the low half
        const uint32_t w = xr[s][e >> 3][(e >> 1) & 3];
        return __builtin_bit_cast(float, (e & 1) ? (w & 0xFFFF0000u) : (w << 16));
      }
    };
    float ga;
    if (p.ga_dynamic != nullptr) {
      // blocks past the rows were loaded as zeros
      float m = 0.0f;
#pragma unroll
      for (int s = 0; s < kRawPerThread; ++s)
#pragma unroll
        for (int e = 0; e < 16; ++e) m = __builtin_fmaxf(m, __builtin_fabsf(raw(s, e)));
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) m = __builtin_fmaxf(m, __shfl_xor(m, off));
      __shared__ float wave_max[kWaves];
      if (lane == 0) wave_max[wave] = m;
      // workgroup barrier for this LDS exchange only: the weight loads stay in flight
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));  // lgkmcnt(0)
      __builtin_amdgcn_s_barrier();
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      float b = wave_max[0];
#pragma unroll
      for (int i = 1; i < kWaves; ++i) b = __builtin_fmaxf(b, wave_max[i]);
      ga = b / 2688.0f;
      if (blockIdx.x == 0 && threadIdx.x == 0) *p.ga_dynamic = ga;
    } else {
      ga = *p.ga;
    }
    ga_used = ga;
#pragma unroll
    for (int s = 0; s < kRawPerThread; ++s) {
      const uint32_t b = threadIdx.x + 256u * s;
      if (b < (uint32_t)kRawBlocks) {
        float x[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) x[e] = raw(s, e);
        uint32_t w0, w1;
        const uint32_t sb = quantize_block16(x, ga, w0, w1);
        const uint32_t m = b >= 16u * L ? 1u : 0u;
        const uint32_t blk = b - m * 16u * L;  // block within the row
        const uint32_t t = blk >> 4, i = blk & 15;
        u4_t* e = tiles + (m * L + t) * 64 + i;
#pragma unroll
        for (int gg = 0; gg < 4; ++gg)
          e[16 * gg] = gg != (int)((i & 7) >> 1) ? u4_t{0u, 0u, 0u, 0u}
                       : (i & 1)                 ? u4_t{0u, 0u, w0, w1}
                                                 : u4_t{w0, w1, 0u, 0u};
        asc[m * (K >> 4) + blk] = e4m3_to_f32(sb);
        if (blockIdx.x == 0) {
          *reinterpret_cast<u2_t*>(p.ac_out + m * (K >> 1) + blk * 8) = u2_t{w0, w1};
          p.as_out[m * (K >> 4) + blk] = (uint8_t)sb;
        }
      }
    }
  }
#pragma unroll
  for (int s = 0; s < kScaleLoads; ++s) {
    const uint32_t rel = 1024u * s + 16u * lane;
    if (rel < wsc_need) *reinterpret_cast<u4_t*>(wsc + rel) = sreg[s];
  }
  __syncthreads();

  // ---- main loop ----
  // Within a group, step t issues the MFMA of line t, reads the LDS operands
  // of line t + 1 and scales the partials of line t - 1, so neither the LDS
  // nor the MFMA latency sits between dependent instructions.
  float acc[MR][4];
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[m][e] = 0.f;

  struct Ops {
    u4_t a[MR];    // activation operand of the line
    uint32_t sw;   // weight scales of blocks 4q .. 4q+3 of this lane's row
    f4_t sa[MR];   // activation scales of the same blocks
  };
  const u4_t* tiles_lane = tiles + lane;
  const float* asc_lane = asc + 4 * q;
  auto read_ops = [&](const uint8_t* wsc_g, int t) {
    Ops o;
#pragma unroll
    for (int m = 0; m < MR; ++m) o.a[m] = tiles_lane[(m * L + t) * 64];
    o.sw = *reinterpret_cast<const uint32_t*>(wsc_g + 16 * t);
#pragma unroll
    for (int m = 0; m < MR; ++m) o.sa[m] = *reinterpret_cast<const f4_t*>(asc_lane + m * (K >> 4) + 16 * t);
    return o;
  };
  auto apply = [&](const f4_t* d, const Ops& o) {
    const f2_t w01 = __builtin_amdgcn_cvt_pk_f32_fp8(o.sw, false);
    const f2_t w23 = __builtin_amdgcn_cvt_pk_f32_fp8(o.sw, true);
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      acc[m][0] = __builtin_fmaf(d[m].x, w01.x * o.sa[m].x, acc[m][0]);
      acc[m][1] = __builtin_fmaf(d[m].y, w01.y * o.sa[m].y, acc[m][1]);
      acc[m][2] = __builtin_fmaf(d[m].z, w23.x * o.sa[m].z, acc[m][2]);
      acc[m][3] = __builtin_fmaf(d[m].w, w23.y * o.sa[m].w, acc[m][3]);
    }
  };

  const uint8_t* wsc_lane = wsc + (uint32_t)(j >> 1) * srow + 4u * q;
  for (int g = 0; g < Gw; ++g) {
    const uint32_t vo_c = b_lane + (row0 + 8u * g) * row_bytes;
    const uint32_t vo_n = g + 1 < Gw ? vo_c + 8u * row_bytes : kOOB;
    const uint8_t* wsc_g = wsc_lane + 8u * srow * g;
    Ops cur = read_ops(wsc_g, 0), prev;
    f4_t dprev[MR];
#pragma unroll
    for (int t = 0; t < L; ++t) {
      f4_t d[MR];
#pragma unroll
      for (int m = 0; m < MR; ++m) d[m] = mfma_e2m1(cur.a[m], ring[t % D]);
      Ops nxt;
      if (t + 1 < L) nxt = read_ops(wsc_g, t + 1);
      if (t > 0) apply(dprev, prev);
#pragma unroll
      for (int m = 0; m < MR; ++m) dprev[m] = d[m];
      prev = cur;
      if (t + 1 < L) cur = nxt;
      __builtin_amdgcn_sched_barrier(0);
      ring[t % D] = t + D < L ? wload(vo_c, t + D) : wload(vo_n, t + D - L);
      __builtin_amdgcn_sched_barrier(0);
    }
    apply(dprev, prev);
    // Row j/2 of this group: its four active lanes (j even with q = 0, 1;
    // j odd with q = 2, 3) hold blocks 0-3, 4-7, 8-11, 12-15 of every line.
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      float s = (acc[m][0] + acc[m][1]) + (acc[m][2] + acc[m][3]);
      s = active ? s : 0.f;
      s += __shfl_xor(s, 1);
      s += __shfl_xor(s, 16);
      s += __shfl_xor(s, 32);
      if (lane < 16 && (lane & 1) == 0) slots[(8 * g + (lane >> 1)) * MR + m] = s;
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[m][e] = 0.f;
    }
  }

  // ---- epilogue: same-wave LDS ops are ordered ----
  const float gscale = (FUSE == 0 ? *p.ga : ga_used) * (*p.gw);
  for (int idx = lane; idx < Gw * 8 * MR; idx += 64) {
    const uint32_t n = row0 + (uint32_t)(idx / MR);
    const int m = idx % MR;
    if (n < (uint32_t)N) {
      const float v = slots[idx] * gscale;
      const int64_t o = (int64_t)m * N + n;
      if constexpr (OUT_BF16) {
        reinterpret_cast<uint16_t*>(p.out)[o] = f32_to_bf16_rne(v);
      } else {
        reinterpret_cast<float*>(p.out)[o] = v;
      }
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

template <int MR, int L, int D, int FUSE>
hipError_t launch_fp4(const GemmArgs& a, int G, int64_t W, hipStream_t stream) {
  const dim3 grid((unsigned)(W / kWaves));
  const uint32_t NG = (uint32_t)(((int64_t)a.N + 7) / 8);
  const size_t lds = fp4_lds_bytes(MR, a.K, G);
  if (a.out_bf16) gemv_fp4_kernel<MR, L, D, true, FUSE><<<grid, 64 * kWaves, lds, stream>>>(a, G, NG);
  else gemv_fp4_kernel<MR, L, D, false, FUSE><<<grid, 64 * kWaves, lds, stream>>>(a, G, NG);
  return hipGetLastError();
}

template <int MR, int L, int D>
hipError_t launch_fp4(const GemmArgs& a, int G, int64_t W, hipStream_t stream) {
  if (!a.a_raw) return launch_fp4<MR, L, D, 0>(a, G, W, stream);
  return a.a_raw_bf16 ? launch_fp4<MR, L, D, 1>(a, G, W, stream) : launch_fp4<MR, L, D, 2>(a, G, W, stream);
}

template <int MR>
hipError_t launch_fp4_k(const GemmArgs& a, int G, int64_t W, hipStream_t stream) {
  switch (a.K / 256) {  // ring depth: a divisor of L near 8
    case 4: return launch_fp4<MR, 4, 4>(a, G, W, stream);
    case 8: return launch_fp4<MR, 8, 8>(a, G, W, stream);
    case 12: return launch_fp4<MR, 12, 6>(a, G, W, stream);
    case 16: return launch_fp4<MR, 16, 8>(a, G, W, stream);
    case 20: return launch_fp4<MR, 20, 10>(a, G, W, stream);
    case 24: return launch_fp4<MR, 24, 8>(a, G, W, stream);
    case 28: return launch_fp4<MR, 28, 7>(a, G, W, stream);
    default: return launch_fp4<MR, 32, 8>(a, G, W, stream);
  }
}

}  // namespace

bool gemv_fp4_supported(const GemmArgs& a) {
  if (a.M < 1 || a.M > 2 || a.K % 1024 != 0 || a.K < 1024 || a.K > 8192) return false;
  // the grid's wave count (at most the group count) times the group count
  // stays below 2^32 (the kernel's 32-bit run arithmetic): N <= 2^18, so at
  // most 2^15 groups of 8 rows
  if ((int64_t)a.N > ((int64_t)1 << 18)) return false;
  return fp4_lds_bytes(a.M, a.K, 1) <= 64 * 1024;
}

// Grid: two workgroups of four waves per CU, the groups of 8 rows dealt out
// to the waves in contiguous runs of equal length +-1, so that every CU
// streams the same share (measured on MI355X at decode_up, 1 x 5120 x 25600:
// 13.18-13.35 us against 13.44-13.49 us for about six waves per CU with two
// groups each, where 144 CUs held two workgroups and 112 one; three
// workgroups per CU 14.8 us, one of eight waves 14.0 us).  Fewer rows: one
// group per wave, as many waves as groups.  More rows than the per-wave
// scale staging and LDS allow: the wave count doubles until they fit.
hipError_t launch_gemv_fp4(const GemmArgs& a, hipStream_t stream) {
  const int64_t NG = ((int64_t)a.N + 7) / 8;
  int64_t W = (int64_t)device_cus() * 2 * kWaves;
  if (NG < W) W = (NG + kWaves - 1) / kWaves * kWaves;
  int G = (int)((NG + W - 1) / W);
  while (G > 1 && ((int64_t)G * a.K / 2 > kScaleLoads * 1024 || fp4_lds_bytes(a.M, a.K, G) > 64 * 1024)) {
    W *= 2;
    G = (int)((NG + W - 1) / W);
  }
  return a.M == 1 ? launch_fp4_k<1>(a, G, W, stream) : launch_fp4_k<2>(a, G, W, stream);
}

}  // namespace nvfp4
