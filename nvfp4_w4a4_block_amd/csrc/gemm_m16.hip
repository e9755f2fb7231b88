// Weight-streaming GEMM for 3 to 16 activation rows: the verification pass of
// a 16-node candidate tree and the language-model head over it (page
// "TensorRT Edge-LLM Completes the MLPerf Edge Agentic Benchmark 6.4x Faster
// on Jetson AGX Thor", sections "Using tree-based multi-token prediction to
// accelerate LLM inference" and "Using NVFP4 quantization to accelerate
// Qwen3.6-27B inference").  At these sizes the product still reads every
// weight once and little else, so the kernel is built like the FP4 GEMV:
//
//   - one 16-byte load per lane covers 8 weight rows x 128 bytes (a 256-element
//     line of each): lane j + 16q holds bytes 64(j%2) + 16q .. +15 of row j/2;
//   - the codes are dequantized exactly to f16 with their E4M3 scale (E2M1 x
//     E4M3 has at most 6 significant bits and lies in [2^-10, 2688]) and are
//     the B operand of v_mfma_f32_16x16x32_f16: column j = (row j/2, half j%2);
//   - the A operand is the 16 activation rows (rows past M read zeros), staged
//     once per workgroup in LDS as codes and scales and dequantized exactly to
//     f16 the same way, line by line; lane i + 16q of the MFMA for piece p and
//     half h holds k = 128h + 32q + 8p .. +7 of activation row i.  Columns of
//     half h meet their own k there, so the MFMA of half h is kept for the
//     columns j with j%2 == h (the other columns are unused cross terms);
//     every product is exact and the fp32 accumulation is the only rounding.
//
// Each wave walks its K range line by line (three lines of weight loads in
// flight) and, per line, dequantizes the activation operand once for G groups
// of 8 rows.  K may be split over the KS (<= 8) waves of a workgroup, whose
// partial sums are added through LDS in a fixed order (results do not depend
// on timing); nothing is written outside the output.  The staged activations
// bound K (about 5K); longer K is served by the other skinny kernels.
#include "device_common.h"
#include "launch.h"

namespace nvfp4 {
namespace {

constexpr uint32_t kOOB = 0x80000000u;  // buffer offset past any array: loads read zeros
constexpr int kFillMax = 16;            // staged-activation pieces per thread (checked on the host)

template <int G>
struct Line {
  u4_t w[G];       // weight codes of each row group
  uint32_t ws[G];  // their two E4M3 scale bytes
};

// LDS layout of the staged activations: 16 rows of codes, then 16
// rows of scales, each row padded by 16 bytes so that the 16 rows read by one
// quarter-wave fall in different banks.
__host__ __device__ constexpr uint32_t alds_code_stride(int K) { return (uint32_t)K / 2 + 16u; }
__host__ __device__ constexpr uint32_t alds_scale_stride(int K) { return (uint32_t)K / 16 + 16u; }
__host__ __device__ constexpr uint32_t alds_bytes_m16(int K) { return 16u * (alds_code_stride(K) + alds_scale_stride(K)); }

template <int G, bool OUT_BF16>
__global__ __launch_bounds__(512) void gemm_m16_kernel(GemmArgs p, int KS, int LW) {
  // LDS: the staged activation codes and scales, then the partial sums
  // [waves][G][8 rows][16 activation rows].
  extern __shared__ __attribute__((aligned(16))) uint8_t lds_m16[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = blockDim.x >> 6;
  const int rb = wave / KS, kc = wave - rb * KS;
  const int M = p.M, K = p.K, N = p.N;
  const uint32_t row_bytes = (uint32_t)K >> 1, srow = (uint32_t)K >> 4;
  const int L = K >> 8;
  const uint32_t row0 = (uint32_t)(blockIdx.x * (nw / KS) + rb) * 8u * G;
  const int t0 = kc * LW;
  const int t1 = t0 + LW < L ? t0 + LW : L;

  const __amdgpu_buffer_rsrc_t ac = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.ac), (short)0, (int)((uint32_t)M * row_bytes), 0x00020000);
  const __amdgpu_buffer_rsrc_t as = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.as), (short)0, (int)((uint32_t)M * srow), 0x00020000);
  const __amdgpu_buffer_rsrc_t wc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.wc), (short)0, (int)((uint32_t)N * row_bytes), 0x00020000);
  const __amdgpu_buffer_rsrc_t ws = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.ws), (short)0, (int)((uint32_t)N * srow), 0x00020000);

  float* part = reinterpret_cast<float*>(lds_m16 + alds_bytes_m16(K));
  const int j = lane & 15, q = lane >> 4;
  // Staged activations: 16-byte pieces, codes of rows 0..15 then their
  // scales (rows past M as zeros).  All pieces of a thread are loaded before
  // any is stored, and the first weight lines are requested in between.
  const uint32_t cs = alds_code_stride(K), ss = alds_scale_stride(K);
  const uint32_t cpr = row_bytes / 16u, spr = srow / 16u;  // pieces per row
  const uint32_t cpieces = 16u * cpr, pieces = cpieces + 16u * spr;
  u4_t fv[kFillMax];
  {
#pragma unroll
    for (int s = 0; s < kFillMax; ++s) {
      const uint32_t pc = threadIdx.x + blockDim.x * s;
      const bool code = pc < cpieces;
      const uint32_t pp = code ? pc : pc - cpieces;
      const uint32_t r = code ? pp / cpr : pp / spr;
      const uint32_t c = code ? pp - r * cpr : pp - r * spr;
      const bool ok = pc < pieces && r < (uint32_t)M;
      fv[s] = code ? __builtin_amdgcn_raw_buffer_load_b128(ac, ok ? r * row_bytes + 16u * c : kOOB, 0, 0)
                   : __builtin_amdgcn_raw_buffer_load_b128(as, ok ? r * srow + 16u * c : kOOB, 0, 0);
    }
  }
  auto fill_store = [&]() {
    {
#pragma unroll
      for (int s = 0; s < kFillMax; ++s) {
        const uint32_t pc = threadIdx.x + blockDim.x * s;
        if (pc < pieces) {
          const bool code = pc < cpieces;
          const uint32_t pp = code ? pc : pc - cpieces;
          const uint32_t r = code ? pp / cpr : pp / spr;
          const uint32_t c = code ? pp - r * cpr : pp - r * spr;
          *reinterpret_cast<u4_t*>(lds_m16 + (code ? r * cs : 16u * cs + r * ss) + 16u * c) = fv[s];
        }
      }
      __syncthreads();
    }
  };

  // weight row row0 + j/2 (+ 8g), half j%2, elements 32q .. 32q+31 of the half
  const uint32_t w_off = (row0 + (j >> 1)) * row_bytes + 64u * (j & 1) + 16u * q;
  const uint32_t ws_off = (row0 + (j >> 1)) * srow + 8u * (j & 1) + 2u * q;

  auto load = [&](int t) {
    Line<G> d;
    const bool ok = t < t1;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      d.w[g] = __builtin_amdgcn_raw_buffer_load_b128(wc, ok ? w_off + 8u * g * row_bytes + 128u * t : kOOB, 0, 2);
      d.ws[g] = __builtin_amdgcn_raw_buffer_load_b16(ws, ok ? ws_off + 8u * g * srow + 16u * t : kOOB, 0, 2);
    }
    return d;
  };

  f4_t acc[G][2];
#pragma unroll
  for (int g = 0; g < G; ++g) acc[g][0] = acc[g][1] = f4_t{0.f, 0.f, 0.f, 0.f};

  const uint8_t* a_lds = lds_m16 + (uint32_t)j * alds_code_stride(K) + 16u * q;
  const uint8_t* as_lds = lds_m16 + 16u * alds_code_stride(K) + (uint32_t)j * alds_scale_stride(K) + 2u * q;
  auto compute = [&](const Line<G>& d, int t) {
    h8_t av[2][4];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // activation row j, elements 32q .. 32q+31 of half h of line t
      const u4_t a = *reinterpret_cast<const u4_t*>(a_lds + 64u * h + 128u * t);
      const uint32_t sa = *reinterpret_cast<const uint16_t*>(as_lds + 8u * h + 16u * t);
      const h2_t s2 = e4m3x2_to_h2(sa);  // blocks 2q and 2q+1 of the half
#pragma unroll
      for (int pc = 0; pc < 4; ++pc) av[h][pc] = dequant8(a[pc], pc < 2 ? s2.x : s2.y);
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const h2_t s2 = e4m3x2_to_h2(d.ws[g]);
#pragma unroll
      for (int pc = 0; pc < 4; ++pc) {
        const h8_t wv = dequant8(d.w[g][pc], pc < 2 ? s2.x : s2.y);
        acc[g][0] = mfma16x16x32(av[0][pc], wv, acc[g][0]);
        acc[g][1] = mfma16x16x32(av[1][pc], wv, acc[g][1]);
      }
    }
  };

  Line<G> b0 = load(t0);
  __builtin_amdgcn_sched_barrier(0);
  Line<G> b1 = load(t0 + 1);
  __builtin_amdgcn_sched_barrier(0);
  Line<G> b2 = load(t0 + 2);
  __builtin_amdgcn_sched_barrier(0);
  fill_store();
  for (int t = t0; t < t1; t += 3) {
    compute(b0, t);
    __builtin_amdgcn_sched_barrier(0);
    b0 = load(t + 3);
    __builtin_amdgcn_sched_barrier(0);
    if (t + 1 < t1) compute(b1, t + 1);
    __builtin_amdgcn_sched_barrier(0);
    b1 = load(t + 4);
    __builtin_amdgcn_sched_barrier(0);
    if (t + 2 < t1) compute(b2, t + 2);
    __builtin_amdgcn_sched_barrier(0);
    b2 = load(t + 5);
    __builtin_amdgcn_sched_barrier(0);
  }

  // D[i][j] of half h sits in lane j + 16(i/4), element i%4: keep the half of
  // this lane's column, add the two halves of a row, park [g][row][i] in LDS.
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const bool odd = (j & 1) != 0;
    f4_t v;
    v.x = odd ? acc[g][1].x : acc[g][0].x;
    v.y = odd ? acc[g][1].y : acc[g][0].y;
    v.z = odd ? acc[g][1].z : acc[g][0].z;
    v.w = odd ? acc[g][1].w : acc[g][0].w;
    v.x += __shfl_xor(v.x, 1);
    v.y += __shfl_xor(v.y, 1);
    v.z += __shfl_xor(v.z, 1);
    v.w += __shfl_xor(v.w, 1);
    if ((j & 1) == 0) *reinterpret_cast<f4_t*>(part + ((wave * G + g) * 8 + (j >> 1)) * 16 + 4 * q) = v;
  }
  __syncthreads();
  if (kc != 0) return;
  const float gscale = (*p.ga) * (*p.gw);
  // With argmax keys, each lane keeps the best (value, column) of its
  // activation row m = lane % 16 (idx steps by 64, so m is fixed per lane).
  uint64_t best = 0;
  for (int idx = lane; idx < G * 128; idx += 64) {
    const int g = idx >> 7, r = (idx >> 4) & 7, m = idx & 15;
    float s = 0.f;
    for (int k2 = 0; k2 < KS; ++k2) s += part[(((rb * KS + k2) * G + g) * 8 + r) * 16 + m];
    const uint32_t n = row0 + 8u * g + r;
    if (n < (uint32_t)N && m < M) {
      const float v = s * gscale;
      if (p.argmax_keys) {
        const uint64_t key = argmax_key(v, n);
        best = key > best ? key : best;
      }
      if (p.out) {
        const int64_t o = (int64_t)m * N + n;
        if constexpr (OUT_BF16) {
          reinterpret_cast<uint16_t*>(p.out)[o] = f32_to_bf16_rne(v);
        } else {
          reinterpret_cast<float*>(p.out)[o] = v;
        }
      }
    }
  }
  if (p.argmax_keys) {
    // lanes m, m + 16, m + 32, m + 48 share row m; the maximum key is
    // independent of the order in which the workgroups merge theirs.
    uint64_t o = __shfl_xor(best, 16);
    best = o > best ? o : best;
    o = __shfl_xor(best, 32);
    best = o > best ? o : best;
    // spread over kKeySlots slots per row to keep same-address atomics few
    const uint32_t slot = blockIdx.x % kKeySlots;
    if (lane < M && best != 0)
      atomicMax(reinterpret_cast<unsigned long long*>(p.argmax_keys) + slot * 16u + lane, best);
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

template <int G>
hipError_t launch_g(const GemmArgs& a, hipStream_t stream) {
  const int L = a.K / 256;
  const int64_t blocks = (a.N + 8 * G - 1) / (8 * G);  // row blocks of 8G rows
  const int cus = device_cus();
  // Split K over the waves of a workgroup until there are >= 8 waves per CU.
  int KS = 1;
  while (KS < 8 && KS < L && blocks * KS < 8LL * cus) ++KS;
  const int e_ks = env_int("NVFP4_M16_KS", 0);
  if (e_ks > 0 && e_ks <= 8) KS = e_ks;
  if (KS > L) KS = L;
  const int LW = (L + KS - 1) / KS;
  KS = (L + LW - 1) / LW;  // no wave without lines
  const int nw = (KS >= 4 ? 1 : 4 / KS) * KS;  // row blocks x K slices: 3 to 8 waves
  const int RB = nw / KS;
  const dim3 grid((unsigned)((blocks + RB - 1) / RB));
  const size_t lds = alds_bytes_m16(a.K) + (size_t)nw * G * 128 * sizeof(float);
  if (a.out_bf16) gemm_m16_kernel<G, true><<<grid, 64 * nw, lds, stream>>>(a, KS, LW);
  else gemm_m16_kernel<G, false><<<grid, 64 * nw, lds, stream>>>(a, KS, LW);
  return hipGetLastError();
}

}  // namespace

// The staged activations and the partial sums of up to 8 waves x 4 groups fit
// in 64 KiB of LDS, and 3 waves' threads cover the staging pieces.
bool gemm_m16_supported(const GemmArgs& a) {
  return a.M >= 1 && a.M <= 16 && a.K % 256 == 0 && alds_bytes_m16(a.K) + 8u * 4u * 128u * 4u <= 64u * 1024u &&
         16 * (a.K / 32 + a.K / 256) <= kFillMax * 64 * 3;
}

// G (row groups sharing one dequantized activation operand): 4 when there are
// enough rows for >= 4 row blocks per CU, else 2, else 1.
hipError_t launch_gemm_m16(const GemmArgs& a, hipStream_t stream) {
  const int64_t cus = device_cus();
  int G = a.N >= 32 * 4 * cus ? 4 : a.N >= 16 * cus ? 2 : 1;
  const int e_g = env_int("NVFP4_M16_G", 0);
  if (e_g == 1 || e_g == 2 || e_g == 4) G = e_g;
  return G == 4 ? launch_g<4>(a, stream) : G == 2 ? launch_g<2>(a, stream) : launch_g<1>(a, stream);
}

}  // namespace nvfp4
