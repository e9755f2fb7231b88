// Read-only streaming ceiling: the bytes a weight-streaming product must read
// (the packed codes and the block scales of one weight matrix), read once with
// nothing else done to them.  Low-batch decoding is bound by DRAM bandwidth
// (page "TensorRT Edge-LLM Completes the MLPerf Edge Agentic Benchmark 6.4x
// Faster on Jetson AGX Thor", section "Using NVFP4 quantization to accelerate
// Qwen3.6-27B inference"), so how fast plain HIP code can read exactly those
// bytes is the practical ceiling a GEMV or M=16 GEMM of the same matrix is
// measured against, beside the 8 TB/s of the HBM3E specification.
//
// Each wave reads one contiguous span of one of the two arrays, 1 KiB per
// instruction (16 bytes per lane), kD instructions in flight, with the
// non-temporal hint (the data is read once).  Loads are buffer loads: the
// tail of a span past its array reads zeros without touching memory.  The
// values each lane reads are folded by XOR and its fold is stored only if it
// equals a caller-chosen value, so the loads cannot be removed and nothing is
// written in practice.
#include "device_common.h"
#include "launch.h"

namespace nvfp4 {
namespace {

// A sweep on MI355X (loads in flight 4 / 8 / 16, 8 .. 32 waves per CU, with
// and without the non-temporal hint; 73.7 MB and 437.6 MB streams over
// rotating copies) put 16 loads and 32 waves per CU at or within 2% of the
// best for both sizes; the hint is worth 10-12%.
constexpr int kD = 16;                // 1 KiB loads in flight per wave
constexpr int kWavesPerGroup = 4;
constexpr int kWavesPerCu = 32;       // waves per compute unit
constexpr uint32_t kOOB = 0x80000000u;

__global__ __launch_bounds__(64 * kWavesPerGroup) void read_stream_kernel(const uint8_t* a, uint32_t a_bytes,
                                                                          const uint8_t* b, uint32_t b_bytes,
                                                                          uint32_t span, uint32_t a_waves,
                                                                          uint32_t* sink, uint32_t magic) {
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t wave = blockIdx.x * kWavesPerGroup + (threadIdx.x >> 6);
  const bool in_a = wave < a_waves;
  const uint32_t w = __builtin_amdgcn_readfirstlane(in_a ? wave : wave - a_waves);
  const uint32_t n = in_a ? a_bytes : b_bytes;
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(in_a ? a : b), (short)0, (int)n, 0x00020000);
  const uint32_t begin = w * span, end = begin + span < n ? begin + span : n;
  uint32_t acc = 0;
  for (uint32_t off = begin; off < end; off += 1024u * kD) {
    u4_t v[kD];
#pragma unroll
    for (int d = 0; d < kD; ++d) {
      const uint32_t o = off + 1024u * d + 16u * lane;
      v[d] = __builtin_amdgcn_raw_buffer_load_b128(r, o < end ? o : kOOB, 0, 2);
    }
#pragma unroll
    for (int d = 0; d < kD; ++d) acc ^= v[d].x ^ v[d].y ^ v[d].z ^ v[d].w;
  }
  if (acc == magic) sink[0] = acc;
}

int stream_cus() {
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

}  // namespace

// The waves split the two arrays in proportion to their sizes; every span is
// a whole number of kilobytes.
hipError_t launch_read_stream(const uint8_t* a, int64_t a_bytes, const uint8_t* b, int64_t b_bytes, uint32_t* sink,
                              uint32_t magic, hipStream_t stream) {
  const int64_t total = a_bytes + b_bytes;
  if (total == 0) return hipSuccess;
  const int64_t waves = (int64_t)stream_cus() * kWavesPerCu;
  const int64_t span = ((total + waves - 1) / waves + 1023) / 1024 * 1024;
  const int64_t a_waves = (a_bytes + span - 1) / span, b_waves = (b_bytes + span - 1) / span;
  const int64_t groups = (a_waves + b_waves + kWavesPerGroup - 1) / kWavesPerGroup;
  read_stream_kernel<<<(unsigned)groups, 64 * kWavesPerGroup, 0, stream>>>(
      a, (uint32_t)a_bytes, b, (uint32_t)b_bytes, (uint32_t)span, (uint32_t)a_waves, sink, magic);
  return hipGetLastError();
}

}  // namespace nvfp4
