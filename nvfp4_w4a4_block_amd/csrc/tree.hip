// Greedy verification of a candidate tree over the LM head.
//
// Page "TensorRT Edge-LLM Completes the MLPerf Edge Agentic Benchmark 6.4x
// Faster on Jetson AGX Thor", section "Using tree-based multi-token
// prediction to accelerate LLM inference": the target model scores a tree of
// drafted candidates (16 nodes in the benchmark's server configuration) in
// one forward pass and keeps the path that matches its own choices; the
// benchmark runs at temperature 0, so the choice after a node is the argmax
// of that node's LM-head row.  Node v is accepted when its parent is and its
// draft token equals the parent's argmax; the path ends at the deepest
// accepted node (lowest index on ties) and is followed by that node's argmax
// (the bonus token).
//
// The argmax of each row is normally fused into the LM-head GEMM (see
// gemm_m16.hip: argmax keys merged by atomic maxima into 64 slots per row, so
// the 16 x vocabulary fp32 logits need not be written); argmax_rows_kernel
// serves the shapes that kernel does not take, from logits already written.
// The acceptance kernel folds the slots and resets them to zero, so the key
// workspace needs clearing only before its first use.  The persistent
// weight-stream kernel (gemm_m16_stream.hip) runs the same fold, reset and
// walk in its last workgroup instead.
#include "device_common.h"
#include "launch.h"

namespace nvfp4 {
namespace {

// grid (chunks, M): block (c, m) reduces columns [c * 4096, (c + 1) * 4096) of row m.
constexpr int kArgmaxChunk = 4096;

__global__ __launch_bounds__(256) void argmax_rows_kernel(const float* logits, int N, uint64_t* keys) {
  __shared__ uint64_t wbest[4];
  const int m = blockIdx.y;
  const int64_t n0 = (int64_t)blockIdx.x * kArgmaxChunk;
  const int64_t n1 = n0 + kArgmaxChunk < N ? n0 + kArgmaxChunk : N;
  uint64_t best = 0;
  for (int64_t n = n0 + threadIdx.x; n < n1; n += blockDim.x) {
    const uint64_t k = argmax_key(logits[(int64_t)m * N + n], (uint32_t)n);
    best = k > best ? k : best;
  }
  for (int off = 32; off > 0; off >>= 1) {
    const uint64_t o = __shfl_xor(best, off);
    best = o > best ? o : best;
  }
  if ((threadIdx.x & 63) == 0) wbest[threadIdx.x >> 6] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < (int)(blockDim.x >> 6); ++w) best = wbest[w] > best ? wbest[w] : best;
    if (best != 0) atomicMax(reinterpret_cast<unsigned long long*>(keys) + (blockIdx.x % kKeySlots) * 16u + m, best);
  }
}

// One workgroup of 1024 threads; n <= 64 nodes.  The greedy token of node v
// is greedy_in[v], or, from argmax keys, the maximum over the kKeySlots slots
// of row v (v < 16); the slots are then reset to zero.  result = [end, L,
// bonus, path[0 .. L-1], -1 ...] (3 + n entries).  A parent index outside
// [0, v) rejects node v (no read outside the arrays).
__global__ __launch_bounds__(1024) void tree_accept_kernel(int n, const int32_t* parent, const int32_t* draft,
                                                           const int32_t* greedy_in, uint64_t* keys,
                                                           int32_t* greedy_out, int32_t* result) {
  __shared__ uint64_t kbest[kKeySlots * 16];
  const int t = threadIdx.x;
  // Node inputs first, so that their loads overlap the key fold: lane v of
  // wave 0 holds node v's parent, draft token and greedy token.
  int32_t par = -1, dr = 0, gv = 0;
  if (t < n) {
    par = parent[t];
    dr = draft[t];
    if (!keys) gv = greedy_in[t];
  }
  if (keys) {
    // thread t = slot * 16 + row holds one key; rows fold over the slots in LDS
    kbest[t] = keys[t];
    __syncthreads();
    keys[t] = 0;
    for (int half = kKeySlots / 2; half >= 1; half >>= 1) {
      if (t < half * 16) kbest[t] = kbest[t] > kbest[t + half * 16] ? kbest[t] : kbest[t + half * 16];
      __syncthreads();
    }
    if (t < n) gv = (int32_t)(0xFFFFFFFFu - (uint32_t)kbest[t]);
  }
  if (t >= 64) return;  // no barrier follows
  if (greedy_out && t < n) greedy_out[t] = gv;
  tree_walk_wave(n, par, dr, gv, result);
}

}  // namespace

hipError_t launch_argmax_rows(const float* logits, int M, int N, uint64_t* keys, hipStream_t stream) {
  const dim3 grid((unsigned)((N + kArgmaxChunk - 1) / kArgmaxChunk), (unsigned)M);
  argmax_rows_kernel<<<grid, 256, 0, stream>>>(logits, N, keys);
  return hipGetLastError();
}

hipError_t launch_tree_accept(int n, const int32_t* parent, const int32_t* draft, const int32_t* greedy_in,
                              uint64_t* keys, int32_t* greedy_out, int32_t* result, hipStream_t stream) {
  tree_accept_kernel<<<1, kKeySlots * 16, 0, stream>>>(n, parent, draft, greedy_in, keys, greedy_out, result);
  return hipGetLastError();
}

}  // namespace nvfp4
