// Block table of a packed (THD) key stream.
//
// Blocks are cut per packed sequence from its first token, block_size tokens
// each, the last one possibly shorter, so that no block straddles two
// sequences (packed sequences keep their boundaries: "Context parallel
// attention: exchange keys and merge softmax globally", paragraph on masks).
#include "common.hpp"

namespace csa {

int64_t count_blocks(const int32_t* cu_host, int n_seq, int block_size) {
  int64_t n = 0;
  for (int s = 0; s < n_seq; ++s) {
    const int64_t len = (int64_t)cu_host[s + 1] - cu_host[s];
    n += (len + block_size - 1) / block_size;
  }
  return n;
}

namespace {

constexpr int kTableThreads = 1024;

// Inclusive scan across the workgroup (1024 threads = 16 waves).
__device__ int block_inclusive_scan(int x, int* s_wave) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(x, off, kWave);
    if (lane >= off) x += y;
  }
  if (lane == kWave - 1) s_wave[wave] = x;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += s_wave[w];
  __syncthreads();
  return x + before;
}

__global__ __launch_bounds__(kTableThreads) void k_block_table(
    const int32_t* __restrict__ cu, int n_seq, int block_size, int n_blocks, BlockTable bt,
    int32_t* __restrict__ fill, int64_t n_fill, int32_t fill_value) {
  __shared__ int s_wave[kTableThreads / kWave];
  __shared__ int s_total;
  for (int64_t t = threadIdx.x; t < n_fill; t += kTableThreads) fill[t] = fill_value;

  int carry = 0;
  for (int base = 0; base < n_seq; base += kTableThreads) {
    const int s = base + threadIdx.x;
    int nb = 0;
    if (s < n_seq) nb = (cu[s + 1] - cu[s] + block_size - 1) / block_size;
    const int incl = block_inclusive_scan(nb, s_wave);
    if (s < n_seq) bt.blk_off[s] = carry + incl - nb;
    // total of this chunk = inclusive value of the last thread of the chunk
    if (threadIdx.x == kTableThreads - 1) s_total = incl;
    __syncthreads();
    carry += s_total;
    __syncthreads();
  }
  if (threadIdx.x == 0) bt.blk_off[n_seq] = carry;
  __syncthreads();

  for (int b = threadIdx.x; b < n_blocks; b += kTableThreads) {
    // largest s in [0, n_seq) with blk_off[s] <= b; empty sequences share an
    // offset with the next one, and the search lands on the non-empty one.
    int lo = 0, hi = n_seq - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (bt.blk_off[mid] <= b) lo = mid; else hi = mid - 1;
    }
    const int seq = lo;
    const int start = cu[seq] + (b - bt.blk_off[seq]) * block_size;
    const int len = min(block_size, cu[seq + 1] - start);
    bt.blocks[b] = make_int2(start, len);
    bt.blk_seq[b] = seq;
  }
}

}  // namespace

hipError_t launch_block_table(const int32_t* cu, int n_seq, int block_size, int n_blocks,
                              BlockTable bt, int32_t* fill, int64_t n_fill,
                              hipStream_t stream) {
  hipLaunchKernelGGL(k_block_table, dim3(1), dim3(kTableThreads), 0, stream, cu, n_seq,
                     block_size, n_blocks, bt, fill, n_fill, (int32_t)0);
  return hipGetLastError();
}

}  // namespace csa
