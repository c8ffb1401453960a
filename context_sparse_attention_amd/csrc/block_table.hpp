// Block table of a packed (THD) key stream, built by one workgroup.
//
// Blocks are cut per packed sequence from its first token, block_size tokens
// each, the last one possibly shorter, so that no block straddles two
// sequences (packed sequences keep their boundaries: "Context parallel
// attention: exchange keys and merge softmax globally", paragraph on masks).
#pragma once

#include "common.hpp"

namespace csa {

constexpr int kTableThreads = 1024;

// Inclusive scan over the kTableThreads threads of the workgroup.
__device__ inline int table_inclusive_scan(int x, int* s_wave) {
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

// Fills bt (blk_off[n_seq + 1], blocks[n_blocks] as (start, len), blk_seq) with
// the workgroup's kTableThreads threads; ends after a barrier, so the caller's
// threads may read bt through the cache right away.
__device__ inline void block_table_wg(const int32_t* __restrict__ cu, int n_seq, int block_size,
                                      int n_blocks, BlockTable bt) {
  __shared__ int s_wave[kTableThreads / kWave];
  __shared__ int s_total;
  int carry = 0;
  for (int base = 0; base < n_seq; base += kTableThreads) {
    const int s = base + threadIdx.x;
    int nb = 0;
    if (s < n_seq) nb = (cu[s + 1] - cu[s] + block_size - 1) / block_size;
    const int incl = table_inclusive_scan(nb, s_wave);
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
  __syncthreads();
}

}  // namespace csa
