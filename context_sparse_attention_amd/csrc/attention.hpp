// Internal interface of the sparse shard attention kernels.
#pragma once

#include "common.hpp"

namespace csa {

struct AttnKernelArgs {
  View q, k, v;
  DevLayout L;
  int mode, idx_heads, idx_width, block_size, dtype, out_dtype;
  const int32_t* idx;
  float scale_log2;  // softmax scale * log2(e): logits are kept in log2 units
  void* out;
  float* lse;
};

hipError_t launch_attn_generic(const AttnKernelArgs& a, hipStream_t stream);

// bf16 block mode with D = Dqk = Dv in {64, 128}, block size a multiple of 64,
// a power-of-two GQA group of at most 128, at most 16384 (key head, block)
// lists and a positive scale.
bool attn_block_mfma_supported(const AttnKernelArgs& a, int n_blocks);
size_t attn_block_mfma_ws_bytes(int n_q, int n_seq, int n_blocks, int hq, int hkv, int dv,
                                int idx_width);
hipError_t launch_attn_block_mfma(const AttnKernelArgs& a, int n_blocks, void* ws,
                                  hipStream_t stream);

// bf16 token mode with one index row per query token, (Dqk, Dv) in
// {(576, 512), (128, 128), (64, 64)}, Hq / Hkv in {32, 64, 128}, positive scale.
bool attn_token_mfma_supported(const AttnKernelArgs& a);
hipError_t launch_attn_token_mfma(const AttnKernelArgs& a, hipStream_t stream);

}  // namespace csa
