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

}  // namespace csa
