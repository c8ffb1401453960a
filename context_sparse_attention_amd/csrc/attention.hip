// Sparse shard attention: picks the kernel family for a request.
#include "attention.hpp"

namespace csa {

size_t attn_ws_bytes(int n_q, int n_seq, int n_blocks, int mode, int hq, int hkv, int dv,
                     int idx_width) {
  if (mode == CSA_SEL_BLOCK)
    return attn_block_mfma_ws_bytes(n_q, n_seq, n_blocks, hq, hkv, dv, idx_width);
  return 256;
}

namespace {
AttnKernelArgs kernel_args(const AttnArgs& a) {
  AttnKernelArgs k;
  k.q = a.q;
  k.k = a.k;
  k.v = a.v;
  k.L = a.L;
  k.mode = a.mode;
  k.idx_heads = a.idx_heads;
  k.idx_width = a.idx_width;
  k.block_size = a.block_size;
  k.dtype = a.dtype;
  k.out_dtype = a.out_dtype;
  k.idx = a.idx;
  k.scale_log2 = a.scale * 1.4426950408889634f;
  k.out = a.out;
  k.lse = a.lse;
  return k;
}
}  // namespace

const char* attention_kernel_family(const AttnArgs& a) {
  const AttnKernelArgs k = kernel_args(a);
  if (attn_block_mfma_supported(k, a.n_blocks)) return "block_mfma";
  if (attn_token_mfma_supported(k)) return "token_mfma";
  return "generic";
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t stream) {
  const AttnKernelArgs k = kernel_args(a);
  if (attn_block_mfma_supported(k, a.n_blocks)) return launch_attn_block_mfma(k, a.n_blocks, a.ws, stream);
  if (attn_token_mfma_supported(k)) return launch_attn_token_mfma(k, stream);
  return launch_attn_generic(k, stream);
}

}  // namespace csa
