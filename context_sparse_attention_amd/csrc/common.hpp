// Shared device helpers and launcher declarations of libcsa (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "csa.h"

namespace csa {

constexpr int kWave = 64;  // CDNA wavefront width

// Device-side view of a csa_tensor3 (element offsets, not bytes).
struct View {
  const void* data;
  int64_t stride_n;
  int64_t stride_h;
  int32_t n, h, d;
};

inline View make_view(const csa_tensor3* t) {
  return View{t->data, t->stride_n, t->stride_h, (int32_t)t->n, t->h, t->d};
}

// Layout arrays on the device.
struct DevLayout {
  const int32_t* q_pos;
  const int32_t* q_seq;
  const int32_t* cu;
  int32_t n_q;
  int32_t n_kv;
  int32_t n_seq;
};

inline DevLayout make_dev_layout(const csa_layout* L) {
  return DevLayout{L->q_pos, L->q_seq, L->cu_seqlens, L->n_q, L->n_kv, L->n_seq};
}

// Permitted keys of a row: [lo, hi] inclusive, inside sequence [lo, end).
struct RowKeys {
  int lo, hi, end, seq;
  bool valid;
};

__device__ inline RowKeys row_keys(const DevLayout& L, int i) {
  RowKeys r;
  r.seq = L.q_seq[i];
  r.valid = false;
  r.lo = 0;
  r.hi = -1;
  r.end = 0;
  if (r.seq >= 0 && r.seq < L.n_seq) {
    const int lo = L.cu[r.seq];
    const int end = L.cu[r.seq + 1];
    const int pos = L.q_pos[i];
    if (pos >= lo && pos < end) {
      r.lo = lo;
      r.hi = pos;
      r.end = end;
      r.valid = true;
    }
  }
  return r;
}

// ---- element access --------------------------------------------------------
__device__ inline float to_f32(float x) { return x; }
__device__ inline float to_f32(__bf16 x) { return (float)x; }

template <typename T>
__device__ inline const T* elem_ptr(const View& v, int64_t t, int h) {
  return reinterpret_cast<const T*>(v.data) + t * v.stride_n + (int64_t)h * v.stride_h;
}

// Load 8 consecutive elements (16 B for bf16, 32 B for f32) as floats.
__device__ inline void load8(const __bf16* p, float* out) {
  const uint4 raw = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    out[2 * j] = __uint_as_float(w[j] << 16);
    out[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
  }
}
__device__ inline void load8(const float* p, float* out) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
  out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}

__device__ inline void store_out(float* p, float x) { *p = x; }
__device__ inline void store_out(__bf16* p, float x) { *p = (__bf16)x; }

// ---- wave reductions (wave64) ----------------------------------------------
__device__ inline float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, kWave));
  return x;
}
__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, kWave);
  return x;
}

// Order-preserving map of a float to uint32 (larger float -> larger key);
// -0.0 is folded onto +0.0 so that equal values tie.
__device__ inline uint32_t float_key(float x) {
  uint32_t b = __float_as_uint(x + 0.0f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Carves 256-byte aligned pieces out of a caller workspace.
struct Carver {
  char* base;
  size_t used = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  template <typename T>
  T* take(size_t count) {
    used = align_up(used, 256);
    T* p = reinterpret_cast<T*>(base ? base + used : nullptr);
    used += count * sizeof(T);
    return p;
  }
};

int device_cus();  // compute units of the current device (attn_block_mfma.hip)

// ---- tracing (trace.hip) ----------------------------------------------------
void trace_begin(hipStream_t stream, const char* kernel, int* slot);
void trace_end(hipStream_t stream, int slot);

// ---- block table of a packed stream ----------------------------------------
struct BlockTable {
  int32_t* blk_off;  // [n_seq + 1] first global block of each sequence
  int2* blocks;      // [n_blocks]  (start, length)
  int32_t* blk_seq;  // [n_blocks]  owning sequence
};

int64_t count_blocks(const int32_t* cu_host, int n_seq, int block_size);

hipError_t launch_block_table(const int32_t* cu, int n_seq, int block_size, int n_blocks,
                              BlockTable bt, int32_t* zero_i32, int64_t n_zero,
                              hipStream_t stream);

// ---- launchers (each returns the launch status) -----------------------------
struct MobaGateArgs {
  View q, k;
  DevLayout L;
  int block_size, topk, n_blocks, dtype;
  int32_t* idx;
  float* score;
  void* ws;
};
size_t moba_gate_ws_bytes(int n_seq, int n_blocks, int hkv, int d, int block_size);
hipError_t launch_moba_gate(const MobaGateArgs& a, hipStream_t stream);

struct DsaArgs {
  View iq, ik;
  const float* w;
  int64_t w_stride;
  DevLayout L;
  int topk, dtype;
  int max_span;  // bound on a row's permitted keys plus its float4 misalignment
  int32_t* idx;
  float* score;
  void* ws;
};
size_t dsa_ws_bytes(int n_q, int n_kv);
hipError_t launch_dsa_indexer(const DsaArgs& a, hipStream_t stream);

struct AttnArgs {
  View q, k, v;
  DevLayout L;
  int mode, idx_heads, idx_width, block_size, n_blocks, dtype, out_dtype;
  const int32_t* idx;
  float scale;
  void* out;
  float* lse;
  void* ws;
};
size_t attn_ws_bytes(int n_q, int n_seq, int n_blocks, int mode, int hq, int hkv, int dv,
                     int idx_width);
hipError_t launch_attention(const AttnArgs& a, hipStream_t stream);
// "block_mfma", "token_mfma" or "generic": the kernel family launch_attention picks
const char* attention_kernel_family(const AttnArgs& a);

struct AttnBwdArgs {
  View q, k, v;
  View o, dout;  // forward output and its gradient [n_q, Hq, Dv]
  int o_dtype, dout_dtype;
  DevLayout L;
  int mode, idx_heads, idx_width, block_size, n_blocks, dtype;
  const int32_t* idx;
  const float* lse;
  float scale;
  float *dq, *dk, *dv;
  void* ws;
};
size_t attn_bwd_ws_bytes(int n_q, int n_kv, int n_seq, int n_blocks, int mode, int dtype, int hq,
                         int hkv, int dqk, int dv, int idx_heads, int idx_width, int block_size);
hipError_t launch_attn_backward(const AttnBwdArgs& a, hipStream_t stream);
// "block_mfma" or "generic": the kernel family launch_attn_backward picks
const char* attn_bwd_kernel_family(int n_q, int n_kv, int n_blocks, int mode, int dtype, int hq,
                                   int hkv, int dqk, int dv, int idx_heads, int idx_width,
                                   int block_size);

struct MergeArgs {
  int n_parts;
  int64_t n_rows;
  int dv;
  const float *m, *l, *z;
  float *m_out, *l_out, *z_out;
  void* o_out;
  int o_dtype;
  float* lse_out;
};
hipError_t launch_summary_merge(const MergeArgs& a, hipStream_t stream);

struct MlaUpArgs {
  View o;  // [n_q, Hq, Dl] bf16
  View w;  // [Hq, Dv, Dl] bf16 (n = head, h = output channel, d = latent channel)
  int n_q;
  void* out;  // [n_q, Hq, Dv] contiguous
  int out_dtype;
};
hipError_t launch_mla_v_up_proj(const MlaUpArgs& a, hipStream_t stream);

}  // namespace csa
