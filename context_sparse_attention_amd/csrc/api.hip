// C ABI of libcsa: host-side checks, workspace sizing and kernel enqueue.
//
// Every entry point validates all arguments before enqueueing anything; a
// failure returns a status and leaves its text in csa_last_error().  No C++
// exception leaves this file.
#include <algorithm>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <exception>
#include <mutex>
#include <string>

#include "common.hpp"

// Fixed scratch of moba_gate_topk_noalloc: one copy per device, held until the
// process ends.  Host code never uses the array's name as an address (on the
// host it is only a stand-in); it uses the device address that
// hipGetSymbolAddress returns, looked up once per device with that device
// current (device_scratch below).  Every no-alloc gate call on a device shares
// that device's copy; the gate kernels write every scratch byte they read
// before reading it, so nothing needs clearing between calls.
static __device__ __align__(256) char scratch[CSA_GATE_SCRATCH_BYTES];

namespace csa {
namespace {

thread_local std::string g_last_error;

csa_status fail(csa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

csa_status hip_fail(hipError_t e, const char* what) {
  return fail(CSA_ERR_HIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

size_t elem_size(int dtype) { return dtype == CSA_BF16 ? 2 : 4; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

csa_status check_tensor(const csa_tensor3* t, const char* name, bool need_data = true) {
  if (!t) return fail(CSA_ERR_INVALID_ARG, "%s: null tensor descriptor", name);
  if (t->dtype != CSA_F32 && t->dtype != CSA_BF16)
    return fail(CSA_ERR_INVALID_ARG, "%s: dtype must be CSA_F32 or CSA_BF16", name);
  if (t->n < 0 || t->h <= 0 || t->d <= 0)
    return fail(CSA_ERR_INVALID_ARG, "%s: bad shape [%lld, %d, %d]", name, (long long)t->n,
                t->h, t->d);
  if (t->n >= (int64_t)1 << 31)
    return fail(CSA_ERR_UNSUPPORTED, "%s: more than 2^31-1 tokens", name);
  if (t->d % 8)
    return fail(CSA_ERR_UNSUPPORTED, "%s: last dimension %d is not a multiple of 8", name, t->d);
  const size_t es = elem_size(t->dtype);
  if ((t->stride_n * es) % 16 || (t->stride_h * es) % 16)
    return fail(CSA_ERR_INVALID_ARG, "%s: strides must be multiples of 16 bytes", name);
  if (t->stride_n < 0 || t->stride_h < 0)
    return fail(CSA_ERR_INVALID_ARG, "%s: negative stride", name);
  if (t->h > 1 && t->stride_h < t->d)
    return fail(CSA_ERR_INVALID_ARG, "%s: heads overlap (stride_h %lld < d %d)", name,
                (long long)t->stride_h, t->d);
  if (t->n > 1 && t->stride_n < (int64_t)(t->h - 1) * t->stride_h + t->d)
    return fail(CSA_ERR_INVALID_ARG, "%s: tokens overlap (stride_n %lld)", name,
                (long long)t->stride_n);
  if (need_data && t->n > 0 && !t->data)
    return fail(CSA_ERR_INVALID_ARG, "%s: null data", name);
  if (t->data && !aligned16(t->data))
    return fail(CSA_ERR_INVALID_ARG, "%s: data not 16-byte aligned", name);
  return CSA_OK;
}

csa_status check_layout(const csa_layout* L) {
  if (!L) return fail(CSA_ERR_INVALID_ARG, "layout: null");
  if (L->n_q < 0 || L->n_kv < 0 || L->n_seq < 1)
    return fail(CSA_ERR_INVALID_ARG, "layout: n_q %d, n_kv %d, n_seq %d", L->n_q, L->n_kv,
                L->n_seq);
  if (!L->cu_seqlens_host || !L->cu_seqlens)
    return fail(CSA_ERR_INVALID_ARG, "layout: cu_seqlens (device and host) required");
  if (L->n_q > 0 && (!L->q_pos || !L->q_seq))
    return fail(CSA_ERR_INVALID_ARG, "layout: q_pos and q_seq required");
  const int32_t* cu = L->cu_seqlens_host;
  if (cu[0] != 0) return fail(CSA_ERR_INVALID_ARG, "layout: cu_seqlens[0] must be 0");
  for (int s = 0; s < L->n_seq; ++s)
    if (cu[s + 1] < cu[s])
      return fail(CSA_ERR_INVALID_ARG, "layout: cu_seqlens decreases at %d", s);
  if (cu[L->n_seq] != L->n_kv)
    return fail(CSA_ERR_INVALID_ARG, "layout: cu_seqlens[n_seq] = %d but n_kv = %d",
                cu[L->n_seq], L->n_kv);
  return CSA_OK;
}

csa_status check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (ws_bytes < need)
    return fail(CSA_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, need);
  if (need > 0 && !ws) return fail(CSA_ERR_WORKSPACE, "null workspace");
  if (((uintptr_t)ws & 255u) != 0) return fail(CSA_ERR_WORKSPACE, "workspace not 256-byte aligned");
  return CSA_OK;
}

// Host checks and kernel arguments of a gate call (everything but the workspace).
csa_status gate_args(const csa_tensor3* q, const csa_tensor3* k, const csa_layout* L,
                     int32_t block_size, int32_t topk, int32_t* idx, float* score,
                     MobaGateArgs* a, size_t* need) {
  csa_status st;
  if ((st = check_tensor(q, "q")) || (st = check_tensor(k, "k")) || (st = check_layout(L)))
    return st;
  if (q->dtype != k->dtype) return fail(CSA_ERR_INVALID_ARG, "q and k dtypes differ");
  if (q->n != L->n_q) return fail(CSA_ERR_INVALID_ARG, "q has %lld rows, layout n_q %d",
                                  (long long)q->n, L->n_q);
  if (k->n != L->n_kv) return fail(CSA_ERR_INVALID_ARG, "k has %lld tokens, layout n_kv %d",
                                   (long long)k->n, L->n_kv);
  if (q->d != k->d) return fail(CSA_ERR_INVALID_ARG, "q and k head dims differ");
  if (q->h % k->h) return fail(CSA_ERR_INVALID_ARG, "Hq %d not a multiple of Hkv %d", q->h, k->h);
  if (q->d > 256) return fail(CSA_ERR_UNSUPPORTED, "gate head dim %d > 256", q->d);
  if (block_size < 1) return fail(CSA_ERR_INVALID_ARG, "block_size %d", block_size);
  if (topk < 0 || topk > 32) return fail(CSA_ERR_UNSUPPORTED, "topk %d outside [0, 32]", topk);
  if (L->n_q > 0 && !idx) return fail(CSA_ERR_INVALID_ARG, "null idx");
  if ((int64_t)L->n_q * q->h * (topk + 1) >= ((int64_t)1 << 31))
    return fail(CSA_ERR_UNSUPPORTED, "index output too large");
  const int64_t nb = count_blocks(L->cu_seqlens_host, L->n_seq, block_size);
  if (nb >= ((int64_t)1 << 30)) return fail(CSA_ERR_UNSUPPORTED, "too many blocks");
  *need = moba_gate_ws_bytes(L->n_seq, (int)nb, k->h, k->d, block_size);
  a->q = make_view(q);
  a->k = make_view(k);
  a->L = make_dev_layout(L);
  a->block_size = block_size;
  a->topk = topk;
  a->n_blocks = (int)nb;
  a->dtype = q->dtype;
  a->idx = idx;
  a->score = score;
  a->ws = nullptr;
  return CSA_OK;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

csa_status device_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(CSA_ERR_UNSUPPORTED, "device id %d >= %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p || ((uintptr_t)p & 255u))
      return fail(CSA_ERR_HIP, "scratch symbol address %p not 256-byte aligned", p);
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return CSA_OK;
}

// Host checks and kernel arguments of an attention call (everything but the
// index, output, lse and workspace pointers).
csa_status attn_args(const csa_tensor3* q, const csa_tensor3* k, const csa_tensor3* v,
                     const csa_layout* L, int32_t mode, int32_t idx_heads, int32_t idx_width,
                     int32_t block_size, float softmax_scale, int32_t out_dtype, AttnArgs* a) {
  csa_status st;
  if ((st = check_tensor(q, "q")) || (st = check_tensor(k, "k")) ||
      (st = check_tensor(v, "v")) || (st = check_layout(L)))
    return st;
  if (q->dtype != k->dtype || k->dtype != v->dtype)
    return fail(CSA_ERR_INVALID_ARG, "q, k, v dtypes differ");
  if (q->n != L->n_q) return fail(CSA_ERR_INVALID_ARG, "q rows %lld != n_q %d",
                                  (long long)q->n, L->n_q);
  if (k->n != L->n_kv || v->n != L->n_kv)
    return fail(CSA_ERR_INVALID_ARG, "k/v tokens != n_kv %d", L->n_kv);
  if (q->d != k->d) return fail(CSA_ERR_INVALID_ARG, "q and k head dims differ");
  if (k->h != v->h) return fail(CSA_ERR_INVALID_ARG, "k and v head counts differ");
  if (q->h % k->h) return fail(CSA_ERR_INVALID_ARG, "Hq %d not a multiple of Hkv %d", q->h, k->h);
  if (q->d > 576) return fail(CSA_ERR_UNSUPPORTED, "head dim %d > 576", q->d);
  if (v->d > 512) return fail(CSA_ERR_UNSUPPORTED, "value dim %d > 512", v->d);
  if (mode != CSA_SEL_BLOCK && mode != CSA_SEL_TOKEN)
    return fail(CSA_ERR_INVALID_ARG, "mode %d", mode);
  if (mode == CSA_SEL_BLOCK && block_size < 1)
    return fail(CSA_ERR_INVALID_ARG, "block_size %d", block_size);
  if (idx_heads != 1 && idx_heads != q->h)
    return fail(CSA_ERR_INVALID_ARG, "idx_heads %d must be 1 or Hq %d", idx_heads, q->h);
  if (idx_width < 1) return fail(CSA_ERR_INVALID_ARG, "idx_width %d", idx_width);
  if (out_dtype != CSA_F32 && out_dtype != CSA_BF16)
    return fail(CSA_ERR_INVALID_ARG, "out_dtype %d", out_dtype);
  if (!isfinite(softmax_scale)) return fail(CSA_ERR_INVALID_ARG, "softmax_scale not finite");
  if ((int64_t)L->n_q * idx_heads * idx_width >= ((int64_t)1 << 31) ||
      (int64_t)L->n_q * q->h * idx_width >= ((int64_t)1 << 31))
    return fail(CSA_ERR_UNSUPPORTED, "index too large");
  int64_t nb = 0;
  if (mode == CSA_SEL_BLOCK) nb = count_blocks(L->cu_seqlens_host, L->n_seq, block_size);
  if (nb >= ((int64_t)1 << 30)) return fail(CSA_ERR_UNSUPPORTED, "too many blocks");
  a->q = make_view(q);
  a->k = make_view(k);
  a->v = make_view(v);
  a->L = make_dev_layout(L);
  a->mode = mode;
  a->idx_heads = idx_heads;
  a->idx_width = idx_width;
  a->block_size = block_size;
  a->n_blocks = (int)nb;
  a->dtype = q->dtype;
  a->out_dtype = out_dtype;
  a->idx = nullptr;
  a->scale = softmax_scale;
  a->out = nullptr;
  a->lse = nullptr;
  a->ws = nullptr;
  return CSA_OK;
}

template <typename F>
csa_status guarded(F&& f) {
  try {
    return f();
  } catch (const std::exception& e) {
    return fail(CSA_ERR_INVALID_ARG, "internal error: %s", e.what());
  } catch (...) {
    return fail(CSA_ERR_INVALID_ARG, "internal error");
  }
}

}  // namespace
}  // namespace csa

using namespace csa;

extern "C" {

const char* csa_last_error(void) { return g_last_error.c_str(); }

size_t moba_gate_topk_workspace_size(const csa_layout* L, int32_t hkv, int32_t d,
                                     int32_t block_size) {
  if (!L || !L->cu_seqlens_host || L->n_seq < 1 || block_size < 1 || hkv < 1 || d < 1) return 0;
  const int64_t nb = count_blocks(L->cu_seqlens_host, L->n_seq, block_size);
  return moba_gate_ws_bytes(L->n_seq, (int)nb, hkv, d, block_size);
}

csa_status moba_gate_topk(const csa_tensor3* q, const csa_tensor3* k, const csa_layout* L,
                          int32_t block_size, int32_t topk, int32_t* idx, float* score,
                          void* ws, size_t ws_bytes, void* stream) {
  return guarded([&]() -> csa_status {
    MobaGateArgs a;
    size_t need = 0;
    csa_status st;
    if ((st = gate_args(q, k, L, block_size, topk, idx, score, &a, &need))) return st;
    if ((st = check_ws(ws, ws_bytes, need))) return st;
    a.ws = ws;
    hipError_t e = launch_moba_gate(a, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "moba_gate_topk");
    return CSA_OK;
  });
}

csa_status moba_gate_topk_noalloc(const csa_tensor3* q, const csa_tensor3* k,
                                  const csa_layout* L, int32_t block_size, int32_t topk,
                                  int32_t* idx, float* score, void* stream) {
  return guarded([&]() -> csa_status {
    MobaGateArgs a;
    size_t need = 0;
    csa_status st;
    if ((st = gate_args(q, k, L, block_size, topk, idx, score, &a, &need))) return st;
    if (need > (size_t)CSA_GATE_SCRATCH_BYTES)
      return fail(CSA_ERR_UNSUPPORTED,
                  "moba_gate_topk_noalloc: this shape needs %zu bytes of scratch, more than "
                  "the library's fixed %d (use moba_gate_topk with a workspace)",
                  need, (int)CSA_GATE_SCRATCH_BYTES);
    void* scratch_ptr = nullptr;
    if ((st = device_scratch(&scratch_ptr))) return st;
    a.ws = scratch_ptr;
    hipError_t e = launch_moba_gate(a, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "moba_gate_topk_noalloc");
    return CSA_OK;
  });
}

size_t dsa_indexer_topk_workspace_size(const csa_layout* L, int32_t topk) {
  (void)topk;
  if (!L || L->n_q < 0 || L->n_kv < 0) return 0;
  return dsa_ws_bytes(L->n_q, L->n_kv);
}

csa_status dsa_indexer_topk(const csa_tensor3* iq, const csa_tensor3* ik, const float* w,
                            int64_t w_stride_n, const csa_layout* L, int32_t topk,
                            int32_t* idx, float* score, void* ws, size_t ws_bytes,
                            void* stream) {
  return guarded([&]() -> csa_status {
    csa_status st;
    if ((st = check_tensor(iq, "iq")) || (st = check_tensor(ik, "ik")) ||
        (st = check_layout(L)))
      return st;
    if (iq->dtype != ik->dtype) return fail(CSA_ERR_INVALID_ARG, "iq and ik dtypes differ");
    if (iq->n != L->n_q) return fail(CSA_ERR_INVALID_ARG, "iq rows %lld != n_q %d",
                                     (long long)iq->n, L->n_q);
    if (ik->n != L->n_kv) return fail(CSA_ERR_INVALID_ARG, "ik tokens %lld != n_kv %d",
                                      (long long)ik->n, L->n_kv);
    if (ik->h != 1) return fail(CSA_ERR_INVALID_ARG, "ik must have one head");
    if (iq->d != ik->d) return fail(CSA_ERR_INVALID_ARG, "iq and ik dims differ");
    if (iq->d > 128) return fail(CSA_ERR_UNSUPPORTED, "indexer dim %d > 128", iq->d);
    if (iq->h > 256 || (int64_t)iq->h * iq->d > 8192)
      return fail(CSA_ERR_UNSUPPORTED, "indexer heads x dim %d x %d too large", iq->h, iq->d);
    if (topk < 1) return fail(CSA_ERR_INVALID_ARG, "topk %d < 1", topk);
    if (L->n_q > 0 && (!w || !idx)) return fail(CSA_ERR_INVALID_ARG, "null w or idx");
    if (w_stride_n < iq->h) return fail(CSA_ERR_INVALID_ARG, "w row stride %lld < H_I %d",
                                        (long long)w_stride_n, iq->h);
    if ((int64_t)L->n_q * topk >= ((int64_t)1 << 31))
      return fail(CSA_ERR_UNSUPPORTED, "index output too large");
    const size_t need = dsa_ws_bytes(L->n_q, L->n_kv);
    if ((st = check_ws(ws, ws_bytes, need))) return st;
    DsaArgs a;
    a.iq = make_view(iq);
    a.ik = make_view(ik);
    a.w = w;
    a.w_stride = w_stride_n;
    a.L = make_dev_layout(L);
    a.topk = topk;
    a.dtype = iq->dtype;
    // a row's keys lie in one sequence; their float4 misalignment in the logits is
    // zero when n_kv and every sequence start are multiples of 4
    {
      const int32_t* cu = L->cu_seqlens_host;
      int longest = 0;
      bool aligned = L->n_kv % 4 == 0;
      for (int s = 0; s < L->n_seq; ++s) {
        longest = std::max(longest, cu[s + 1] - cu[s]);
        aligned = aligned && cu[s] % 4 == 0;
      }
      a.max_span = longest + (aligned ? 0 : 3);
    }
    a.idx = idx;
    a.score = score;
    a.ws = ws;
    hipError_t e = launch_dsa_indexer(a, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "dsa_indexer_topk");
    return CSA_OK;
  });
}

size_t sparse_attn_fwd_shard_workspace_size(const csa_layout* L, int32_t mode, int32_t hq,
                                            int32_t hkv, int32_t dv, int32_t idx_width,
                                            int32_t block_size) {
  if (!L || !L->cu_seqlens_host || L->n_seq < 1 || hq < 1 || hkv < 1 || dv < 1 ||
      idx_width < 1)
    return 0;
  int64_t nb = 0;
  if (mode == CSA_SEL_BLOCK) {
    if (block_size < 1) return 0;
    nb = count_blocks(L->cu_seqlens_host, L->n_seq, block_size);
  }
  return attn_ws_bytes(L->n_q, L->n_seq, (int)nb, mode, hq, hkv, dv, idx_width);
}

csa_status sparse_attn_fwd_shard(const csa_tensor3* q, const csa_tensor3* k,
                                 const csa_tensor3* v, const csa_layout* L, int32_t mode,
                                 const int32_t* idx, int32_t idx_heads, int32_t idx_width,
                                 int32_t block_size, float softmax_scale, void* out,
                                 int32_t out_dtype, float* lse, void* ws, size_t ws_bytes,
                                 void* stream) {
  return guarded([&]() -> csa_status {
    AttnArgs a;
    csa_status st;
    if ((st = attn_args(q, k, v, L, mode, idx_heads, idx_width, block_size, softmax_scale,
                        out_dtype, &a)))
      return st;
    if (L->n_q > 0 && (!idx || !out)) return fail(CSA_ERR_INVALID_ARG, "null idx or out");
    if (out && !aligned16(out)) return fail(CSA_ERR_INVALID_ARG, "out not 16-byte aligned");
    const size_t need = attn_ws_bytes(L->n_q, L->n_seq, a.n_blocks, mode, q->h, k->h, v->d,
                                      idx_width);
    if ((st = check_ws(ws, ws_bytes, need))) return st;
    a.idx = idx;
    a.out = out;
    a.lse = lse;
    a.ws = ws;
    hipError_t e = launch_attention(a, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "sparse_attn_fwd_shard");
    return CSA_OK;
  });
}

const char* sparse_attn_fwd_shard_kernel(const csa_tensor3* q, const csa_tensor3* k,
                                         const csa_tensor3* v, const csa_layout* L,
                                         int32_t mode, int32_t idx_heads, int32_t idx_width,
                                         int32_t block_size, float softmax_scale,
                                         int32_t out_dtype) {
  const char* name = nullptr;
  guarded([&]() -> csa_status {
    AttnArgs a;
    csa_status st;
    if ((st = attn_args(q, k, v, L, mode, idx_heads, idx_width, block_size, softmax_scale,
                        out_dtype, &a)))
      return st;
    name = attention_kernel_family(a);
    return CSA_OK;
  });
  return name;
}

// Block count of a backward's shape arguments, or -1 when they are malformed.
static int64_t bwd_shape_blocks(const csa_layout* L, int32_t mode, int32_t dtype, int32_t hq,
                                int32_t hkv, int32_t dqk, int32_t dv, int32_t idx_heads,
                                int32_t idx_width, int32_t block_size) {
  if (!L || !L->cu_seqlens_host || L->n_seq < 1 || L->n_q < 0 || L->n_kv < 0 || hq < 1 ||
      hkv < 1 || dqk < 1 || dv < 1 || idx_heads < 1 || idx_width < 1 ||
      (dtype != CSA_F32 && dtype != CSA_BF16) || (mode != CSA_SEL_BLOCK && mode != CSA_SEL_TOKEN))
    return -1;
  if (mode != CSA_SEL_BLOCK) return 0;
  if (block_size < 1) return -1;
  const int64_t nb = count_blocks(L->cu_seqlens_host, L->n_seq, block_size);
  return nb >= ((int64_t)1 << 30) ? -1 : nb;
}

size_t sparse_attn_bwd_shard_workspace_size(const csa_layout* L, int32_t mode, int32_t dtype,
                                            int32_t hq, int32_t hkv, int32_t dqk, int32_t dv,
                                            int32_t idx_heads, int32_t idx_width,
                                            int32_t block_size) {
  const int64_t nb =
      bwd_shape_blocks(L, mode, dtype, hq, hkv, dqk, dv, idx_heads, idx_width, block_size);
  if (nb < 0) return 0;
  return attn_bwd_ws_bytes(L->n_q, L->n_kv, L->n_seq, (int)nb, mode, dtype, hq, hkv, dqk, dv,
                           idx_heads, idx_width, block_size);
}

const char* sparse_attn_bwd_shard_kernel(const csa_layout* L, int32_t mode, int32_t dtype,
                                         int32_t hq, int32_t hkv, int32_t dqk, int32_t dv,
                                         int32_t idx_heads, int32_t idx_width,
                                         int32_t block_size) {
  const int64_t nb =
      bwd_shape_blocks(L, mode, dtype, hq, hkv, dqk, dv, idx_heads, idx_width, block_size);
  if (nb < 0) {
    fail(CSA_ERR_INVALID_ARG, "sparse_attn_bwd_shard_kernel: malformed arguments");
    return nullptr;
  }
  return attn_bwd_kernel_family(L->n_q, L->n_kv, (int)nb, mode, dtype, hq, hkv, dqk, dv,
                                idx_heads, idx_width, block_size);
}

csa_status sparse_attn_bwd_shard(const csa_tensor3* q, const csa_tensor3* k,
                                 const csa_tensor3* v, const csa_layout* L, int32_t mode,
                                 const int32_t* idx, int32_t idx_heads, int32_t idx_width,
                                 int32_t block_size, float softmax_scale,
                                 const csa_tensor3* out, const csa_tensor3* dout,
                                 const float* lse, float* dq, float* dk, float* dv, void* ws,
                                 size_t ws_bytes, void* stream) {
  return guarded([&]() -> csa_status {
    csa_status st;
    if ((st = check_tensor(q, "q")) || (st = check_tensor(k, "k")) ||
        (st = check_tensor(v, "v")) || (st = check_tensor(out, "out")) ||
        (st = check_tensor(dout, "dout")) || (st = check_layout(L)))
      return st;
    if (q->dtype != k->dtype || k->dtype != v->dtype)
      return fail(CSA_ERR_INVALID_ARG, "q, k, v dtypes differ");
    if (q->n != L->n_q) return fail(CSA_ERR_INVALID_ARG, "q rows %lld != n_q %d",
                                    (long long)q->n, L->n_q);
    if (k->n != L->n_kv || v->n != L->n_kv)
      return fail(CSA_ERR_INVALID_ARG, "k/v tokens != n_kv %d", L->n_kv);
    if (q->d != k->d) return fail(CSA_ERR_INVALID_ARG, "q and k head dims differ");
    if (k->h != v->h) return fail(CSA_ERR_INVALID_ARG, "k and v head counts differ");
    if (q->h % k->h) return fail(CSA_ERR_INVALID_ARG, "Hq %d not a multiple of Hkv %d", q->h, k->h);
    if (q->d > 576) return fail(CSA_ERR_UNSUPPORTED, "head dim %d > 576", q->d);
    if (v->d > 512) return fail(CSA_ERR_UNSUPPORTED, "value dim %d > 512", v->d);
    for (const csa_tensor3* t : {out, dout})
      if (t->n != L->n_q || t->h != q->h || t->d != v->d)
        return fail(CSA_ERR_INVALID_ARG, "out / dout must be [n_q, Hq, Dv] = [%d, %d, %d]",
                    L->n_q, q->h, v->d);
    if (mode != CSA_SEL_BLOCK && mode != CSA_SEL_TOKEN)
      return fail(CSA_ERR_INVALID_ARG, "mode %d", mode);
    if (mode == CSA_SEL_BLOCK && block_size < 1)
      return fail(CSA_ERR_INVALID_ARG, "block_size %d", block_size);
    if (idx_heads != 1 && idx_heads != q->h)
      return fail(CSA_ERR_INVALID_ARG, "idx_heads %d must be 1 or Hq %d", idx_heads, q->h);
    if (idx_width < 1) return fail(CSA_ERR_INVALID_ARG, "idx_width %d", idx_width);
    if (!isfinite(softmax_scale)) return fail(CSA_ERR_INVALID_ARG, "softmax_scale not finite");
    if (L->n_q > 0 && (!idx || !lse || !dq))
      return fail(CSA_ERR_INVALID_ARG, "null idx, lse or dq");
    if (L->n_kv > 0 && (!dk || !dv)) return fail(CSA_ERR_INVALID_ARG, "null dk or dv");
    if ((int64_t)L->n_q * idx_heads * idx_width >= ((int64_t)1 << 31) ||
        (int64_t)L->n_q * q->h >= ((int64_t)1 << 31) ||
        (int64_t)L->n_kv * k->h * 576 >= ((int64_t)1 << 40))
      return fail(CSA_ERR_UNSUPPORTED, "shard too large for int32 index rows");
    int64_t nb = 0;
    if (mode == CSA_SEL_BLOCK) nb = count_blocks(L->cu_seqlens_host, L->n_seq, block_size);
    if (nb >= ((int64_t)1 << 30)) return fail(CSA_ERR_UNSUPPORTED, "too many blocks");
    if ((mode == CSA_SEL_TOKEN ? (int64_t)L->n_kv : nb) * (idx_heads == 1 ? 1 : k->h) >=
        ((int64_t)1 << 30))
      return fail(CSA_ERR_UNSUPPORTED, "too many key lists");
    const size_t need = attn_bwd_ws_bytes(L->n_q, L->n_kv, L->n_seq, (int)nb, mode, q->dtype,
                                          q->h, k->h, q->d, v->d, idx_heads, idx_width,
                                          block_size);
    if ((st = check_ws(ws, ws_bytes, need))) return st;
    AttnBwdArgs a;
    a.q = make_view(q);
    a.k = make_view(k);
    a.v = make_view(v);
    a.o = make_view(out);
    a.dout = make_view(dout);
    a.o_dtype = out->dtype;
    a.dout_dtype = dout->dtype;
    a.L = make_dev_layout(L);
    a.mode = mode;
    a.idx_heads = idx_heads;
    a.idx_width = idx_width;
    a.block_size = block_size;
    a.n_blocks = (int)nb;
    a.dtype = q->dtype;
    a.idx = idx;
    a.lse = lse;
    a.scale = softmax_scale;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.ws = ws;
    hipError_t e = launch_attn_backward(a, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "sparse_attn_bwd_shard");
    return CSA_OK;
  });
}

csa_status summary_merge(int32_t n_parts, int64_t n_rows, int32_t dv, const float* m,
                         const float* l, const float* z, float* m_out, float* l_out,
                         float* z_out, void* o_out, int32_t o_dtype, float* lse_out,
                         void* stream) {
  return guarded([&]() -> csa_status {
    if (n_parts < 0 || n_rows < 0 || dv < 1)
      return fail(CSA_ERR_INVALID_ARG, "n_parts %d, n_rows %lld, dv %d", n_parts,
                  (long long)n_rows, dv);
    if (n_rows * dv >= ((int64_t)1 << 40)) return fail(CSA_ERR_UNSUPPORTED, "too large");
    const bool want_sum = m_out || l_out || z_out;
    const bool want_fin = o_out || lse_out;
    if (want_sum && !(m_out && l_out && z_out))
      return fail(CSA_ERR_INVALID_ARG, "m_out, l_out, z_out must be given together");
    if (want_fin && !(o_out && lse_out))
      return fail(CSA_ERR_INVALID_ARG, "o_out and lse_out must be given together");
    if (!want_sum && !want_fin) return fail(CSA_ERR_INVALID_ARG, "no output requested");
    if (want_fin && o_dtype != CSA_F32 && o_dtype != CSA_BF16)
      return fail(CSA_ERR_INVALID_ARG, "o_dtype %d", o_dtype);
    if (n_parts > 0 && n_rows > 0 && (!m || !l || !z))
      return fail(CSA_ERR_INVALID_ARG, "null input summary");
    MergeArgs a;
    a.n_parts = n_parts;
    a.n_rows = n_rows;
    a.dv = dv;
    a.m = m;
    a.l = l;
    a.z = z;
    a.m_out = m_out;
    a.l_out = l_out;
    a.z_out = z_out;
    a.o_out = o_out;
    a.o_dtype = o_dtype;
    a.lse_out = lse_out;
    hipError_t e = launch_summary_merge(a, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "summary_merge");
    return CSA_OK;
  });
}

csa_status mla_v_up_proj(const csa_tensor3* o, const csa_tensor3* w, void* out,
                         int32_t out_dtype, void* stream) {
  return guarded([&]() -> csa_status {
    csa_status st;
    if ((st = check_tensor(o, "o")) || (st = check_tensor(w, "w"))) return st;
    if (o->dtype != CSA_BF16 || w->dtype != CSA_BF16)
      return fail(CSA_ERR_UNSUPPORTED, "o and w must be bf16");
    if (w->n != o->h)
      return fail(CSA_ERR_INVALID_ARG, "w has %lld heads, o has %d", (long long)w->n, o->h);
    if (w->d != o->d)
      return fail(CSA_ERR_INVALID_ARG, "w latent width %d != o width %d", w->d, o->d);
    if (o->d % 64 || o->d > 8192)
      return fail(CSA_ERR_UNSUPPORTED, "latent width %d (a multiple of 64, at most 8192)", o->d);
    if (o->stride_n * 2 * 128 >= ((int64_t)1 << 32))
      return fail(CSA_ERR_UNSUPPORTED, "o: row stride %lld too large", (long long)o->stride_n);
    if (w->h % 32 || w->h > 128)
      return fail(CSA_ERR_UNSUPPORTED, "output width %d (32, 64, 96 or 128)", w->h);
    if (out_dtype != CSA_F32 && out_dtype != CSA_BF16)
      return fail(CSA_ERR_INVALID_ARG, "out_dtype %d", out_dtype);
    if (o->n > 0 && !out) return fail(CSA_ERR_INVALID_ARG, "out: null");
    if (out && !aligned16(out)) return fail(CSA_ERR_INVALID_ARG, "out: not 16-byte aligned");
    MlaUpArgs a;
    a.o = make_view(o);
    a.w = make_view(w);
    a.n_q = (int)o->n;
    a.out = out;
    a.out_dtype = out_dtype;
    hipError_t e = launch_mla_v_up_proj(a, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "mla_v_up_proj");
    return CSA_OK;
  });
}

}  // extern "C"
