// DSA-style token indexer and top-k token selection.
//
// Megatron-LM PR #3674 ("[1/2] Enable DSA CP, THD with absorbed MLA",
// Description): an indexer picks the top-k key tokens of each query before
// sparse attention; Megatron-LM issue #4878 ("Strategy: allgather CP mode"):
// the indexer runs over the gathered keys and emits indices in global
// coordinates under the causal mask shifted to the shard's offset.  Logit of
// key j for row i: sum_h w[i,h] * max(0, iq[i,h] . ik[j]) over the permitted
// keys j in [lo_i, pos_i] only ("logits cleaning": nothing else is written).
//
// Two kernels:
//   k_dsa_logits - one workgroup per (row, 256-key tile): the row's indexer
//                  queries sit in LDS, each thread holds one key in registers
//                  and reduces the 64 heads in fp32;
//   k_dsa_select - one workgroup per row: 4-pass 8-bit radix select of the
//                  k-th largest logit on order-preserving uint32 keys, then an
//                  index-order compaction that takes every larger logit and
//                  the lowest-index equal ones (ties to the lower index).
#include "common.hpp"

namespace csa {

namespace {

constexpr int kLogitThreads = 256;
constexpr int kSelectThreads = 1024;
constexpr int kMaxIndexerElems = 8192;  // H_I * D_I held in LDS as fp32

template <typename T, int DI_MAX>
__global__ __launch_bounds__(kLogitThreads) void k_dsa_logits(View iq, View ik,
                                                              const float* __restrict__ w,
                                                              int64_t w_stride, DevLayout L,
                                                              float* __restrict__ logits) {
  const int i = blockIdx.y;
  const RowKeys r = row_keys(L, i);
  if (!r.valid) return;
  const int j = r.lo + blockIdx.x * kLogitThreads + threadIdx.x;
  if (r.lo + blockIdx.x * kLogitThreads > r.hi) return;  // whole tile beyond the row

  const int hi = iq.h, di = iq.d;
  __shared__ float s_q[kMaxIndexerElems];
  __shared__ float s_w[256];
  for (int e = threadIdx.x * 8; e < hi * di; e += kLogitThreads * 8) {
    float x[8];
    load8(elem_ptr<T>(iq, i, e / di) + (e % di), x);
#pragma unroll
    for (int t = 0; t < 8; ++t) s_q[e + t] = x[t];
  }
  for (int h = threadIdx.x; h < hi; h += kLogitThreads) s_w[h] = w[(int64_t)i * w_stride + h];
  __syncthreads();
  if (j > r.hi) return;

  float kv[DI_MAX];
#pragma unroll
  for (int d8 = 0; d8 < DI_MAX; d8 += 8) {
    if (d8 < di) load8(elem_ptr<T>(ik, j, 0) + d8, kv + d8);
    else {
#pragma unroll
      for (int t = 0; t < 8; ++t) kv[d8 + t] = 0.f;
    }
  }
  float acc = 0.f;
  for (int h = 0; h < hi; ++h) {
    const float* qh = s_q + h * di;
    float dot = 0.f;
#pragma unroll
    for (int d = 0; d < DI_MAX; ++d)
      if (d < di) dot = fmaf(qh[d], kv[d], dot);
    acc = fmaf(s_w[h], fmaxf(dot, 0.f), acc);
  }
  logits[(int64_t)i * L.n_kv + j] = acc;
}

// Exclusive prefix count of a per-thread flag across the workgroup, plus the total.
__device__ inline int block_excl_count(bool flag, int* s_wave, int* total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const uint64_t ballot = __ballot(flag);
  const int before_in_wave = __popcll(ballot & ((1ull << lane) - 1ull));
  if (lane == 0) s_wave[wave] = __popcll(ballot);
  __syncthreads();
  int before = 0, all = 0;
  for (int w = 0; w < kSelectThreads / kWave; ++w) {
    const int c = s_wave[w];
    if (w < wave) before += c;
    all += c;
  }
  __syncthreads();
  *total = all;
  return before + before_in_wave;
}

__global__ __launch_bounds__(kSelectThreads) void k_dsa_select(DevLayout L, int topk,
                                                               const float* __restrict__ logits,
                                                               int32_t* __restrict__ idx,
                                                               float* __restrict__ score) {
  const int i = blockIdx.x;
  const RowKeys r = row_keys(L, i);
  const int n = r.valid ? r.hi - r.lo + 1 : 0;
  const float* row = logits + (int64_t)i * L.n_kv + r.lo;
  int32_t* out = idx + (int64_t)i * topk;
  float* out_s = score ? score + (int64_t)i * topk : nullptr;

  if (n <= topk) {
    for (int t = threadIdx.x; t < topk; t += kSelectThreads) {
      out[t] = t < n ? r.lo + t : -1;
      if (out_s) out_s[t] = t < n ? row[t] : -INFINITY;
    }
    return;
  }

  __shared__ int s_hist[256];
  __shared__ int s_wave[kSelectThreads / kWave];
  __shared__ uint32_t s_prefix;
  __shared__ int s_remaining;
  uint32_t prefix = 0, mask = 0;
  int remaining = topk;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int b = threadIdx.x; b < 256; b += kSelectThreads) s_hist[b] = 0;
    __syncthreads();
    for (int t = threadIdx.x; t < n; t += kSelectThreads) {
      const uint32_t u = float_key(row[t]);
      if ((u & mask) == prefix) atomicAdd(&s_hist[(u >> shift) & 255u], 1);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      int above = 0;
      int digit = 255;
      for (; digit > 0; --digit) {
        if (above + s_hist[digit] >= remaining) break;
        above += s_hist[digit];
      }
      s_prefix = prefix | ((uint32_t)digit << shift);
      s_remaining = remaining - above;
    }
    __syncthreads();
    prefix = s_prefix;
    remaining = s_remaining;
    mask |= 255u << shift;
    __syncthreads();
  }
  // prefix is the key of the k-th largest logit; `remaining` equal keys are taken
  int eq_carry = 0, out_carry = 0;
  for (int base = 0; base < n; base += kSelectThreads) {
    const int t = base + threadIdx.x;
    uint32_t u = 0;
    float x = 0.f;
    if (t < n) {
      x = row[t];
      u = float_key(x);
    }
    const bool gt = t < n && u > prefix;
    const bool eq = t < n && u == prefix;
    int eq_total;
    const int eq_rank = eq_carry + block_excl_count(eq, s_wave, &eq_total);
    const bool sel = gt || (eq && eq_rank < remaining);
    int sel_total;
    const int slot = out_carry + block_excl_count(sel, s_wave, &sel_total);
    if (sel) {
      out[slot] = r.lo + t;
      if (out_s) out_s[slot] = x;
    }
    eq_carry += eq_total;
    out_carry += sel_total;
  }
}

template <typename T>
hipError_t launch_typed(const DsaArgs& a, hipStream_t stream) {
  float* logits = static_cast<float*>(a.ws);
  if (a.L.n_q == 0) return hipSuccess;
  const int tiles = (a.L.n_kv + kLogitThreads - 1) / kLogitThreads;
  if (tiles > 0) {
    hipLaunchKernelGGL((k_dsa_logits<T, 128>), dim3(tiles, a.L.n_q), dim3(kLogitThreads), 0,
                       stream, a.iq, a.ik, a.w, a.w_stride, a.L, logits);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_dsa_select, dim3(a.L.n_q), dim3(kSelectThreads), 0, stream, a.L,
                     a.topk, logits, a.idx, a.score);
  return hipGetLastError();
}

}  // namespace

size_t dsa_ws_bytes(int n_q, int n_kv) {
  return align_up((size_t)n_q * (size_t)n_kv * sizeof(float), 256);
}

int dsa_max_indexer_elems() { return kMaxIndexerElems; }

hipError_t launch_dsa_indexer(const DsaArgs& a, hipStream_t stream) {
  if (a.dtype == CSA_BF16) return launch_typed<__bf16>(a, stream);
  return launch_typed<float>(a, stream);
}

}  // namespace csa
