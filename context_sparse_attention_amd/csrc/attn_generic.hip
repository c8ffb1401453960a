// Sparse shard attention, general-shape path (fp32 math on the vector ALUs).
//
// One wavefront per (row, query head).  The row's selected keys are visited
// 64 at a time (one key per lane): block slots in block order, token slots in
// slot order.  Each visited group is a chunk whose (m, l, z) summary is merged
// into the running one by rescaling to the larger maximum, as in "Context
// parallel attention: exchange keys and merge softmax globally" (paragraph on
// the chunk summary); m is kept in log2 units inside the kernel and turned
// into a natural-log log-sum-exp at the end.  A (row, head) with no selected
// key keeps the neutral summary (-inf, 0, 0) and writes out = 0, lse = -inf.
//
// This path serves fp32 inputs (where accuracy must stay at fp32 level) and
// any shape the MFMA kernels do not cover.
#include "attention.hpp"

namespace csa {

namespace {

constexpr int kWavesPerBlock = 4;
constexpr int kMaxDqk = 576;

template <typename T, typename TO, int DV_LANE>
__global__ __launch_bounds__(kWavesPerBlock * kWave) void k_attn_generic(AttnKernelArgs a) {
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t pair = (int64_t)blockIdx.x * kWavesPerBlock + wave;
  const int hq = a.q.h;
  __shared__ float s_q[kWavesPerBlock][kMaxDqk];
  __shared__ float s_p[kWavesPerBlock][kWave];
  __shared__ int s_key[kWavesPerBlock][kWave];
  if (pair >= (int64_t)a.L.n_q * hq) return;
  const int i = (int)(pair / hq);
  const int h = (int)(pair % hq);
  const int g = h / (hq / a.k.h);
  const int dqk = a.q.d, dv = a.v.d;

  for (int d = lane; d < dqk; d += kWave) s_q[wave][d] = to_f32(elem_ptr<T>(a.q, i, h)[d]);
  __builtin_amdgcn_wave_barrier();

  const RowKeys r = row_keys(a.L, i);
  float m = -INFINITY, l = 0.f;
  float o[DV_LANE];
#pragma unroll
  for (int j = 0; j < DV_LANE; ++j) o[j] = 0.f;

  // fold one group of up to 64 keys (one per lane; key < 0 means none) into (m, l, o)
  auto fold = [&](int key) {
    float x = -INFINITY;
    if (key >= 0) {
      const T* kp = elem_ptr<T>(a.k, key, g);
      float dot = 0.f;
      for (int d = 0; d < dqk; d += 8) {
        float kx[8];
        load8(kp + d, kx);
#pragma unroll
        for (int t = 0; t < 8; ++t) dot = fmaf(s_q[wave][d + t], kx[t], dot);
      }
      x = dot * a.scale_log2;
    }
    const float cm = wave_max(x);
    if (cm == -INFINITY) return;  // all-masked group: neutral, nothing to merge
    const float mn = fmaxf(m, cm);
    const float alpha = (m == -INFINITY) ? 0.f : exp2f(m - mn);
    const float p = (key >= 0) ? exp2f(x - mn) : 0.f;
    l = l * alpha + wave_sum(p);
    s_p[wave][lane] = p;
    s_key[wave][lane] = key;
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int j = 0; j < DV_LANE; ++j) o[j] *= alpha;
    for (int t = 0; t < kWave; ++t) {
      const int kt = s_key[wave][t];
      if (kt < 0) continue;
      const float pt = s_p[wave][t];
      const T* vp = elem_ptr<T>(a.v, kt, g);
#pragma unroll
      for (int j = 0; j < DV_LANE; ++j) {
        const int d = lane + j * kWave;
        if (d < dv) o[j] = fmaf(pt, to_f32(vp[d]), o[j]);
      }
    }
    __builtin_amdgcn_wave_barrier();
    m = mn;
  };

  if (r.valid) {
    const int32_t* slots = a.idx + ((int64_t)i * a.idx_heads + (a.idx_heads == 1 ? 0 : h)) *
                                       a.idx_width;
    if (a.mode == CSA_SEL_BLOCK) {
      for (int s = 0; s < a.idx_width; ++s) {
        const int start = slots[s];
        if (start < r.lo || start > r.hi || (start - r.lo) % a.block_size) continue;
        const int stop = min(min(start + a.block_size, r.end), r.hi + 1);
        for (int base = start; base < stop; base += kWave) {
          const int key = base + lane;
          fold(key < stop ? key : -1);
        }
      }
    } else {
      for (int base = 0; base < a.idx_width; base += kWave) {
        const int s = base + lane;
        int key = -1;
        if (s < a.idx_width) {
          key = slots[s];
          if (key < r.lo || key > r.hi) key = -1;
        }
        fold(key);
      }
    }
  }

  TO* out = reinterpret_cast<TO*>(a.out) + ((int64_t)i * hq + h) * dv;
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int j = 0; j < DV_LANE; ++j) {
    const int d = lane + j * kWave;
    if (d < dv) store_out(out + d, o[j] * inv);
  }
  if (a.lse && lane == 0)
    a.lse[(int64_t)i * hq + h] = l > 0.f ? (m + log2f(l)) * 0.69314718055994531f : -INFINITY;
}

template <typename T, typename TO>
hipError_t launch_dv(const AttnKernelArgs& a, hipStream_t stream) {
  const int64_t pairs = (int64_t)a.L.n_q * a.q.h;
  const int grid = (int)((pairs + kWavesPerBlock - 1) / kWavesPerBlock);
  const dim3 block(kWavesPerBlock * kWave);
  int slot;
  trace_begin(stream, "k_attn_generic", &slot);
  if (a.v.d <= 64)
    hipLaunchKernelGGL((k_attn_generic<T, TO, 1>), dim3(grid), block, 0, stream, a);
  else if (a.v.d <= 128)
    hipLaunchKernelGGL((k_attn_generic<T, TO, 2>), dim3(grid), block, 0, stream, a);
  else if (a.v.d <= 256)
    hipLaunchKernelGGL((k_attn_generic<T, TO, 4>), dim3(grid), block, 0, stream, a);
  else
    hipLaunchKernelGGL((k_attn_generic<T, TO, 8>), dim3(grid), block, 0, stream, a);
  trace_end(stream, slot);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_generic(const AttnKernelArgs& a, hipStream_t stream) {
  if (a.L.n_q == 0) return hipSuccess;
  if (a.dtype == CSA_BF16) {
    if (a.out_dtype == CSA_BF16) return launch_dv<__bf16, __bf16>(a, stream);
    return launch_dv<__bf16, float>(a, stream);
  }
  if (a.out_dtype == CSA_BF16) return launch_dv<float, __bf16>(a, stream);
  return launch_dv<float, float>(a, stream);
}

}  // namespace csa
