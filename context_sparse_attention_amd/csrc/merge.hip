// summary_merge: merge P chunk summaries per row, then optionally finalize.
//
// "Context parallel attention: exchange keys and merge softmax globally",
// paragraph on the chunk summary: both summaries are rescaled to the larger
// maximum before denominators and numerators are added, and the division
// happens once at the end; paragraph on masking: the neutral summary
// (-inf, 0, 0) of an all-masked chunk merges without NaN, and a row with no
// contribution finalizes to output 0 and log-sum-exp -inf.
//
// One thread per (row, value column); parts are visited in ascending order.
#include "common.hpp"

namespace csa {

namespace {

constexpr int kMergeThreads = 256;

template <typename TO>
__global__ __launch_bounds__(kMergeThreads) void k_summary_merge(MergeArgs a) {
  const int64_t t = (int64_t)blockIdx.x * kMergeThreads + threadIdx.x;
  if (t >= a.n_rows * a.dv) return;
  const int64_t r = t / a.dv;
  const int d = (int)(t % a.dv);
  float m = -INFINITY, l = 0.f, z = 0.f;
  for (int p = 0; p < a.n_parts; ++p) {
    const int64_t pr = (int64_t)p * a.n_rows + r;
    const float mp = a.m[pr];
    const float mn = fmaxf(m, mp);
    if (mn == -INFINITY) continue;  // both neutral: stay neutral
    const float wa = (m == -INFINITY) ? 0.f : expf(m - mn);
    const float wb = (mp == -INFINITY) ? 0.f : expf(mp - mn);
    l = wa * l + wb * a.l[pr];
    z = wa * z + wb * a.z[pr * a.dv + d];
    m = mn;
  }
  if (a.z_out) {
    a.z_out[t] = z;
    if (d == 0) {
      a.m_out[r] = m;
      a.l_out[r] = l;
    }
  }
  if (a.o_out) {
    const bool any = l > 0.f && m != -INFINITY;
    store_out(reinterpret_cast<TO*>(a.o_out) + t, any ? z / l : 0.f);
    if (d == 0) a.lse_out[r] = any ? m + logf(l) : -INFINITY;
  }
}

}  // namespace

hipError_t launch_summary_merge(const MergeArgs& a, hipStream_t stream) {
  const int64_t n = a.n_rows * a.dv;
  if (n == 0) return hipSuccess;
  const int grid = (int)((n + kMergeThreads - 1) / kMergeThreads);
  if (a.o_out && a.o_dtype == CSA_BF16)
    hipLaunchKernelGGL((k_summary_merge<__bf16>), dim3(grid), dim3(kMergeThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((k_summary_merge<float>), dim3(grid), dim3(kMergeThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace csa
