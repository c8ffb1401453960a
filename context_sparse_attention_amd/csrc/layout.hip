// Block table of a packed (THD) key stream (construction in block_table.hpp).
#include "block_table.hpp"

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

__global__ __launch_bounds__(kTableThreads) void k_block_table(
    const int32_t* __restrict__ cu, int n_seq, int block_size, int n_blocks, BlockTable bt,
    int32_t* __restrict__ fill, int64_t n_fill, int32_t fill_value) {
  for (int64_t t = threadIdx.x; t < n_fill; t += kTableThreads) fill[t] = fill_value;
  block_table_wg(cu, n_seq, block_size, n_blocks, bt);
}

}  // namespace

hipError_t launch_block_table(const int32_t* cu, int n_seq, int block_size, int n_blocks,
                              BlockTable bt, int32_t* fill, int64_t n_fill,
                              hipStream_t stream) {
  hipLaunchKernelGGL(k_block_table, dim3(1), dim3(kTableThreads), 0, stream, cu, n_seq,
                     block_size, n_blocks, bt, fill, n_fill, (int32_t)0);
  return hipGetLastError();
}

int device_cus() {
  // queried once per process; the library drives one device model
  static int cus = 0;
  if (!cus) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        n > 0)
      cus = n;
    else
      cus = 256;
  }
  return cus;
}

}  // namespace csa
