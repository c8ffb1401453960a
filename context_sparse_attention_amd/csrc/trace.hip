// Kernel tracing: HIP event pairs around the dominant kernel of each call.
//
// While tracing is on, every call records one event pair on its own stream
// around its dominant kernel (the query-tile kernel of block-mode attention,
// the token kernel of token-mode attention, the logits kernel of the indexer,
// the scoring kernel of the gate).  Records go to a ring allocated by
// csa_trace_begin; csa_trace_collect waits for them and returns the times.
#include <mutex>
#include <vector>

#include "common.hpp"

namespace csa {
namespace {

struct Record {
  hipEvent_t begin = nullptr, end = nullptr;
  const char* kernel = "";
};

std::mutex g_mu;
std::vector<Record> g_ring;
int g_next = 0;
bool g_on = false;

}  // namespace

void trace_begin(hipStream_t stream, const char* kernel, int* slot) {
  *slot = -1;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_on || g_next >= (int)g_ring.size()) return;
  *slot = g_next++;
  g_ring[*slot].kernel = kernel;
  (void)hipEventRecord(g_ring[*slot].begin, stream);
}

void trace_end(hipStream_t stream, int slot) {
  if (slot < 0) return;
  std::lock_guard<std::mutex> lock(g_mu);
  (void)hipEventRecord(g_ring[slot].end, stream);
}

}  // namespace csa

using namespace csa;

extern "C" {

int csa_trace_begin(int max_records) {
  std::lock_guard<std::mutex> lock(g_mu);
  for (auto& r : g_ring) {
    (void)hipEventDestroy(r.begin);
    (void)hipEventDestroy(r.end);
  }
  g_ring.clear();
  g_next = 0;
  g_on = false;
  if (max_records <= 0) return 0;
  g_ring.resize(max_records);
  for (auto& r : g_ring) {
    if (hipEventCreate(&r.begin) != hipSuccess || hipEventCreate(&r.end) != hipSuccess)
      return CSA_ERR_HIP;
  }
  g_on = true;
  return 0;
}

int csa_trace_collect(float* ms, const char** kernels, int max) {
  std::lock_guard<std::mutex> lock(g_mu);
  const int n = g_next < max ? g_next : max;
  for (int i = 0; i < n; ++i) {
    float t = -1.f;
    if (hipEventSynchronize(g_ring[i].end) == hipSuccess)
      (void)hipEventElapsedTime(&t, g_ring[i].begin, g_ring[i].end);
    if (ms) ms[i] = t;
    if (kernels) kernels[i] = g_ring[i].kernel;
  }
  g_next = 0;
  return n;
}

}  // extern "C"
