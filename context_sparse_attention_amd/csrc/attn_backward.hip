// Backward of the sparse shard attention with the selection held fixed.
//
// "Context parallel attention: exchange keys and merge softmax globally",
// paragraph on positions and masks: the backward pass must return the key and
// value gradients to their owners; Megatron-LM issue #4878, "Strategy:
// allgather CP mode", backward step: the gathered keys' and values' gradients
// are computed on each rank, then reduce-scattered (that reduction is outside
// this one-GPU library).  With the loss's gradient dO of the output, the
// forward's log-sum-exp and P_j = exp(x_j - lse), x_j = scale q . k_j:
//
//   D      = dO . O                       (k_bwd_delta)
//   dx_j   = P_j (dO . v_j - D)
//   dq     = scale sum_j dx_j k_j         (k_bwd_dq: one wave per (row, head))
//   dk_j   = scale sum dx_j q,  dv_j = sum P_j dO
//            over every (row, head) whose selection holds key j (k_bwd_dkdv)
//
// dK/dV need, per key, the index rows that selected it: the selection is
// inverted into lists, one per chunk (a key in token mode, a block in block
// mode; per key head when every query head has its own index row).  The lists
// hold flat slot ids (index row * width + slot) in ascending order, so each
// key's sums run in a fixed order and the results are bitwise reproducible
// without floating-point atomics:
//   k_bwd_hist   each wave counts its consecutive index rows' entries per list
//   k_scan_*     exclusive scan of the counts, list-major then wave
//   k_bwd_fill   each wave places its index rows one at a time, in order (a
//                row's entries in one list are its repeated slots, whose order
//                does not change any sum)
// With at most kLdsLists lists, one workgroup per range takes the place of the
// waves, with the counts and cursors in LDS: the same counts, offsets and list
// order (up to a row's repeated slots) without a global atomic per entry.  Index
// rows of at least kBwThreads slots go row by row (k_bwd_hist_lds, k_bwd_fill_lds),
// shorter ones in flat batches of entries (k_bwd_hist_flat, k_bwd_fill_flat).
// bf16 block mode with D in {64, 128} and one index row per query head runs the
// matrix-core kernels of attn_backward_mfma.hip over these lists; every other
// case runs k_bwd_dq / k_bwd_dkdv below, fp32 on the vector ALUs (exact bf16
// inputs widened).
#include <algorithm>

#include "backward.hpp"

namespace csa {

namespace {

constexpr int kBwThreads = 256;
constexpr int kBwWaves = kBwThreads / kWave;
constexpr int kMaxDq = 576;  // the widest key
constexpr int kMaxDvB = 512;
constexpr int kDqL = kMaxDq / kWave;   // per-lane key dims (lane + 64 t)
constexpr int kDvL = kMaxDvB / kWave;  // per-lane value dims
constexpr float kLog2e = 1.4426950408889634f;

struct BwArgs {
  View q, k, v, o, dout;
  DevLayout L;
  int mode, idx_heads, idx_width, block_size, n_blocks;
  const int32_t* idx;
  const float* lse;
  float scale, scale_log2;
  float* dq;
  float* dk;
  float* dv;
  // workspace
  float* delta;      // [n_q * Hq]
  BlockTable bt;     // block mode
  int32_t* hist;     // [n_lists * R]: counts, then cursors
  int32_t* list_off; // [n_lists + 1]
  int32_t* totals;   // scan block totals
  int32_t* entries;  // index-row ids, list by list
  int n_lists, R, rows_per_range;
  int64_t n_hist;
};

__device__ __forceinline__ float ld(const View& t, int dtype, int64_t n, int h, int e) {
  if (dtype == CSA_BF16) return (float)elem_ptr<__bf16>(t, n, h)[e];
  return elem_ptr<float>(t, n, h)[e];
}

// List id of slot value s of index row (i, hi), or -1 when the slot selects no
// permitted key of the row.
__device__ __forceinline__ int slot_list(const BwArgs& a, const RowKeys& r, int hi, int s) {
  if (!r.valid || s < r.lo || s > r.hi) return -1;
  const int G = a.q.h / a.k.h;
  const int gsel = a.idx_heads == 1 ? 0 : hi / G;
  if (a.mode == CSA_SEL_TOKEN) return gsel * a.L.n_kv + s;
  if ((s - r.lo) % a.block_size) return -1;
  const int b = a.bt.blk_off[r.seq] + (s - r.lo) / a.block_size;
  return gsel * a.n_blocks + b;
}

__global__ void k_fill_i32(int32_t* p, int64_t n, int32_t v) {
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < n;
       t += (int64_t)gridDim.x * blockDim.x)
    p[t] = v;
}

// D[i, h] = dO[i, h] . O[i, h], one wave per (row, head)
__global__ __launch_bounds__(kBwThreads) void k_bwd_delta(BwArgs a, int odt, int gdt) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t pair = (int64_t)blockIdx.x * kBwWaves + threadIdx.x / kWave;
  if (pair >= (int64_t)a.L.n_q * a.q.h) return;
  const int i = (int)(pair / a.q.h), h = (int)(pair % a.q.h);
  const int D = a.v.d;
  float acc = 0.f;
  const void* gp = gdt == CSA_BF16 ? (const void*)elem_ptr<__bf16>(a.dout, i, h)
                                   : (const void*)elem_ptr<float>(a.dout, i, h);
  const void* op = odt == CSA_BF16 ? (const void*)elem_ptr<__bf16>(a.o, i, h)
                                   : (const void*)elem_ptr<float>(a.o, i, h);
  if (D % 8 == 0 && ((reinterpret_cast<uintptr_t>(gp) | reinterpret_cast<uintptr_t>(op)) & 15) == 0) {
    // 8 consecutive elements a lane per step, 16-byte loads (wave-uniform branch)
    for (int e = 8 * lane; e < D; e += 8 * kWave) {
      float g[8], o[8];
      if (gdt == CSA_BF16) load8(static_cast<const __bf16*>(gp) + e, g);
      else load8(static_cast<const float*>(gp) + e, g);
      if (odt == CSA_BF16) load8(static_cast<const __bf16*>(op) + e, o);
      else load8(static_cast<const float*>(op) + e, o);
#pragma unroll
      for (int t = 0; t < 8; ++t) acc = fmaf(g[t], o[t], acc);
    }
  } else {
    for (int d = lane; d < D; d += kWave) acc = fmaf(ld(a.dout, gdt, i, h, d), ld(a.o, odt, i, h, d), acc);
  }
  acc = wave_sum(acc);
  if (lane == 0) a.delta[pair] = acc;
}

// Per-list entry counts of each wave's index rows.
__global__ __launch_bounds__(kBwThreads) void k_bwd_hist(BwArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int r = blockIdx.x * kBwWaves + threadIdx.x / kWave;
  if (r >= a.R) return;
  const int64_t n_rows = (int64_t)a.L.n_q * a.idx_heads;
  const int64_t e0 = (int64_t)r * a.rows_per_range;
  const int64_t e1 = min(n_rows, e0 + a.rows_per_range);
  for (int64_t e = e0; e < e1; ++e) {
    const int i = (int)(e / a.idx_heads), hi = (int)(e % a.idx_heads);
    const RowKeys rk = row_keys(a.L, i);
    const int32_t* slots = a.idx + e * a.idx_width;
    for (int s = lane; s < a.idx_width; s += kWave) {
      const int c = slot_list(a, rk, hi, slots[s]);
      if (c >= 0) atomicAdd(&a.hist[(int64_t)c * a.R + r], 1);
    }
  }
}

// Each wave places its index rows one after another: an index row's entries
// take their positions before the next row's are issued (each position is
// the returned value of the cursor's atomic add, waited for before the store),
// so every list holds ascending index-row ids.
__global__ __launch_bounds__(kBwThreads) void k_bwd_fill(BwArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int r = blockIdx.x * kBwWaves + threadIdx.x / kWave;
  if (r >= a.R) return;
  const int64_t n_rows = (int64_t)a.L.n_q * a.idx_heads;
  const int64_t e0 = (int64_t)r * a.rows_per_range;
  const int64_t e1 = min(n_rows, e0 + a.rows_per_range);
  for (int64_t e = e0; e < e1; ++e) {
    const int i = (int)(e / a.idx_heads), hi = (int)(e % a.idx_heads);
    const RowKeys rk = row_keys(a.L, i);
    const int32_t* slots = a.idx + e * a.idx_width;
    for (int s = lane; s < a.idx_width; s += kWave) {
      const int c = slot_list(a, rk, hi, slots[s]);
      if (c >= 0) {
        const int pos = atomicAdd(&a.hist[(int64_t)c * a.R + r], 1);
        a.entries[pos] = (int32_t)(e * a.idx_width + s);  // flat slot id
      }
    }
    // every cursor update of this index row has returned before the next row's
    // are issued (and the compiler moves no memory access across this point)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
}

// Lists whose counts and cursors one workgroup keeps in LDS (64 KiB), and the
// number of ranges (workgroups) the index rows are cut into on that path.
constexpr int kLdsLists = 16384;
constexpr int kLdsRanges = 512;

// One workgroup per range: its index rows' entry counts per list, counted in
// LDS, then stored into the (zeroed) count table where not zero.
__global__ __launch_bounds__(kBwThreads) void k_bwd_hist_lds(BwArgs a) {
  extern __shared__ int s_cnt[];
  const int r = blockIdx.x;
  for (int c = threadIdx.x; c < a.n_lists; c += kBwThreads) s_cnt[c] = 0;
  __syncthreads();
  const int64_t n_rows = (int64_t)a.L.n_q * a.idx_heads;
  const int64_t e0 = (int64_t)r * a.rows_per_range;
  const int64_t e1 = min(n_rows, e0 + a.rows_per_range);
  for (int64_t e = e0; e < e1; ++e) {
    const int i = (int)(e / a.idx_heads), hi = (int)(e % a.idx_heads);
    const RowKeys rk = row_keys(a.L, i);
    const int32_t* slots = a.idx + e * a.idx_width;
    for (int s = threadIdx.x; s < a.idx_width; s += kBwThreads) {
      const int c = slot_list(a, rk, hi, slots[s]);
      if (c >= 0) atomicAdd(&s_cnt[c], 1);
    }
  }
  __syncthreads();
  for (int c = threadIdx.x; c < a.n_lists; c += kBwThreads) {
    const int v = s_cnt[c];
    if (v) a.hist[(int64_t)c * a.R + r] = v;
  }
}

// One workgroup per range: the cursors of the lists its rows touch come from
// the scanned table into LDS; then its index rows are placed one at a time,
// with a barrier between rows, so every list holds ascending index-row ids
// (within a row, a list's entries are its repeated slots).
__global__ __launch_bounds__(kBwThreads) void k_bwd_fill_lds(BwArgs a) {
  extern __shared__ int s_cur[];
  const int r = blockIdx.x;
  for (int c = threadIdx.x; c < a.n_lists; c += kBwThreads) s_cur[c] = -1;
  __syncthreads();
  const int64_t n_rows = (int64_t)a.L.n_q * a.idx_heads;
  const int64_t e0 = (int64_t)r * a.rows_per_range;
  const int64_t e1 = min(n_rows, e0 + a.rows_per_range);
  for (int64_t e = e0; e < e1; ++e) {  // mark the lists this range touches
    const int i = (int)(e / a.idx_heads), hi = (int)(e % a.idx_heads);
    const RowKeys rk = row_keys(a.L, i);
    const int32_t* slots = a.idx + e * a.idx_width;
    for (int s = threadIdx.x; s < a.idx_width; s += kBwThreads) {
      const int c = slot_list(a, rk, hi, slots[s]);
      if (c >= 0) s_cur[c] = 0;
    }
  }
  __syncthreads();
  for (int c = threadIdx.x; c < a.n_lists; c += kBwThreads)
    if (s_cur[c] == 0) s_cur[c] = a.hist[(int64_t)c * a.R + r];
  __syncthreads();
  for (int64_t e = e0; e < e1; ++e) {
    const int i = (int)(e / a.idx_heads), hi = (int)(e % a.idx_heads);
    const RowKeys rk = row_keys(a.L, i);
    const int32_t* slots = a.idx + e * a.idx_width;
    for (int s = threadIdx.x; s < a.idx_width; s += kBwThreads) {
      const int c = slot_list(a, rk, hi, slots[s]);
      if (c >= 0) a.entries[atomicAdd(&s_cur[c], 1)] = (int32_t)(e * a.idx_width + s);
    }
    __syncthreads();  // this row's positions are taken before the next row's
  }
}

// The range's entries in flat order (index row * width + slot): entry f of row
// e = f / width, slot f % width, and its list (-1 when it selects no permitted
// key).
__device__ __forceinline__ int entry_list(const BwArgs& a, int64_t f) {
  const int64_t e = f / a.idx_width;
  const int i = (int)(e / a.idx_heads), hi = (int)(e % a.idx_heads);
  return slot_list(a, row_keys(a.L, i), hi, a.idx[f]);
}

// Narrow index rows: one workgroup per range over its entries in flat order,
// counted in LDS, then stored into the (zeroed) count table where not zero.
__global__ __launch_bounds__(kBwThreads) void k_bwd_hist_flat(BwArgs a) {
  extern __shared__ int s_cnt[];
  const int r = blockIdx.x;
  for (int c = threadIdx.x; c < a.n_lists; c += kBwThreads) s_cnt[c] = 0;
  __syncthreads();
  const int64_t n_rows = (int64_t)a.L.n_q * a.idx_heads;
  const int64_t f0 = (int64_t)r * a.rows_per_range * a.idx_width;
  const int64_t f1 = min(n_rows, (int64_t)(r + 1) * a.rows_per_range) * a.idx_width;
  for (int64_t f = f0 + threadIdx.x; f < f1; f += kBwThreads) {
    const int c = entry_list(a, f);
    if (c >= 0) atomicAdd(&s_cnt[c], 1);
  }
  __syncthreads();
  for (int c = threadIdx.x; c < a.n_lists; c += kBwThreads) {
    const int v = s_cnt[c];
    if (v) a.hist[(int64_t)c * a.R + r] = v;
  }
}

// One workgroup per range: the cursors of the lists its entries touch come from
// the scanned table into LDS; then the entries are placed kBwThreads at a time in
// flat order. Within a batch an entry's place is its list's cursor plus the number
// of earlier entries of the batch in the same list, so every list holds ascending
// flat slot ids; the cursors then advance by the batch's counts.
__global__ __launch_bounds__(kBwThreads) void k_bwd_fill_flat(BwArgs a) {
  extern __shared__ int s_cur[];
  __shared__ int s_c[kBwThreads];
  const int r = blockIdx.x;
  for (int c = threadIdx.x; c < a.n_lists; c += kBwThreads) s_cur[c] = -1;
  __syncthreads();
  const int64_t n_rows = (int64_t)a.L.n_q * a.idx_heads;
  const int64_t f0 = (int64_t)r * a.rows_per_range * a.idx_width;
  const int64_t f1 = min(n_rows, (int64_t)(r + 1) * a.rows_per_range) * a.idx_width;
  for (int64_t f = f0 + threadIdx.x; f < f1; f += kBwThreads) {  // mark the touched lists
    const int c = entry_list(a, f);
    if (c >= 0) s_cur[c] = 0;
  }
  __syncthreads();
  for (int c = threadIdx.x; c < a.n_lists; c += kBwThreads)
    if (s_cur[c] == 0) s_cur[c] = a.hist[(int64_t)c * a.R + r];
  __syncthreads();
  for (int64_t fb = f0; fb < f1; fb += kBwThreads) {
    const int64_t f = fb + threadIdx.x;
    const int c = f < f1 ? entry_list(a, f) : -1;
    s_c[threadIdx.x] = c;
    __syncthreads();
    if (c >= 0) {
      int rank = 0;
      for (int t = 0; t < (int)threadIdx.x; ++t) rank += s_c[t] == c;
      a.entries[s_cur[c] + rank] = (int32_t)f;
    }
    __syncthreads();  // every cursor read before any advance
    if (c >= 0) atomicAdd(&s_cur[c], 1);
    __syncthreads();
  }
}

// ---- exclusive scan of hist (n_hist elements) ---------------------------------
constexpr int kScanPer = 4;                       // elements per thread
constexpr int kScanTile = kBwThreads * kScanPer;  // elements per workgroup

__device__ int wg_exclusive_scan(int x, int* s_wave, int* total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  int incl = x;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += y;
  }
  if (lane == kWave - 1) s_wave[wave] = incl;
  __syncthreads();
  int before = 0, all = 0;
  for (int w = 0; w < kBwWaves; ++w) {
    if (w < wave) before += s_wave[w];
    all += s_wave[w];
  }
  __syncthreads();
  *total = all;
  return before + incl - x;
}

__global__ __launch_bounds__(kBwThreads) void k_scan_tiles(int32_t* x, int64_t n,
                                                           int32_t* totals) {
  __shared__ int s_wave[kBwWaves];
  const int64_t base = (int64_t)blockIdx.x * kScanTile + (int64_t)threadIdx.x * kScanPer;
  int v[kScanPer], sum = 0;
#pragma unroll
  for (int j = 0; j < kScanPer; ++j) {
    v[j] = base + j < n ? x[base + j] : 0;
    sum += v[j];
  }
  int total;
  int run = wg_exclusive_scan(sum, s_wave, &total);
#pragma unroll
  for (int j = 0; j < kScanPer; ++j) {
    if (base + j < n) x[base + j] = run;
    run += v[j];
  }
  if (threadIdx.x == 0) totals[blockIdx.x] = total;
}

// One workgroup: exclusive scan of the tile totals in place; grand total at [n].
__global__ __launch_bounds__(kBwThreads) void k_scan_totals(int32_t* totals, int n) {
  __shared__ int s_wave[kBwWaves];
  int carry = 0;
  for (int b = 0; b < n; b += kBwThreads) {
    const int t = b + threadIdx.x;
    const int v = t < n ? totals[t] : 0;
    int total;
    const int ex = wg_exclusive_scan(v, s_wave, &total);
    if (t < n) totals[t] = carry + ex;
    carry += total;
  }
  if (threadIdx.x == 0) totals[n] = carry;
}

// Adds each tile's offset; writes each list's first entry (and the end).
__global__ __launch_bounds__(kBwThreads) void k_scan_add(BwArgs a) {
  const int64_t base = (int64_t)blockIdx.x * kScanTile;
  const int off = a.totals[blockIdx.x];
  for (int j = threadIdx.x; j < kScanTile; j += kBwThreads) {
    const int64_t t = base + j;
    if (t >= a.n_hist) break;
    const int v = a.hist[t] + off;
    a.hist[t] = v;
    if (t % a.R == 0) a.list_off[t / a.R] = v;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    const int n_tiles = (int)((a.n_hist + kScanTile - 1) / kScanTile);
    a.list_off[a.n_lists] = a.totals[n_tiles];
  }
}

// ---- dq: one wave per (row, head) -------------------------------------------------
// Keys are visited 64 at a time, one per lane: the lane computes the logit and
// dO . v of its key, then the wave adds scale * dx_j * k_j over the 64 keys
// with lanes over the key dimensions.
template <typename T>
__global__ __launch_bounds__(kBwThreads) void k_bwd_dq(BwArgs a, int gdt) {
  __shared__ float s_q[kBwWaves][kMaxDq];
  __shared__ float s_do[kBwWaves][kMaxDvB];
  __shared__ float s_dx[kBwWaves][kWave];
  __shared__ int s_key[kBwWaves][kWave];
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t pair = (int64_t)blockIdx.x * kBwWaves + wave;
  const int hq = a.q.h;
  if (pair >= (int64_t)a.L.n_q * hq) return;
  const int i = (int)(pair / hq), h = (int)(pair % hq);
  const int g = h / (hq / a.k.h);
  const int dqk = a.q.d, dv = a.v.d;
  for (int d = lane; d < dqk; d += kWave) s_q[wave][d] = to_f32(elem_ptr<T>(a.q, i, h)[d]);
  for (int d = lane; d < dv; d += kWave) s_do[wave][d] = ld(a.dout, gdt, i, h, d);
  __builtin_amdgcn_wave_barrier();
  const float lse2 = a.lse[pair] * kLog2e;
  const float D = a.delta[pair];
  float acc[kDqL];
#pragma unroll
  for (int t = 0; t < kDqL; ++t) acc[t] = 0.f;
  const RowKeys r = row_keys(a.L, i);

  auto fold = [&](int key) {  // key < 0: none
    float dx = 0.f;
    if (key >= 0 && lse2 > -INFINITY) {
      const T* kp = elem_ptr<T>(a.k, key, g);
      const T* vp = elem_ptr<T>(a.v, key, g);
      float x = 0.f, dp = 0.f;
      for (int d = 0; d < dqk; d += 8) {
        float kx[8];
        load8(kp + d, kx);
#pragma unroll
        for (int t = 0; t < 8; ++t) x = fmaf(s_q[wave][d + t], kx[t], x);
      }
      for (int d = 0; d < dv; d += 8) {
        float vx[8];
        load8(vp + d, vx);
#pragma unroll
        for (int t = 0; t < 8; ++t) dp = fmaf(s_do[wave][d + t], vx[t], dp);
      }
      const float p = exp2f(x * a.scale_log2 - lse2);
      dx = p * (dp - D);
    }
    s_dx[wave][lane] = dx;
    s_key[wave][lane] = key;
    __builtin_amdgcn_wave_barrier();
    for (int t = 0; t < kWave; ++t) {
      const int kt = s_key[wave][t];
      if (kt < 0) continue;
      const float w = s_dx[wave][t] * a.scale;
      const T* kp = elem_ptr<T>(a.k, kt, g);
#pragma unroll
      for (int u = 0; u < kDqL; ++u) {
        const int d = lane + u * kWave;
        if (d < dqk) acc[u] = fmaf(w, to_f32(kp[d]), acc[u]);
      }
    }
    __builtin_amdgcn_wave_barrier();
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
  float* out = a.dq + pair * dqk;
#pragma unroll
  for (int u = 0; u < kDqL; ++u) {
    const int d = lane + u * kWave;
    if (d < dqk) out[d] = acc[u];
  }
}

// ---- dk, dv: one wave per (key, key head) -------------------------------------------
// The wave walks its list (ascending index rows); each entry brings one query
// head (per-head index rows) or the G query heads of the key head (shared index
// rows).  64 (row, head) items at a time, one per lane: the lane computes its
// item's dx and P; then the wave adds them into dk, dv with lanes over dims.
template <typename T>
__global__ __launch_bounds__(kBwThreads) void k_bwd_dkdv(BwArgs a, int gdt) {
  __shared__ float s_k[kBwWaves][kMaxDq];
  __shared__ float s_v[kBwWaves][kMaxDvB];
  __shared__ float s_dx[kBwWaves][kWave];
  __shared__ float s_p[kBwWaves][kWave];
  __shared__ int s_item[kBwWaves][kWave];
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t kp_id = (int64_t)blockIdx.x * kBwWaves + wave;
  const int hkv = a.k.h;
  if (kp_id >= (int64_t)a.L.n_kv * hkv) return;
  const int j = (int)(kp_id / hkv), g = (int)(kp_id % hkv);
  const int hq = a.q.h, G = hq / hkv;
  const int dqk = a.q.d, dv = a.v.d;
  for (int d = lane; d < dqk; d += kWave) s_k[wave][d] = to_f32(elem_ptr<T>(a.k, j, g)[d]);
  for (int d = lane; d < dv; d += kWave) s_v[wave][d] = to_f32(elem_ptr<T>(a.v, j, g)[d]);
  __builtin_amdgcn_wave_barrier();

  // the list of key j for key head g
  const int gsel = a.idx_heads == 1 ? 0 : g;
  int list;
  if (a.mode == CSA_SEL_TOKEN) {
    list = gsel * a.L.n_kv + j;
  } else {
    int lo = 0, hi = a.L.n_seq - 1;  // sequence of key j: last s with cu[s] <= j
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.L.cu[mid] <= j) lo = mid; else hi = mid - 1;
    }
    list = gsel * a.n_blocks + a.bt.blk_off[lo] + (j - a.L.cu[lo]) / a.block_size;
  }
  const int e0 = a.list_off[list], e1 = a.list_off[list + 1];
  const int per_entry = a.idx_heads == 1 ? G : 1;
  const int64_t n_items = (int64_t)(e1 - e0) * per_entry;

  float ak[kDqL], av[kDvL];
#pragma unroll
  for (int t = 0; t < kDqL; ++t) ak[t] = 0.f;
#pragma unroll
  for (int t = 0; t < kDvL; ++t) av[t] = 0.f;

  for (int64_t base = 0; base < n_items; base += kWave) {
    const int64_t it = base + lane;
    float dx = 0.f, p = 0.f;
    int item = -1;  // i * hq + h
    if (it < n_items) {
      const int e = a.entries[e0 + (int)(it / per_entry)] / a.idx_width;  // index row
      const int i = e / a.idx_heads;
      const int h = a.idx_heads == 1 ? g * G + (int)(it % per_entry) : e % a.idx_heads;
      const RowKeys r = row_keys(a.L, i);
      const int64_t pair = (int64_t)i * hq + h;
      const float lse2 = a.lse[pair] * kLog2e;
      // block lists hold the whole block: keys past the row's position are masked
      if (j <= r.hi && lse2 > -INFINITY) {
        const T* qp = elem_ptr<T>(a.q, i, h);
        float x = 0.f, dp = 0.f;
        for (int d = 0; d < dqk; d += 8) {
          float qx[8];
          load8(qp + d, qx);
#pragma unroll
          for (int t = 0; t < 8; ++t) x = fmaf(qx[t], s_k[wave][d + t], x);
        }
        for (int d = 0; d < dv; d += 8) {
          float gx[8];
          if (gdt == CSA_BF16) load8(elem_ptr<__bf16>(a.dout, i, h) + d, gx);
          else load8(elem_ptr<float>(a.dout, i, h) + d, gx);
#pragma unroll
          for (int t = 0; t < 8; ++t) dp = fmaf(gx[t], s_v[wave][d + t], dp);
        }
        p = exp2f(x * a.scale_log2 - lse2);
        dx = p * (dp - a.delta[pair]);
        item = (int)pair;
      }
    }
    s_dx[wave][lane] = dx * a.scale;
    s_p[wave][lane] = p;
    s_item[wave][lane] = item;
    __builtin_amdgcn_wave_barrier();
    for (int t = 0; t < kWave; ++t) {
      const int pt = s_item[wave][t];
      if (pt < 0) continue;
      const int i = pt / hq, h = pt % hq;
      const float wk = s_dx[wave][t], wv = s_p[wave][t];
      const T* qp = elem_ptr<T>(a.q, i, h);
#pragma unroll
      for (int u = 0; u < kDqL; ++u) {
        const int d = lane + u * kWave;
        if (d < dqk) ak[u] = fmaf(wk, to_f32(qp[d]), ak[u]);
      }
#pragma unroll
      for (int u = 0; u < kDvL; ++u) {
        const int d = lane + u * kWave;
        if (d < dv) av[u] = fmaf(wv, ld(a.dout, gdt, i, h, d), av[u]);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
  float* ok = a.dk + kp_id * dqk;
  float* ov = a.dv + kp_id * dv;
#pragma unroll
  for (int u = 0; u < kDqL; ++u) {
    const int d = lane + u * kWave;
    if (d < dqk) ok[d] = ak[u];
  }
#pragma unroll
  for (int u = 0; u < kDvL; ++u) {
    const int d = lane + u * kWave;
    if (d < dv) ov[d] = av[u];
  }
}

struct BwLayout {
  int n_lists, R, rows_per_range, n_tiles;
  int64_t n_hist, n_entries;
  bool lds_lists;      // counts and cursors in LDS, one workgroup per range
  bool mfma;           // block mode on the matrix cores
  int64_t max_tiles;   // its dQ chunks
  int64_t n_part;      // its dQ partials (floats)
  int64_t n_info;      // its entry records
  int64_t n_dout16;    // its bf16 dO copy (elements)
  bool tok;            // token mode on the matrix cores
  int wpad;
  int64_t n_ds;        // its dS' and P per slot (bf16, each)
  int64_t n_ck, n_cv;  // its per-slot contributions (bf16)
};

BwLayout bw_layout(int n_q, int n_kv, int n_blocks, int mode, int dtype, int hq, int hkv,
                   int dqk, int dv, int idx_heads, int idx_width, int block_size) {
  BwLayout b;
  const int64_t chunks = mode == CSA_SEL_TOKEN ? n_kv : n_blocks;
  b.n_lists = (int)((idx_heads == 1 ? 1 : hkv) * chunks);
  const int64_t n_rows = (int64_t)n_q * idx_heads;
  // ranges: one per wave, enough to fill the chip, the count table within 2^24; or,
  // with the counts in LDS, one per workgroup, kLdsRanges of them
  b.lds_lists = b.n_lists <= kLdsLists;
  int64_t R = std::max<int64_t>(1, std::min<int64_t>((1 << 24) / std::max(1, b.n_lists),
                                                     (n_rows + 3) / 4));
  R = std::min<int64_t>(R, 1 << 16);
  if (b.lds_lists) R = std::max<int64_t>(1, std::min<int64_t>(kLdsRanges, n_rows));
  b.rows_per_range = (int)std::max<int64_t>(1, (n_rows + R - 1) / R);
  b.R = (int)std::max<int64_t>(1, (n_rows + b.rows_per_range - 1) / b.rows_per_range);
  b.n_hist = (int64_t)b.n_lists * b.R;
  b.n_tiles = (int)((b.n_hist + kScanTile - 1) / kScanTile);
  b.n_entries = n_rows * idx_width;
  b.mfma = attn_bwd_block_mfma_supported(mode, dtype, dqk, dv, hq, idx_heads, block_size,
                                         b.n_lists, b.n_entries);
  b.max_tiles = b.mfma ? attn_bwd_block_mfma_max_tiles(b.n_entries, b.n_lists) : 0;
  b.n_part = b.mfma ? b.n_entries * dqk : 0;
  b.n_info = b.mfma ? b.n_entries + 128 : 0;
  b.n_dout16 = b.mfma ? (int64_t)n_q * hq * dqk : 0;
  b.tok = attn_bwd_token_mfma_supported(mode, dtype, dqk, dv, hq, hkv, idx_heads, idx_width);
  b.wpad = b.tok ? attn_bwd_token_wpad(idx_width) : 0;
  b.n_ds = b.tok ? (int64_t)n_q * hq * b.wpad : 0;
  b.n_ck = b.tok ? (int64_t)n_q * idx_width * hkv * dqk : 0;
  b.n_cv = b.tok ? (int64_t)n_q * idx_width * hkv * dv : 0;
  if (b.tok) b.n_dout16 = (int64_t)n_q * hq * dv;
  return b;
}

struct BwWs {
  float* delta;
  BlockTable bt;
  int32_t *hist, *list_off, *totals, *entries;
  float* dq_part;
  int2* tiles;
  int32_t* n_tiles;
  BwEntryInfo* info;
  __bf16* dout16;
  __bf16 *ds, *pb, *ck, *cv;
};

BwWs carve_bw(void* base, const BwLayout& b, int n_q, int hq, int n_seq, int n_blocks,
              size_t* used) {
  Carver c(base);
  BwWs w;
  w.delta = c.take<float>((size_t)n_q * hq);
  w.bt.blk_off = c.take<int32_t>(n_seq + 1);
  w.bt.blocks = c.take<int2>(std::max(1, n_blocks));
  w.bt.blk_seq = c.take<int32_t>(std::max(1, n_blocks));
  w.hist = c.take<int32_t>(b.n_hist);
  w.list_off = c.take<int32_t>(b.n_lists + 1);
  w.totals = c.take<int32_t>(b.n_tiles + 1);
  w.entries = c.take<int32_t>(std::max<int64_t>(1, b.n_entries));
  w.dq_part = c.take<float>(b.n_part);
  w.tiles = c.take<int2>(b.max_tiles);
  w.n_tiles = c.take<int32_t>(b.mfma ? 1 : 0);
  w.info = c.take<BwEntryInfo>(b.n_info);
  w.dout16 = c.take<__bf16>(b.n_dout16);
  w.ds = c.take<__bf16>(b.n_ds);
  w.pb = c.take<__bf16>(b.n_ds);
  w.ck = c.take<__bf16>(b.n_ck);
  w.cv = c.take<__bf16>(b.n_cv);
  if (used) *used = c.used;
  return w;
}

unsigned grid_for(int64_t items, int per_block) {
  return (unsigned)((items + per_block - 1) / per_block);
}

}  // namespace

size_t attn_bwd_ws_bytes(int n_q, int n_kv, int n_seq, int n_blocks, int mode, int dtype, int hq,
                         int hkv, int dqk, int dv, int idx_heads, int idx_width, int block_size) {
  const BwLayout b = bw_layout(n_q, n_kv, n_blocks, mode, dtype, hq, hkv, dqk, dv, idx_heads,
                               idx_width, block_size);
  size_t used = 0;
  carve_bw(nullptr, b, n_q, hq, n_seq, n_blocks, &used);
  return align_up(used, 256);
}

const char* attn_bwd_kernel_family(int n_q, int n_kv, int n_blocks, int mode, int dtype, int hq,
                                   int hkv, int dqk, int dv, int idx_heads, int idx_width,
                                   int block_size) {
  const BwLayout b = bw_layout(n_q, n_kv, n_blocks, mode, dtype, hq, hkv, dqk, dv, idx_heads,
                               idx_width, block_size);
  return b.mfma ? "block_mfma" : b.tok ? "token_mfma" : "generic";
}

hipError_t launch_attn_backward(const AttnBwdArgs& x, hipStream_t stream) {
  BwArgs a;
  a.q = x.q;
  a.k = x.k;
  a.v = x.v;
  a.o = x.o;
  a.dout = x.dout;
  a.L = x.L;
  a.mode = x.mode;
  a.idx_heads = x.idx_heads;
  a.idx_width = x.idx_width;
  a.block_size = x.block_size;
  a.n_blocks = x.n_blocks;
  a.idx = x.idx;
  a.lse = x.lse;
  a.scale = x.scale;
  a.scale_log2 = x.scale * kLog2e;
  a.dq = x.dq;
  a.dk = x.dk;
  a.dv = x.dv;
  const BwLayout b = bw_layout(x.L.n_q, x.L.n_kv, x.n_blocks, x.mode, x.dtype, x.q.h, x.k.h,
                               x.q.d, x.v.d, x.idx_heads, x.idx_width, x.block_size);
  BwWs w = carve_bw(x.ws, b, x.L.n_q, x.q.h, x.L.n_seq, x.n_blocks, nullptr);
  a.delta = w.delta;
  a.bt = w.bt;
  a.hist = w.hist;
  a.list_off = w.list_off;
  a.totals = w.totals;
  a.entries = w.entries;
  a.n_lists = b.n_lists;
  a.R = b.R;
  a.rows_per_range = b.rows_per_range;
  a.n_hist = b.n_hist;
  hipError_t e;
  const int64_t pairs = (int64_t)x.L.n_q * x.q.h;
  const int64_t kpairs = (int64_t)x.L.n_kv * x.k.h;
  if (x.mode == CSA_SEL_BLOCK && x.n_blocks > 0) {
    e = launch_block_table(x.L.cu, x.L.n_seq, x.block_size, x.n_blocks, w.bt, nullptr, 0, stream);
    if (e != hipSuccess) return e;
  }
  if (b.n_hist > 0) {
    hipLaunchKernelGGL(k_fill_i32, dim3(std::min<int64_t>(4096, grid_for(b.n_hist, 256))),
                       dim3(256), 0, stream, w.hist, b.n_hist, 0);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (pairs > 0) {
    hipLaunchKernelGGL(k_bwd_delta, dim3(grid_for(pairs, kBwWaves)), dim3(kBwThreads), 0,
                       stream, a, x.o_dtype, x.dout_dtype);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // wide index rows: counts and cursors in LDS, one workgroup per range
  const bool lds_lists = b.lds_lists;
  const size_t lds_bytes = (size_t)b.n_lists * sizeof(int);
  if (pairs > 0) {
    if (lds_lists && x.idx_width >= kBwThreads)
      hipLaunchKernelGGL(k_bwd_hist_lds, dim3(b.R), dim3(kBwThreads), lds_bytes, stream, a);
    else if (lds_lists)
      hipLaunchKernelGGL(k_bwd_hist_flat, dim3(b.R), dim3(kBwThreads), lds_bytes, stream, a);
    else
      hipLaunchKernelGGL(k_bwd_hist, dim3(grid_for(b.R, kBwWaves)), dim3(kBwThreads), 0,
                         stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (b.n_tiles > 0) {
    hipLaunchKernelGGL(k_scan_tiles, dim3(b.n_tiles), dim3(kBwThreads), 0, stream, w.hist,
                       b.n_hist, w.totals);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(k_scan_totals, dim3(1), dim3(kBwThreads), 0, stream, w.totals,
                       b.n_tiles);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(k_scan_add, dim3(b.n_tiles), dim3(kBwThreads), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (pairs > 0) {
    if (lds_lists && x.idx_width >= kBwThreads)
      hipLaunchKernelGGL(k_bwd_fill_lds, dim3(b.R), dim3(kBwThreads), lds_bytes, stream, a);
    else if (lds_lists)
      hipLaunchKernelGGL(k_bwd_fill_flat, dim3(b.R), dim3(kBwThreads), lds_bytes, stream, a);
    else
      hipLaunchKernelGGL(k_bwd_fill, dim3(grid_for(b.R, kBwWaves)), dim3(kBwThreads), 0,
                         stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (b.tok) {
    BwTokArgs t;
    t.q = x.q;
    t.k = x.k;
    t.v = x.v;
    t.dout = x.dout;
    t.dout_dtype = x.dout_dtype;
    t.g16 = x.dout;
    t.L = x.L;
    t.idx = x.idx;
    t.idx_width = x.idx_width;
    t.lse = x.lse;
    t.delta = w.delta;
    t.scale = x.scale;
    t.scale_log2 = x.scale * kLog2e;
    t.dq = x.dq;
    t.dk = x.dk;
    t.dv = x.dv;
    t.dout16 = w.dout16;
    t.ds = w.ds;
    t.pb = w.pb;
    t.wpad = b.wpad;
    t.ck = w.ck;
    t.cv = w.cv;
    t.list_off = w.list_off;
    t.entries = w.entries;
    return launch_attn_bwd_token(t, stream);
  }
  if (b.mfma) {
    BwMfmaArgs m;
    m.q = x.q;
    m.k = x.k;
    m.v = x.v;
    m.dout = x.dout;
    m.dout_dtype = x.dout_dtype;
    m.L = x.L;
    m.idx = x.idx;
    m.idx_width = x.idx_width;
    m.block_size = x.block_size;
    m.n_blocks = x.n_blocks;
    m.n_lists = b.n_lists;
    m.n_sub = attn_bwd_block_mfma_subtiles(x.block_size);
    m.bt = w.bt;
    m.list_off = w.list_off;
    m.entries = w.entries;
    m.lse = x.lse;
    m.delta = w.delta;
    m.scale = x.scale;
    m.scale_log2 = x.scale * kLog2e;
    m.dq = x.dq;
    m.dk = x.dk;
    m.dv = x.dv;
    m.dq_part = w.dq_part;
    m.tiles = w.tiles;
    m.n_tiles = w.n_tiles;
    m.max_tiles = b.max_tiles;
    m.max_entries = b.n_entries;
    m.info = w.info;
    m.dout16 = w.dout16;
    m.g16 = x.dout;
    return launch_attn_bwd_block_mfma(m, stream);
  }
  int slot;
  if (pairs > 0) {
    trace_begin(stream, "k_bwd_dq", &slot);
    if (x.dtype == CSA_BF16)
      hipLaunchKernelGGL(k_bwd_dq<__bf16>, dim3(grid_for(pairs, kBwWaves)), dim3(kBwThreads),
                         0, stream, a, x.dout_dtype);
    else
      hipLaunchKernelGGL(k_bwd_dq<float>, dim3(grid_for(pairs, kBwWaves)), dim3(kBwThreads),
                         0, stream, a, x.dout_dtype);
    trace_end(stream, slot);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (kpairs > 0) {
    trace_begin(stream, "k_bwd_dkdv", &slot);
    if (x.dtype == CSA_BF16)
      hipLaunchKernelGGL(k_bwd_dkdv<__bf16>, dim3(grid_for(kpairs, kBwWaves)), dim3(kBwThreads),
                         0, stream, a, x.dout_dtype);
    else
      hipLaunchKernelGGL(k_bwd_dkdv<float>, dim3(grid_for(kpairs, kBwWaves)), dim3(kBwThreads),
                         0, stream, a, x.dout_dtype);
    trace_end(stream, slot);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace csa
