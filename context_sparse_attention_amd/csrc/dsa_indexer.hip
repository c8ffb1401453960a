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
// Kernels:
//   k_dsa_logits_mfma - bf16, D_I in {64, 128}, H_I a multiple of 32 up to 128:
//                  32x32x16 bf16 MFMA over LDS-staged key tiles (below);
//   k_dsa_logits - other cases: one workgroup per (row, 256-key tile): the row's indexer
//                  queries sit in LDS, each thread holds one key in registers
//                  and reduces the 64 heads in fp32;
//   k_dsa_select_reg - persistent, one row at a time per workgroup, rows of up to
//                  kRgSpan aligned positions, the row in registers: a value-range histogram finds the bin of the
//                  k-th largest logit, an exact (value, lower index first) order
//                  resolves that bin, and an index-order compaction writes the
//                  selection (ties to the lower index);
//   k_dsa_select - longer rows: one workgroup per row, row cached in LDS when it
//                  fits: 4-pass 8-bit radix select of the k-th largest logit on
//                  order-preserving uint32 keys, then the same compaction.
#include <algorithm>

#include "common.hpp"
#include "gather.hpp"

namespace csa {

namespace {

constexpr int kLogitThreads = 256;
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

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

constexpr int kLgWaves = 4;                 // query tokens per workgroup (one per wave)
constexpr int kLgThreads = kLgWaves * kWave;
constexpr int kLgKeys = 64;                 // keys per LDS tile
constexpr int kLgChunk = 2048;              // keys per workgroup

// bf16 indexer logits on the matrix cores.  Wave w owns query token
// t0 + w: its H_I x D_I indexer queries sit in registers as the A operand
// (rows = heads), each 64-key ik tile is staged once in LDS for the four
// tokens of the workgroup and read as the B operand (columns = keys), so the
// 32x32 accumulator gives a lane one key column and 16 heads per M tile; the
// ReLU and head weights are applied in-lane and the two lane halves are added.
// Only permitted keys [lo_i, pos_i] are written.
template <int DI, int MT>
__global__ __launch_bounds__(kLgThreads, 2) void k_dsa_logits_mfma(View iq, View ik,
                                                                   const float* __restrict__ w,
                                                                   int64_t w_stride, DevLayout L,
                                                                   float* __restrict__ logits) {
  // key tiles [kLgKeys][DI + 8]: pitch 4 mod 32 banks, so eight consecutive rows
  // read at one column (the B operand reads) cover all 32 banks once
  constexpr int KP = DI + 8;
  __shared__ __bf16 s_k[2][kLgKeys * KP];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // uniform: scalar branches
  const int half = lane >> 5;
  const int t0 = blockIdx.x * kLgWaves;
  const int row = t0 + wave;
  int lo = 0, hi = -1;
  if (row < L.n_q) {
    const RowKeys r = row_keys(L, row);
    if (r.valid) {
      lo = r.lo;
      hi = r.hi;
    }
  }
  // key range of the workgroup: the union of its tokens' ranges, cut to this chunk
  __shared__ int s_lo, s_hi;
  if (threadIdx.x == 0) {
    s_lo = INT32_MAX;
    s_hi = -1;
  }
  __syncthreads();
  if (lane == 0 && hi >= lo) {
    atomicMin(&s_lo, lo);
    atomicMax(&s_hi, hi);
  }
  __syncthreads();
  const int k_begin = max(s_lo, blockIdx.y * kLgChunk);
  const int k_end = min(s_hi + 1, (blockIdx.y + 1) * kLgChunk);
  if (k_begin >= k_end) return;  // whole workgroup

  constexpr int KS = DI / 16;
  bf16x8 a[MT][KS];
  float wr[MT][16];
  const int rowc = row < L.n_q ? row : t0;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const __bf16* qp = elem_ptr<__bf16>(iq, rowc, mt * 32 + (lane & 31));
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      a[mt][ks] = *reinterpret_cast<const bf16x8*>(qp + 16 * ks + 8 * half);
#pragma unroll
    for (int j = 0; j < 16; ++j)
      wr[mt][j] = w[(int64_t)rowc * w_stride + mt * 32 + 8 * (j >> 2) + 4 * half + (j & 3)];
  }

  // Tile gather: chunk c (1 KiB) of a tile is issued by wave c % kLgWaves; lane
  // l of chunk c fills 16-byte slot 64 c + l, i.e. unit (slot % kU) of row
  // (slot / kU); pad slots re-read unit 0.  Rows past k_end repeat the last key.
  constexpr int kU = KP / 8;
  constexpr int kChunks = kLgKeys * kU / 64;
  constexpr int kPer = (kChunks + kLgWaves - 1) / kLgWaves;
  static_assert(kLgKeys * kU % 64 == 0, "tiles must be whole KiBs");
  uint32_t goff[kPer];
  auto offsets = [&](int rows) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int slot = (wave + kLgWaves * j) * 64 + lane;
      const int r = min(slot / kU, rows - 1);
      const int u = slot % kU;
      goff[j] = (uint32_t)((r * ik.stride_n + (u < DI / 8 ? u : 0) * 8) * (int64_t)sizeof(__bf16));
    }
  };
  auto issue = [&](int key0, int buf) {
    const char* base = reinterpret_cast<const char*>(elem_ptr<__bf16>(ik, key0, 0));
    const uint32_t l0 = lds_addr(&s_k[buf][0]);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int c = wave + kLgWaves * j;
      if (c < kChunks) gather16(goff[j], base, __builtin_amdgcn_readfirstlane(l0 + c * 1024));
    }
  };
  const int n_kt = (k_end - k_begin + kLgKeys - 1) / kLgKeys;
  offsets(min(kLgKeys, k_end - k_begin));
  issue(k_begin, 0);
  wait_gathers();
  __syncthreads();
  for (int kt = 0; kt < n_kt; ++kt) {
    const int buf = kt & 1;
    const int key0 = k_begin + kt * kLgKeys;
    if (kt + 1 < n_kt) {
      const int next = key0 + kLgKeys;
      if (k_end - next < kLgKeys) offsets(k_end - next);
      issue(next, buf ^ 1);  // lands while this tile is computed
    }
    if (hi >= lo && key0 <= hi) {
#pragma unroll
      for (int nt = 0; nt < kLgKeys / 32; ++nt) {
        const int r = nt * 32 + (lane & 31);
        const __bf16* kp = &s_k[buf][r * KP + 8 * half];
        f32x16 acc[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x16{};
        bf16x8 bq[3];
        bq[0] = *reinterpret_cast<const bf16x8*>(kp);
        if (KS > 1) bq[1] = *reinterpret_cast<const bf16x8*>(kp + 16);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          if (ks + 2 < KS) bq[(ks + 2) % 3] = *reinterpret_cast<const bf16x8*>(kp + 16 * (ks + 2));
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mt][ks], bq[ks % 3], acc[mt], 0, 0, 0);
        }
        // ReLU as a signed max on the bit pattern: negative values and -0 become
        // +0, others pass unchanged (one instruction; fmaxf adds a NaN-quieting one)
        float v = 0.f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int j = 0; j < 16; ++j)
            v = fmaf(wr[mt][j], __int_as_float(max(__float_as_int(acc[mt][j]), 0)), v);
        v += __shfl_xor(v, 32, kWave);
        const int key = key0 + r;
        if (half == 0 && key >= lo && key <= hi && key < k_end)
          logits[(int64_t)row * L.n_kv + key] = v;
      }
    }
    wait_gathers();
    __syncthreads();  // the next tile has landed; this buffer is free for reuse
  }
}

constexpr int kSelThreads = 256;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kSelCache = 12288;  // row keys cached in LDS (48 KiB)
constexpr int kSelPer = 8;        // elements per thread in the compaction

// Exclusive prefix sum of one int per thread across a workgroup of NW waves,
// plus the total.
template <int NW>
__device__ inline int sel_excl_scan_n(int x, int* s_wave, int* total) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  int incl = x;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += y;
  }
  if (lane == kWave - 1) s_wave[wave] = incl;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    if (w < wave) before += s_wave[w];
    all += s_wave[w];
  }
  __syncthreads();
  *total = all;
  return before + incl - x;
}

// Exclusive prefix sum of one int per thread across the workgroup, plus the total.
__device__ inline int sel_excl_scan(int x, int* s_wave, int* total) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  int incl = x;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += y;
  }
  if (lane == kWave - 1) s_wave[wave] = incl;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    if (w < wave) before += s_wave[w];
    all += s_wave[w];
  }
  __syncthreads();
  *total = all;
  return before + incl - x;
}

// One workgroup per row.  The row's logits become order-preserving uint32 keys
// (cached in LDS when the row fits); four 8-bit radix passes find the key T of
// the k-th largest logit and how many keys equal to T are taken; a compaction
// in index order then writes every key > T and the lowest-index keys == T.
__global__ __launch_bounds__(kSelThreads) void k_dsa_select(DevLayout L, int topk,
                                                            const float* __restrict__ logits,
                                                            int32_t* __restrict__ idx,
                                                            float* __restrict__ score,
                                                            int span) {
  __shared__ uint32_t s_key[kSelCache];
  __shared__ int s_hist[256];
  __shared__ int s_wave[kSelWaves];
  __shared__ uint32_t s_prefix;
  __shared__ int s_remaining;
  const int i = blockIdx.x;
  const int lane = threadIdx.x & (kWave - 1);
  const RowKeys r = row_keys(L, i);
  const int n = r.valid ? r.hi - r.lo + 1 : 0;
  // rows the register-resident select takes: short ones and those that fit its span
  if (n <= topk || n + (int)(((int64_t)i * L.n_kv + r.lo) & 3) <= span) return;
  const float* row = logits + (int64_t)i * L.n_kv + r.lo;
  int32_t* out = idx + (int64_t)i * topk;
  float* out_s = score ? score + (int64_t)i * topk : nullptr;

  if (n <= topk) {
    for (int t = threadIdx.x; t < topk; t += kSelThreads) {
      out[t] = t < n ? r.lo + t : -1;
      if (out_s) out_s[t] = t < n ? row[t] : -INFINITY;
    }
    return;
  }
  const bool cached = n <= kSelCache;
  if (cached) {
    // eight independent, coalesced loads in flight per thread
    constexpr int kU = 8;
    for (int base = 0; base < n; base += kSelThreads * kU) {
      float x[kU];
#pragma unroll
      for (int j = 0; j < kU; ++j) {
        const int t = base + j * kSelThreads + threadIdx.x;
        x[j] = t < n ? row[t] : 0.f;
      }
#pragma unroll
      for (int j = 0; j < kU; ++j) {
        const int t = base + j * kSelThreads + threadIdx.x;
        if (t < n) s_key[t] = float_key(x[j]);
      }
    }
  }

  uint32_t prefix = 0, mask = 0;
  int remaining = topk;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int b = threadIdx.x; b < 256; b += kSelThreads) s_hist[b] = 0;
    __syncthreads();
    for (int base = 0; base < n; base += kSelThreads) {
      const int t = base + threadIdx.x;
      bool act = false;
      uint32_t dg = 0;
      if (t < n) {
        const uint32_t u = cached ? s_key[t] : float_key(row[t]);
        act = (u & mask) == prefix;
        dg = (u >> shift) & 255u;
      }
      if (shift == 24) {
        // leading bytes of nearby logits coincide: one atomic per distinct digit per wave
        uint64_t pending = __ballot(act);
        while (pending) {
          const int leader = __ffsll((unsigned long long)pending) - 1;
          const uint32_t dl = __shfl(dg, leader, kWave);
          const uint64_t same = __ballot(act && dg == dl);
          if (lane == leader) atomicAdd(&s_hist[dl], __popcll(same));
          pending &= ~same;
          act = act && dg != dl;
        }
      } else if (act) {
        atomicAdd(&s_hist[dg], 1);
      }
    }
    __syncthreads();
    if (threadIdx.x < kWave) {
      // lane l owns digits 255-4l .. 252-4l; find the digit holding the remaining-th key
      int c[4], sum = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c[j] = s_hist[255 - 4 * lane - j];
        sum += c[j];
      }
      int incl = sum;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const int y = __shfl_up(incl, off, kWave);
        if (lane >= off) incl += y;
      }
      int above = incl - sum;
      int found = -1, above_found = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (found < 0 && above + c[j] >= remaining) {
          found = 255 - 4 * lane - j;
          above_found = above;
        }
        above += c[j];
      }
      const uint64_t hit = __ballot(found >= 0);
      const int first = __ffsll((unsigned long long)hit) - 1;
      if (lane == first) {
        s_prefix = prefix | ((uint32_t)found << shift);
        s_remaining = remaining - above_found;
      }
    }
    __syncthreads();
    prefix = s_prefix;
    remaining = s_remaining;
    mask |= 255u << shift;
    __syncthreads();
  }

  // compaction in index order: keys > prefix, then the first `remaining` keys == prefix
  int eq_carry = 0, out_carry = 0;
  for (int base = 0; base < n; base += kSelThreads * kSelPer) {
    const int t0 = base + threadIdx.x * kSelPer;
    uint32_t u[kSelPer];
    int n_eq = 0;
#pragma unroll
    for (int j = 0; j < kSelPer; ++j) {
      const int t = t0 + j;
      u[j] = t < n ? (cached ? s_key[t] : float_key(row[t])) : 0u;
      n_eq += (t < n && u[j] == prefix);
    }
    int eq_total;
    int eq_rank = eq_carry + sel_excl_scan(n_eq, s_wave, &eq_total);
    bool sel[kSelPer];
    int n_sel = 0;
#pragma unroll
    for (int j = 0; j < kSelPer; ++j) {
      const int t = t0 + j;
      const bool eq = t < n && u[j] == prefix;
      sel[j] = t < n && (u[j] > prefix || (eq && eq_rank < remaining));
      eq_rank += eq;
      n_sel += sel[j];
    }
    int sel_total;
    int slot = out_carry + sel_excl_scan(n_sel, s_wave, &sel_total);
#pragma unroll
    for (int j = 0; j < kSelPer; ++j) {
      if (sel[j]) {
        out[slot] = r.lo + t0 + j;
        if (out_s) out_s[slot] = row[t0 + j];
        ++slot;
      }
    }
    eq_carry += eq_total;
    out_carry += sel_total;
  }
}

// ---- register-resident select ----------------------------------------------
//
// One workgroup per row, the row held in registers (float4 groups, coalesced).
// 1. min / max of the row and a monotone map of value to one of kRgBins bins,
//    bin(x) = min(trunc(max(fma(x, s, o), -1)), kRgBins - 1), s = kRgBins / (max - min):
//    a higher bin holds strictly larger values, equal values share a bin.
// 2. LDS histogram; the bin T holding the k-th largest value and the count of
//    values in higher bins.
// 3. One pass counts, per (group, wave), the values in bins above T and
//    collects the values of bin T as composite keys (value key, then lower
//    index first); the bin of a value is recomputed with the same instructions,
//    so it is the one the histogram counted.  The (k - above)-th largest composite (v*, i*) is found by pairwise
//    ranking, or by an 8-bit radix select re-reading the row when T holds more
//    than kRgCand values (mass ties, e.g. a constant row).
// 4. The selection is {e : x_e > v* or (x_e == v* and e <= i*)} (just x_e >= v*
//    when no value equal to v* is left out); it is written in index order, each
//    lane's offset taken from wave ballots.
// Non-finite logits are never selected (a row with fewer than k finite logits
// is padded with -1).
constexpr int kRgThreads = 512;
constexpr int kRgWaves = kRgThreads / kWave;
constexpr int kRgPer4 = 8;                                     // float4 groups per thread
constexpr int kRgSpan = kRgThreads * 4 * kRgPer4;              // aligned positions of a row
constexpr int kRgBins = 2048;
constexpr int kRgCand = 1024;
constexpr int kRgSlots = kRgWaves * kRgPer4;                   // (group j, wave) counters

__device__ __forceinline__ int rg_bin(float x, float s, float o) {
  const float t = fmaxf(fmaf(x, s, o), -1.0f);  // NaN -> -1
  return min((int)t, kRgBins - 1);
}

__device__ __forceinline__ float rg_key_float(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

__device__ inline uint64_t rg_composite(float x, int e) {
  return ((uint64_t)float_key(x) << 32) | (uint64_t)(0xffffffffu - (uint32_t)e);
}

// One workgroup per row; the row is loaded from memory straight into registers.
__global__ __launch_bounds__(kRgThreads, 6) void k_dsa_select_reg(DevLayout L, int topk,
                                                                  const float* __restrict__ logits,
                                                                  int32_t* __restrict__ idx,
                                                                  float* __restrict__ score) {
  __shared__ uint64_t s_hc[(kRgBins + 2) / 2];  // histogram, then candidates, then the output
  __shared__ float s_red[2][kRgWaves];
  __shared__ int s_wave[kRgWaves];
  __shared__ int s_cnt[kRgSlots];    // selected per (j, wave), index j * kRgWaves + wave
  __shared__ int s_base[kRgSlots];   // exclusive prefix of s_cnt in index order
  __shared__ int s_bin, s_above, s_ncand, s_rem, s_straddle;
  __shared__ uint64_t s_cstar, s_prefix;
  int* const s_hist = reinterpret_cast<int*>(s_hc);  // [kRgBins + 1], entry 0 counts nothing
  uint64_t* const s_cand = s_hc;                      // [kRgCand], after the histogram is read
  static_assert(kRgCand <= (kRgBins + 2) / 2, "candidates alias the histogram");

  const int i = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  const RowKeys r = row_keys(L, i);
  const int n = r.valid ? r.hi - r.lo + 1 : 0;
  const int lo = r.lo;
  const int64_t g0 = (int64_t)i * L.n_kv + lo;
  // element e of the row is aligned position e + sh; group q = tid + kRgThreads * j
  // of this thread holds positions 4q .. 4q+3
  const int sh = (int)(g0 & 3);
  if (n > topk && n + sh > kRgSpan) return;  // rows longer than the registers: k_dsa_select
  int32_t* out = idx + (int64_t)i * topk;
  float* out_s = score ? score + (int64_t)i * topk : nullptr;
  if (n <= topk) {
    for (int t = tid; t < topk; t += kRgThreads) {
      out[t] = t < n ? lo + t : -1;
      if (out_s) out_s[t] = t < n ? logits[g0 + t] : -INFINITY;
    }
    return;
  }
  const int n4 = (n + sh + 3) >> 2;
  const int e0 = 4 * tid - sh;  // element of (j, c) = e0 + 4 * kRgThreads * j + c
  float x[kRgPer4][4];
  {
    const float4* base4 = reinterpret_cast<const float4*>(logits + (g0 - sh));
#pragma unroll
    for (int j = 0; j < kRgPer4; ++j) {
      const int q = tid + kRgThreads * j;
      float4 v = make_float4(NAN, NAN, NAN, NAN);
      if (q < n4) v = base4[q];
      x[j][0] = v.x; x[j][1] = v.y; x[j][2] = v.z; x[j][3] = v.w;
    }
  }
  // positions outside the row (the first sh of group 0, the tail of the last
  // group) become NaN; written per thread so that no per-element index stays live
  if (tid == 0) {
#pragma unroll
    for (int c = 0; c < 3; ++c)
      if (c < sh) x[0][c] = NAN;
  }
  if (tid == (n4 - 1) % kRgThreads) {
    const int jl = (n4 - 1) / kRgThreads;
    const int cl = n + sh - 4 * (n4 - 1);  // elements of the last group inside the row
#pragma unroll
    for (int j = 0; j < kRgPer4; ++j)
      if (j == jl) {
#pragma unroll
        for (int c = 1; c < 4; ++c)
          if (c >= cl) x[j][c] = NAN;
      }
  }

  float mx = -INFINITY, mn = INFINITY;
#pragma unroll
  for (int j = 0; j < kRgPer4; ++j)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      mx = fmaxf(mx, x[j][c]);
      mn = fminf(mn, x[j][c]);
    }
  mx = wave_max(mx);
  mn = -wave_max(-mn);
  if (__builtin_expect(mx == INFINITY || mn == -INFINITY, 0)) {
    // infinite logits are never selected either: make them NaN (rare, per wave)
    mx = -INFINITY;
    mn = INFINITY;
#pragma unroll
    for (int j = 0; j < kRgPer4; ++j)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if (fabsf(x[j][c]) == INFINITY) x[j][c] = NAN;
        mx = fmaxf(mx, x[j][c]);
        mn = fminf(mn, x[j][c]);
      }
    mx = wave_max(mx);
    mn = -wave_max(-mn);
  }
  for (int b = tid; b <= kRgBins; b += kRgThreads) s_hist[b] = 0;
  if (tid < kRgSlots) s_cnt[tid] = 0;
  if (lane == 0) {
    s_red[0][wave] = mx;
    s_red[1][wave] = mn;
  }
  if (tid == 0) {  // defaults that only non-finite logits leave in place
    s_ncand = 0;
    s_cstar = 0;
    s_prefix = 0;
    s_rem = 1;
    s_bin = -1;
    s_above = 0;
    s_straddle = 1;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kRgWaves; ++w) {
    mx = fmaxf(mx, s_red[0][w]);
    mn = fminf(mn, s_red[1][w]);
  }
  const float range = mx - mn;
  const bool spread = range > 0.f && range <= 3.0e38f;
  const float bs = spread ? (float)kRgBins / range : 0.f;
  const float bo = spread ? -mn * bs : 0.f;

  // groups j with kRgThreads * j >= n4 hold no element of the row in any thread
  const int jn = (n4 + kRgThreads - 1) / kRgThreads;
#pragma unroll
  for (int j = 0; j < kRgPer4; ++j)
    if (j < jn) {
#pragma unroll
      for (int c = 0; c < 4; ++c) atomicAdd(&s_hist[rg_bin(x[j][c], bs, bo) + 1], 1);
    }
  __syncthreads();

  // threshold bin: thread t owns bins kRgBins-1-4t .. kRgBins-4-4t (from the top)
  {
    int cnt[4], sum = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      cnt[j] = s_hist[kRgBins - 4 * tid - j];
      sum += cnt[j];
    }
    int total;
    int above = sel_excl_scan_n<kRgWaves>(sum, s_wave, &total);
    if (above < topk && above + sum >= topk) {
      int T = 0, ab = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (above < topk && above + cnt[j] >= topk) {
          T = kRgBins - 1 - 4 * tid - j;
          ab = above;
        }
        above += cnt[j];
      }
      s_bin = T;
      s_above = ab;
    }
  }
  __syncthreads();
  const int T = s_bin;  // -1: fewer than k finite logits, all of them are taken
  const int rem = topk - s_above;
  const int nT = T >= 0 ? s_hist[T + 1] : 0;

  // counts of bins above T per (j, wave); the values of bin T become candidates
  // (T = -1: every finite value counts).  The map's parameters pass through an
  // empty asm so that the histogram's bins are recomputed here rather than kept
  // live in registers; the values, and so the bins, are the same.
  float bs2 = bs, bo2 = bo;
  asm volatile("" : "+v"(bs2), "+v"(bo2));
#pragma unroll
  for (int j = 0; j < kRgPer4; ++j) {
    if (j < jn) {
      int above = 0;
      bool any = false;
      int b[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        b[c] = rg_bin(x[j][c], bs2, bo2);
        above += __popcll(__ballot(b[c] > T));
        any |= b[c] == T;
      }
      if (lane == 0) s_cnt[j * kRgWaves + wave] += above;
      if (nT <= kRgCand && __ballot(any)) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          if (b[c] == T) {
            const int slot = atomicAdd(&s_ncand, 1);
            if (slot < kRgCand) s_cand[slot] = rg_composite(x[j][c], e0 + 4 * kRgThreads * j + c);
          }
        }
      }
    }
  }
  __syncthreads();

  // (j, wave) slot of element e: q = (e + sh) / 4 = tid' + kRgThreads * j
  auto slot_of = [&](int e) {
    const int q = (e + sh) >> 2;
    return (q / kRgThreads) * kRgWaves + (q % kRgThreads) / kWave;
  };
  if (T >= 0 && nT <= kRgCand) {
    for (int a = tid; a < nT; a += kRgThreads) {
      const uint64_t ca = s_cand[a];
      int rank = 0, tie_below = 0;
      for (int b = 0; b < nT; ++b) {
        const uint64_t cb = s_cand[b];
        rank += cb > ca;
        tie_below += (cb >> 32) == (ca >> 32) && cb < ca;
      }
      if (rank < rem) atomicAdd(&s_cnt[slot_of((int)(0xffffffffu - (uint32_t)ca))], 1);
      if (rank == rem - 1) {
        s_cstar = ca;
        s_straddle = tie_below > 0;  // an equal value with a higher index is left out
      }
    }
    __syncthreads();
  } else if (T >= 0) {
    // mass ties in bin T: radix select of the rem-th largest composite, 8 bits a
    // pass, re-reading the row from memory each pass
    const float* row = logits + g0;
    uint64_t prefix = 0, mask = 0;
    int remaining = rem;
    for (int shift = 56; shift >= 0; shift -= 8) {
      for (int b = tid; b < 256; b += kRgThreads) s_hist[b] = 0;
      __syncthreads();
      for (int e = tid; e < n; e += kRgThreads) {
        const float v = row[e];
        if (rg_bin(v, bs, bo) == T) {
          const uint64_t u = rg_composite(v, e);
          if ((u & mask) == prefix) atomicAdd(&s_hist[(int)((u >> shift) & 255u)], 1);
        }
      }
      __syncthreads();
      if (tid < kWave) {
        int cnt[4], sum = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          cnt[j] = s_hist[255 - 4 * lane - j];
          sum += cnt[j];
        }
        int incl = sum;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
          const int y = __shfl_up(incl, off, kWave);
          if (lane >= off) incl += y;
        }
        int above = incl - sum;
        if (above < remaining && above + sum >= remaining) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (above < remaining && above + cnt[j] >= remaining) {
              s_prefix = prefix | ((uint64_t)(255 - 4 * lane - j) << shift);
              s_rem = remaining - above;
            }
            above += cnt[j];
          }
        }
      }
      __syncthreads();
      prefix = s_prefix;
      remaining = s_rem;
      mask |= (uint64_t)255u << shift;
      __syncthreads();
    }
    if (tid == 0) s_cstar = prefix;  // s_straddle stays 1: the exact predicate
    for (int e = tid; e < n; e += kRgThreads) {
      const float v = row[e];
      if (rg_bin(v, bs, bo) == T && rg_composite(v, e) >= prefix) atomicAdd(&s_cnt[slot_of(e)], 1);
    }
    __syncthreads();
  }
  // exclusive prefix of the counts in index order (j, then wave)
  if (tid < kWave) {
    const int a0 = 2 * lane < kRgSlots ? s_cnt[2 * lane] : 0;
    const int a1 = 2 * lane + 1 < kRgSlots ? s_cnt[2 * lane + 1] : 0;
    int incl = a0 + a1;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int y = __shfl_up(incl, off, kWave);
      if (lane >= off) incl += y;
    }
    if (2 * lane < kRgSlots) s_base[2 * lane] = incl - a0 - a1;
    if (2 * lane + 1 < kRgSlots) s_base[2 * lane + 1] = incl - a1;
    if (lane == kWave - 1) s_wave[0] = incl;
  }
  __syncthreads();
  const uint64_t cstar = s_cstar;
  const float vstar = T >= 0 ? rg_key_float((uint32_t)(cstar >> 32)) : -INFINITY;
  const int istar = T >= 0 ? (int)(0xffffffffu - (uint32_t)cstar) : -1;
  const int total = s_wave[0];

  // the indices are gathered in LDS (the histogram's space) and written out
  // coalesced when the selection fits there
  int* const s_stage = s_hist;
  const bool stage = topk <= 2 * ((kRgBins + 2) / 2);
  auto place = [&](auto sel_of) {
#pragma unroll
    for (int j = 0; j < kRgPer4; ++j) {
      if (j < jn) {
        const int ej = e0 + 4 * kRgThreads * j;
        bool sel[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) sel[c] = sel_of(x[j][c], ej + c);
        int slot = s_base[j * kRgWaves + wave];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint64_t m = __ballot(sel[c]);
          slot = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                           __builtin_amdgcn_mbcnt_lo((uint32_t)m, (uint32_t)slot));
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          if (sel[c] && slot < topk) {
            if (stage) s_stage[slot] = lo + ej + c;
            else out[slot] = lo + ej + c;
            if (out_s) out_s[slot] = x[j][c];
          }
          slot += sel[c];
        }
      }
    }
  };
  if (T >= 0 && !s_straddle) {
    place([&](float v, int) { return v >= vstar; });
  } else {
    place([&](float v, int e) { return v > vstar || (v == vstar && e <= istar); });
  }
  if (stage) {
    __syncthreads();
    for (int t = tid; t < topk; t += kRgThreads) out[t] = t < total ? s_stage[t] : -1;
    if (out_s)
      for (int t = total + tid; t < topk; t += kRgThreads) out_s[t] = -INFINITY;
  } else {
    for (int t = total + tid; t < topk; t += kRgThreads) {
      out[t] = -1;
      if (out_s) out_s[t] = -INFINITY;
    }
  }
}

template <typename T>
hipError_t launch_typed(const DsaArgs& a, hipStream_t stream) {
  float* logits = static_cast<float*>(a.ws);
  if (a.L.n_q == 0) return hipSuccess;
  const int hi = a.iq.h, di = a.iq.d;
  const bool mfma = a.dtype == CSA_BF16 && (di == 64 || di == 128) && hi % 32 == 0 && hi <= 128;
  int slot;
  trace_begin(stream, mfma ? "k_dsa_logits_mfma" : "k_dsa_logits", &slot);
  if (mfma && a.L.n_kv > 0) {
    const dim3 grid((a.L.n_q + kLgWaves - 1) / kLgWaves, (a.L.n_kv + kLgChunk - 1) / kLgChunk);
    const dim3 block(kLgThreads);
#define CSA_LG(DI, MT) \
  hipLaunchKernelGGL((k_dsa_logits_mfma<DI, MT>), grid, block, 0, stream, a.iq, a.ik, a.w, \
                     a.w_stride, a.L, logits)
    if (di == 64) {
      if (hi == 32) CSA_LG(64, 1); else if (hi == 64) CSA_LG(64, 2);
      else if (hi == 96) CSA_LG(64, 3); else CSA_LG(64, 4);
    } else {
      if (hi == 32) CSA_LG(128, 1); else if (hi == 64) CSA_LG(128, 2);
      else if (hi == 96) CSA_LG(128, 3); else CSA_LG(128, 4);
    }
#undef CSA_LG
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  } else {
    const int tiles = (a.L.n_kv + kLogitThreads - 1) / kLogitThreads;
    if (tiles > 0) {
      hipLaunchKernelGGL((k_dsa_logits<T, 128>), dim3(tiles, a.L.n_q), dim3(kLogitThreads), 0,
                         stream, a.iq, a.ik, a.w, a.w_stride, a.L, logits);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  trace_end(stream, slot);
  trace_begin(stream, "k_dsa_select_reg", &slot);
  const int grid = a.L.n_q;  // one row per workgroup
  hipLaunchKernelGGL(k_dsa_select_reg, dim3(grid), dim3(kRgThreads), 0, stream, a.L, a.topk,
                     logits, a.idx, a.score);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && a.max_span > kRgSpan) {
    // rows longer than the register-resident span
    hipLaunchKernelGGL(k_dsa_select, dim3(a.L.n_q), dim3(kSelThreads), 0, stream, a.L,
                       a.topk, logits, a.idx, a.score, kRgSpan);
    e = hipGetLastError();
  }
  trace_end(stream, slot);
  return e;
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
