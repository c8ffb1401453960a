// MoBA block gating and top-k block selection.
//
// MoBA issue #34 ("Question on Implementing Context Parallelism with MoBA
// Efficient Attention", opening question): each query ranks key blocks by a
// gating score computed from Q x K^T and keeps its top-k blocks; under context
// parallelism the local queries rank blocks of the gathered keys.  The score
// of a block is the query's dot product with the block's mean key (the plain
// reading of "Q x K^T" at block granularity: q . mean(k) = mean(q . k)).
//
// Kernels:
//   k_block_table + k_moba_need - block table and, per packed sequence, the
//                  highest own block of any local row (blocks at or after it
//                  are never candidates, so they are not pooled); for small
//                  shards the pool kernel works both out itself;
//   k_moba_pool  - fp32 block means (and their bf16 high/low split), one
//                  workgroup per (block, key head), coalesced 16-byte loads,
//                  fixed-order LDS reduction (deterministic);
//   k_moba_gate_mfma - bf16: 16 rows x 16 blocks per MFMA, per-row register
//                  top-k (score desc, ties to the lower block), own block
//                  appended, ascending output;
//   k_moba_gate  - fp32 and other shapes: one thread per (row, query head).
#include <float.h>

#include "common.hpp"
#include "block_table.hpp"

namespace csa {

namespace {

constexpr int kPoolThreads = 256;
constexpr int kGateThreads = 256;

struct MobaWs {
  BlockTable bt;
  int32_t* need;    // [n_seq]
  float* mu;        // [n_blocks, hkv*d]
  __bf16* mu_hi;    // [n_blocks, hkv*d]  bf16 split of mu (high part)
  __bf16* mu_lo;    // [n_blocks, hkv*d]  (low part)
};

MobaWs carve_moba(void* base, int n_seq, int n_blocks, int hkv, int d, int block_size) {
  Carver c(base);
  MobaWs w;
  w.bt.blk_off = c.take<int32_t>(n_seq + 1);
  w.bt.blocks = c.take<int2>(n_blocks);
  w.bt.blk_seq = c.take<int32_t>(n_blocks);
  w.need = c.take<int32_t>(n_seq);
  w.mu = c.take<float>((size_t)n_blocks * hkv * d);
  w.mu_hi = c.take<__bf16>((size_t)n_blocks * hkv * d);
  w.mu_lo = c.take<__bf16>((size_t)n_blocks * hkv * d);
  return w;
}

size_t carve_bytes(int n_seq, int n_blocks, int hkv, int d, int block_size) {
  Carver c(nullptr);
  c.take<int32_t>(n_seq + 1);
  c.take<int2>(n_blocks);
  c.take<int32_t>(n_blocks);
  c.take<int32_t>(n_seq);
  c.take<float>((size_t)n_blocks * hkv * d);
  c.take<__bf16>((size_t)n_blocks * hkv * d);
  c.take<__bf16>((size_t)n_blocks * hkv * d);
  return align_up(c.used, 256);
}

// Block table and per-sequence need in one workgroup, for shards of at most
// kPrepRows rows in at most kPrepSeqs sequences (the need is reduced in LDS);
// larger shards are faster with the separate, wide k_moba_need.
constexpr int kPrepSeqs = 4096;
constexpr int kPrepRows = 4096;

__global__ __launch_bounds__(kTableThreads) void k_gate_prep(DevLayout L, int block_size,
                                                             int n_blocks, BlockTable bt,
                                                             int32_t* __restrict__ need) {
  __shared__ int s_need[kPrepSeqs];
  for (int s = threadIdx.x; s < L.n_seq; s += kTableThreads) s_need[s] = 0;
  block_table_wg(L.cu, L.n_seq, block_size, n_blocks, bt);  // ends with a barrier
  for (int i = threadIdx.x; i < L.n_q; i += kTableThreads) {
    const RowKeys r = row_keys(L, i);
    if (r.valid) atomicMax(&s_need[r.seq], bt.blk_off[r.seq] + (r.hi - r.lo) / block_size);
  }
  __syncthreads();
  for (int s = threadIdx.x; s < L.n_seq; s += kTableThreads) need[s] = s_need[s];
}

__global__ void k_moba_need(DevLayout L, int block_size, const int32_t* __restrict__ blk_off,
                            int32_t* __restrict__ need) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  int seq = -1, own = -1;
  if (i < L.n_q) {
    const RowKeys r = row_keys(L, i);
    if (r.valid) {
      seq = r.seq;
      own = blk_off[r.seq] + (r.hi - r.lo) / block_size;
    }
  }
  // rows of one wave are usually in one sequence: one atomic per wave then
  const int seq0 = __shfl(seq, 0, kWave);
  if (__all(seq == seq0)) {
    int m = own;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = max(m, __shfl_xor(m, off, kWave));
    if ((threadIdx.x & (kWave - 1)) == 0 && seq0 >= 0) atomicMax(&need[seq0], m);
  } else if (seq >= 0) {
    atomicMax(&need[seq], own);
  }
}

// One workgroup per (block, key head): D/8 lanes cover a key row with 16-byte
// loads, the other lanes stride over the block's keys, and the partial sums
// are reduced through LDS in a fixed order (deterministic, no atomics, no
// cross-workgroup fences).
// LOCAL (small shards): no table or need kernel runs before; each workgroup
// builds the sequences' block offsets in LDS, finds its block's sequence and
// extent, and checks over the shard's rows whether any row's own block lies
// after it; workgroup 0 writes the block table for the gate kernel.
template <typename T, bool LOCAL>
__global__ __launch_bounds__(kPoolThreads) void k_moba_pool(View k, DevLayout L, int block_size,
                                                            BlockTable bt,
                                                            const int32_t* __restrict__ need,
                                                            float* __restrict__ mu,
                                                            __bf16* __restrict__ mu_hi,
                                                            __bf16* __restrict__ mu_lo) {
  const int b = blockIdx.x / k.h;
  const int g = blockIdx.x % k.h;
  int2 blk;
  if (LOCAL) {
    __shared__ int s_off[kPrepSeqs + 1];
    __shared__ int s_wave[kPoolThreads / kWave];
    __shared__ int s_max[kPoolThreads / kWave];
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    int carry = 0;
    for (int base = 0; base < L.n_seq; base += kPoolThreads) {
      const int s = base + threadIdx.x;
      const int nb = s < L.n_seq ? (L.cu[s + 1] - L.cu[s] + block_size - 1) / block_size : 0;
      int incl = nb;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const int y = __shfl_up(incl, off, kWave);
        if (lane >= off) incl += y;
      }
      if (lane == kWave - 1) s_wave[wave] = incl;
      __syncthreads();
      int before = 0, all = 0;
#pragma unroll
      for (int w = 0; w < kPoolThreads / kWave; ++w) {
        before += w < wave ? s_wave[w] : 0;
        all += s_wave[w];
      }
      if (s < L.n_seq) s_off[s] = carry + before + incl - nb;
      carry += all;
      __syncthreads();
    }
    if (threadIdx.x == 0) s_off[L.n_seq] = carry;
    __syncthreads();
    auto seq_of = [&](int bb) {  // last sequence whose first block is <= bb
      int lo = 0, hi = L.n_seq - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_off[mid] <= bb) lo = mid; else hi = mid - 1;
      }
      return lo;
    };
    if (blockIdx.x == 0) {
      for (int s = threadIdx.x; s <= L.n_seq; s += kPoolThreads) bt.blk_off[s] = s_off[s];
      for (int bb = threadIdx.x; bb < gridDim.x / k.h; bb += kPoolThreads) {
        const int s = seq_of(bb);
        const int start = L.cu[s] + (bb - s_off[s]) * block_size;
        bt.blocks[bb] = make_int2(start, min(block_size, L.cu[s + 1] - start));
        bt.blk_seq[bb] = s;
      }
    }
    const int seq = seq_of(b);
    const int bl = b - s_off[seq];  // block within its sequence
    blk.x = L.cu[seq] + bl * block_size;
    blk.y = min(block_size, L.cu[seq + 1] - blk.x);
    // needed when some row of the sequence has its own block after this one;
    // the rows' sequence ids and positions are read four at a time, all loads
    // of a thread in flight together
    const int lo_s = L.cu[seq], end_s = L.cu[seq + 1];
    int own = -1;
    constexpr int kRowsPer = kPrepRows / kPoolThreads;  // rows of one thread, at most
    static_assert(kRowsPer % 4 == 0, "rows are read in groups of four");
    int4 sq[kRowsPer / 4], ps[kRowsPer / 4];
    const bool vec = (L.n_q & 3) == 0 && ((uintptr_t)L.q_seq & 15) == 0 &&
                     ((uintptr_t)L.q_pos & 15) == 0;
#pragma unroll
    for (int j = 0; j < kRowsPer / 4; ++j) {
      const int i0 = 4 * (threadIdx.x + kPoolThreads * j);
      sq[j] = make_int4(-1, -1, -1, -1);
      ps[j] = make_int4(0, 0, 0, 0);
      if (vec && i0 < L.n_q) {
        sq[j] = *reinterpret_cast<const int4*>(L.q_seq + i0);
        ps[j] = *reinterpret_cast<const int4*>(L.q_pos + i0);
      } else if (!vec) {
        int s4[4] = {-1, -1, -1, -1}, p4[4] = {0, 0, 0, 0};
        for (int t = 0; t < 4; ++t)
          if (i0 + t < L.n_q) {
            s4[t] = L.q_seq[i0 + t];
            p4[t] = L.q_pos[i0 + t];
          }
        sq[j] = make_int4(s4[0], s4[1], s4[2], s4[3]);
        ps[j] = make_int4(p4[0], p4[1], p4[2], p4[3]);
      }
    }
    auto take = [&](int s, int p) {
      if (s == seq && p >= lo_s && p < end_s) own = max(own, (p - lo_s) / block_size);
    };
#pragma unroll
    for (int j = 0; j < kRowsPer / 4; ++j) {
      take(sq[j].x, ps[j].x);
      take(sq[j].y, ps[j].y);
      take(sq[j].z, ps[j].z);
      take(sq[j].w, ps[j].w);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) own = max(own, __shfl_xor(own, off, kWave));
    if (lane == 0) s_max[wave] = own;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kPoolThreads / kWave; ++w) own = max(own, s_max[w]);
    if (bl >= own) return;  // never a candidate of any local row
  } else {
    if (b >= need[bt.blk_seq[b]]) return;  // never a candidate of any local row
    blk = bt.blocks[b];
  }
  const int d = k.d;
  const int units = d / 8;                // <= 32
  const int lanes_k = kPoolThreads / units;
  const int u = threadIdx.x % units;
  const int kl = threadIdx.x / units;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  const int t1 = kl < lanes_k ? blk.x + blk.y : 0;  // spare threads add nothing
#pragma unroll 8
  for (int t = blk.x + kl; t < t1; t += lanes_k) {
    float x[8];
    load8(elem_ptr<T>(k, t, g) + u * 8, x);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] += x[j];
  }
  __shared__ float s_red[kPoolThreads * 8];
#pragma unroll
  for (int j = 0; j < 8; ++j) s_red[threadIdx.x * 8 + j] = acc[j];
  __syncthreads();
  const float inv = 1.0f / (float)blk.y;
  const size_t base = ((size_t)b * k.h + g) * d;
  for (int e = threadIdx.x; e < d; e += kPoolThreads) {
    float s = 0.f;
    for (int l = 0; l < lanes_k; ++l) s += s_red[(l * units + e / 8) * 8 + e % 8];
    const float m = s * inv;
    mu[base + e] = m;
    if (mu_hi) {
      // bf16 pair whose sum carries the fp32 mean to ~2^-17 relative
      const __bf16 hi = (__bf16)m;
      mu_hi[base + e] = hi;
      mu_lo[base + e] = (__bf16)(m - (float)hi);
    }
  }
}

// Bitonic sort of (key, val) pairs ascending by key; N a power of two, fully unrolled.
template <int N>
__device__ inline void sort_pairs_asc(int* key, float* val) {
#pragma unroll
  for (int size = 2; size <= N; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const int j = i ^ stride;
        if (j > i) {
          const bool up = ((i & size) == 0);
          const bool swap = up ? (key[i] > key[j]) : (key[i] < key[j]);
          if (swap) {
            const int tk = key[i]; key[i] = key[j]; key[j] = tk;
            const float tv = val[i]; val[i] = val[j]; val[j] = tv;
          }
        }
      }
    }
  }
}

template <typename T, int KMAX>
__global__ __launch_bounds__(kGateThreads) void k_moba_gate(View q, DevLayout L, int hkv,
                                                            int block_size, int topk,
                                                            BlockTable bt,
                                                            const float* __restrict__ mu,
                                                            int32_t* __restrict__ idx,
                                                            float* __restrict__ score) {
  const int64_t pair = (int64_t)blockIdx.x * kGateThreads + threadIdx.x;
  const int hq = q.h;
  if (pair >= (int64_t)L.n_q * hq) return;
  const int i = (int)(pair / hq);
  const int h = (int)(pair % hq);
  const int g = h / (hq / hkv);
  const int width = topk + 1;
  int32_t* out = idx + pair * width;
  float* out_s = score ? score + pair * width : nullptr;

  const RowKeys r = row_keys(L, i);
  if (!r.valid) {
    for (int t = 0; t < width; ++t) {
      out[t] = -1;
      if (out_s) out_s[t] = -INFINITY;
    }
    return;
  }
  const int j_own = (r.hi - r.lo) / block_size;
  const int first = bt.blk_off[r.seq];
  const int own = first + j_own;

  float best_s[KMAX];
  int best_b[KMAX];
#pragma unroll
  for (int t = 0; t < KMAX; ++t) {
    best_s[t] = -INFINITY;
    best_b[t] = INT32_MAX;
  }
  const int d = q.d;
  const T* qp = elem_ptr<T>(q, i, h);
  const int hd = hkv * d;
  for (int c = 0; c < j_own; ++c) {
    const float* m = mu + (size_t)(first + c) * hd + (size_t)g * d;
    float s = 0.f;
    for (int d8 = 0; d8 < d; d8 += 8) {
      float x[8];
      load8(qp + d8, x);
      const float4 m0 = *reinterpret_cast<const float4*>(m + d8);
      const float4 m1 = *reinterpret_cast<const float4*>(m + d8 + 4);
      s = fmaf(x[0], m0.x, s); s = fmaf(x[1], m0.y, s);
      s = fmaf(x[2], m0.z, s); s = fmaf(x[3], m0.w, s);
      s = fmaf(x[4], m1.x, s); s = fmaf(x[5], m1.y, s);
      s = fmaf(x[6], m1.z, s); s = fmaf(x[7], m1.w, s);
    }
    // insert: strictly greater moves ahead, so an equal score keeps the earlier block
    float cs = s;
    int cb = first + c;
#pragma unroll
    for (int t = 0; t < KMAX; ++t) {
      if (t < topk && cs > best_s[t]) {
        const float ts = best_s[t];
        const int tb = best_b[t];
        best_s[t] = cs;
        best_b[t] = cb;
        cs = ts;
        cb = tb;
      }
    }
  }
  // unfilled entries keep the INT32_MAX sentinel and sort last (a NaN score,
  // possible only for non-finite inputs, is never inserted)
  sort_pairs_asc<KMAX>(best_b, best_s);
  int kept = 0;
#pragma unroll
  for (int u = 0; u < KMAX; ++u) {
    if (best_b[u] != INT32_MAX) {
      out[u] = bt.blocks[best_b[u]].x;
      if (out_s) out_s[u] = best_s[u];
      ++kept;
    }
  }
  int t = kept;
  out[t] = bt.blocks[own].x;
  if (out_s) out_s[t] = INFINITY;
  for (++t; t < width; ++t) {
    out[t] = -1;
    if (out_s) out_s[t] = -INFINITY;
  }
}

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr int kGateCols = 64;  // score cells per row and pass: 64 / RG block columns

// bf16 gate on the matrix cores.  One wave scores 16 RG consecutive rows of one
// query head against 16-block column tiles with 16x16x32 bf16 MFMA: the A
// operand is the rows' queries, the B operand the block means split into a
// bf16 high and low part (two products per step, so the score keeps the fp32
// mean to ~2^-17 relative); each B fragment serves the RG row groups.  The
// score chunk goes through LDS; 4 / RG lanes per row each keep a register top
// list over the row's own candidates (blocks of its sequence before its own
// block) in a residue class of the columns, in ascending block order so that
// ties keep the lower block, and the lists are merged by shuffles.
// Four workgroups per CU (128 registers) for the common shapes, so that a
// 32K-row shard's waves are resident at once; wider lists and rows get more.
template <int D, int KMAX>
constexpr int gate_wgs_per_cu() { return (D <= 128 && KMAX <= 4) ? 4 : 2; }

template <int D, int KMAX, int RG>
__global__ __launch_bounds__(kGateThreads, (gate_wgs_per_cu<D, KMAX>())) void k_moba_gate_mfma(
    View q, DevLayout L, int hkv, int block_size, int topk, int n_blocks, BlockTable bt,
    const __bf16* __restrict__ mu_hi, const __bf16* __restrict__ mu_lo,
    int32_t* __restrict__ idx, float* __restrict__ score) {
  static_assert(RG == 1 || RG == 2 || RG == 4, "row groups per wave");
  constexpr int RW = 16 * RG;          // rows per wave
  constexpr int PW = kGateCols / RG;   // block columns per pass
  constexpr int LPR = 4 / RG;          // selection lanes per row
  __shared__ float s_sc[kGateThreads / kWave][RW][PW + 1];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int hq = q.h;
  const int n_rg = (L.n_q + RW - 1) / RW;
  const int wg = blockIdx.x * (kGateThreads / kWave) + wave;
  if (wg >= n_rg * hq) return;  // whole wave
  const int h = wg % hq;
  const int rg = wg / hq;
  const int g = h / (hq / hkv);
  const int rl = lane & 15;
  const int quad = lane >> 4;
  // selection: lane -> row sr of the wave, residue part of the columns
  const int sr = lane & (RW - 1);
  const int part = lane / RW;
  const int row = rg * RW + sr;

  int first = 0, own = -1;
  if (row < L.n_q) {
    const RowKeys r = row_keys(L, row);
    if (r.valid) {
      first = bt.blk_off[r.seq];
      own = first + (r.hi - r.lo) / block_size;
    }
  }
  int col_lo = own >= 0 ? first : INT32_MAX;
  int col_hi = own;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    col_lo = min(col_lo, __shfl_xor(col_lo, off, kWave));
    col_hi = max(col_hi, __shfl_xor(col_hi, off, kWave));
  }

  bf16x8 a[RG][D / 32];
#pragma unroll
  for (int gi = 0; gi < RG; ++gi) {
    const int qr = rg * RW + gi * 16 + rl;
    const __bf16* qp = elem_ptr<__bf16>(q, qr < L.n_q ? qr : 0, h);
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks)
      a[gi][ks] = *reinterpret_cast<const bf16x8*>(qp + 32 * ks + 8 * quad);
  }

  float best_s[KMAX];
  int best_b[KMAX];
#pragma unroll
  for (int t = 0; t < KMAX; ++t) {
    best_s[t] = -INFINITY;
    best_b[t] = INT32_MAX;
  }
  const int hd = hkv * D;
  for (int cb = col_lo; cb < col_hi; cb += PW) {
#pragma unroll
    for (int t = 0; t < PW / 16; ++t) {
      const int c0 = cb + 16 * t;
      if (c0 >= col_hi) break;  // uniform across the wave
      const int blk = min(c0 + rl, n_blocks - 1);
      const __bf16* ph = mu_hi + (size_t)blk * hd + (size_t)g * D + 8 * quad;
      const __bf16* pl = mu_lo + (size_t)blk * hd + (size_t)g * D + 8 * quad;
      f32x4 acc[RG];
#pragma unroll
      for (int gi = 0; gi < RG; ++gi) acc[gi] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) {
        const bf16x8 bh = *reinterpret_cast<const bf16x8*>(ph + 32 * ks);
        const bf16x8 bl = *reinterpret_cast<const bf16x8*>(pl + 32 * ks);
#pragma unroll
        for (int gi = 0; gi < RG; ++gi) {
          acc[gi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[gi][ks], bh, acc[gi], 0, 0, 0);
          acc[gi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[gi][ks], bl, acc[gi], 0, 0, 0);
        }
      }
      // lane holds block c0 + rl for rows 16 gi + 4 quad .. 16 gi + 4 quad + 3
#pragma unroll
      for (int gi = 0; gi < RG; ++gi)
#pragma unroll
        for (int j = 0; j < 4; ++j) s_sc[wave][16 * gi + 4 * quad + j][16 * t + rl] = acc[gi][j];
    }
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
    // lane part p takes the columns c = p (mod LPR) in increasing order: a
    // per-lane top list, descending, ties to the earlier column.  The lane's
    // 16 columns are read together and columns outside the row's candidates
    // become -inf (they never enter the list), so the insertion runs without
    // branches or waits between columns.
    static_assert(PW == 16 * LPR, "16 columns per lane and pass");
    const int n = min(PW, col_hi - cb);
    float v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int c = part + LPR * j;
      const int b = cb + c;
      const float x = s_sc[wave][sr][c];
      v[j] = (c < n && b >= first && b < own) ? x : -INFINITY;
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (LPR * j >= n) break;  // wave-uniform: no lane has a column left
      float cs = v[j];
      int cbk = cb + part + LPR * j;
#pragma unroll
      for (int t = 0; t < KMAX; ++t) {
        const bool take = t < topk && cs > best_s[t];
        const float ts = best_s[t];
        const int tb = best_b[t];
        best_s[t] = take ? cs : ts;
        best_b[t] = take ? cbk : tb;
        cs = take ? ts : cs;
        cbk = take ? tb : cbk;
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
  if (LPR > 1) {
    // merge the lists of each row: topk rounds, each taking the best head
    // (larger score, then smaller block) and popping it from the lane that held it
    float out_s[KMAX];
    int out_b[KMAX];
#pragma unroll
    for (int t = 0; t < KMAX; ++t) {
      float ws = best_s[0];
      int wb = best_b[0];
#pragma unroll
      for (int off = RW; off < kWave; off <<= 1) {
        const float os = __shfl_xor(ws, off, kWave);
        const int ob = __shfl_xor(wb, off, kWave);
        if (os > ws || (os == ws && ob < wb)) {
          ws = os;
          wb = ob;
        }
      }
      out_s[t] = ws;
      out_b[t] = wb;
      if (best_b[0] == wb && wb != INT32_MAX) {
#pragma unroll
        for (int u = 0; u + 1 < KMAX; ++u) {
          best_s[u] = best_s[u + 1];
          best_b[u] = best_b[u + 1];
        }
        best_s[KMAX - 1] = -INFINITY;
        best_b[KMAX - 1] = INT32_MAX;
      }
    }
#pragma unroll
    for (int t = 0; t < KMAX; ++t) {
      const bool keep = t < topk;
      best_s[t] = keep ? out_s[t] : -INFINITY;
      best_b[t] = keep ? out_b[t] : INT32_MAX;
    }
  }
  if (part != 0 || row >= L.n_q) return;
  const int width = topk + 1;
  int32_t* out = idx + ((int64_t)row * hq + h) * width;
  float* out_s = score ? score + ((int64_t)row * hq + h) * width : nullptr;
  if (own < 0) {
    for (int t = 0; t < width; ++t) {
      out[t] = -1;
      if (out_s) out_s[t] = -INFINITY;
    }
    return;
  }
  sort_pairs_asc<KMAX>(best_b, best_s);
  int kept = 0;
#pragma unroll
  for (int u = 0; u < KMAX; ++u) {
    if (best_b[u] != INT32_MAX) {
      out[u] = bt.blocks[best_b[u]].x;
      if (out_s) out_s[u] = best_s[u];
      ++kept;
    }
  }
  int t = kept;
  out[t] = bt.blocks[own].x;
  if (out_s) out_s[t] = INFINITY;
  for (++t; t < width; ++t) {
    out[t] = -1;
    if (out_s) out_s[t] = -INFINITY;
  }
}
// Waves of 64 rows once there are enough of them to fill the chip: each block
// mean fragment then serves four MFMAs.
constexpr int64_t kGateWideWaves = 16384;

template <int D, int KMAX, int RG>
hipError_t launch_gate_rg(const MobaGateArgs& a, const MobaWs& w, hipStream_t stream) {
  const int64_t waves = (int64_t)((a.L.n_q + 16 * RG - 1) / (16 * RG)) * a.q.h;
  const int per_wg = kGateThreads / kWave;
  const int grid = (int)((waves + per_wg - 1) / per_wg);
  hipLaunchKernelGGL((k_moba_gate_mfma<D, KMAX, RG>), dim3(grid), dim3(kGateThreads), 0, stream,
                     a.q, a.L, a.k.h, a.block_size, a.topk, a.n_blocks, w.bt, w.mu_hi,
                     w.mu_lo, a.idx, a.score);
  return hipGetLastError();
}
template <int D, int KMAX>
hipError_t launch_gate_mfma(const MobaGateArgs& a, const MobaWs& w, hipStream_t stream) {
  if ((int64_t)((a.L.n_q + 15) / 16) * a.q.h >= kGateWideWaves)
    return launch_gate_rg<D, KMAX, 4>(a, w, stream);
  return launch_gate_rg<D, KMAX, 1>(a, w, stream);
}

template <int D>
hipError_t launch_gate_mfma_k(const MobaGateArgs& a, const MobaWs& w, hipStream_t stream) {
  if (a.topk <= 4) return launch_gate_mfma<D, 4>(a, w, stream);
  if (a.topk <= 8) return launch_gate_mfma<D, 8>(a, w, stream);
  if (a.topk <= 16) return launch_gate_mfma<D, 16>(a, w, stream);
  return launch_gate_mfma<D, 32>(a, w, stream);
}

template <typename T, int KMAX>
hipError_t launch_gate_k(const MobaGateArgs& a, const MobaWs& w, hipStream_t stream) {
  const int64_t pairs = (int64_t)a.L.n_q * a.q.h;
  const int grid = (int)((pairs + kGateThreads - 1) / kGateThreads);
  hipLaunchKernelGGL((k_moba_gate<T, KMAX>), dim3(grid), dim3(kGateThreads), 0, stream, a.q,
                     a.L, a.k.h, a.block_size, a.topk, w.bt, w.mu, a.idx, a.score);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_typed(const MobaGateArgs& a, hipStream_t stream) {
  const int n_seq = a.L.n_seq;
  MobaWs w = carve_moba(a.ws, n_seq, a.n_blocks, a.k.h, a.k.d, a.block_size);
  hipError_t e;
  const bool local = n_seq <= kPrepSeqs && a.L.n_q <= kPrepRows && a.n_blocks > 0;
  if (local) {
    if (a.L.n_q == 0) return hipSuccess;
  } else if (n_seq <= kPrepSeqs && a.L.n_q <= kPrepRows) {
    hipLaunchKernelGGL(k_gate_prep, dim3(1), dim3(kTableThreads), 0, stream, a.L, a.block_size,
                       a.n_blocks, w.bt, w.need);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (a.L.n_q == 0) return hipSuccess;
  } else {
    e = launch_block_table(a.L.cu, n_seq, a.block_size, a.n_blocks, w.bt, w.need, n_seq,
                           stream);
    if (e != hipSuccess) return e;
    if (a.L.n_q == 0) return hipSuccess;
    hipLaunchKernelGGL(k_moba_need, dim3((a.L.n_q + 255) / 256), dim3(256), 0, stream, a.L,
                       a.block_size, w.bt.blk_off, w.need);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const bool use_mfma = a.dtype == CSA_BF16 && (a.q.d == 64 || a.q.d == 128 || a.q.d == 256);
  if (a.n_blocks > 0) {
    if (local)
      hipLaunchKernelGGL((k_moba_pool<T, true>), dim3(a.n_blocks * a.k.h), dim3(kPoolThreads), 0,
                         stream, a.k, a.L, a.block_size, w.bt, w.need, w.mu,
                         use_mfma ? w.mu_hi : nullptr, use_mfma ? w.mu_lo : nullptr);
    else
      hipLaunchKernelGGL((k_moba_pool<T, false>), dim3(a.n_blocks * a.k.h), dim3(kPoolThreads),
                         0, stream, a.k, a.L, a.block_size, w.bt, w.need, w.mu,
                         use_mfma ? w.mu_hi : nullptr, use_mfma ? w.mu_lo : nullptr);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  int slot;
  trace_begin(stream, use_mfma ? "k_moba_gate_mfma" : "k_moba_gate", &slot);
  if (use_mfma) {
    if (a.q.d == 64) e = launch_gate_mfma_k<64>(a, w, stream);
    else if (a.q.d == 128) e = launch_gate_mfma_k<128>(a, w, stream);
    else e = launch_gate_mfma_k<256>(a, w, stream);
  } else if (a.topk <= 4) {
    e = launch_gate_k<T, 4>(a, w, stream);
  } else if (a.topk <= 8) {
    e = launch_gate_k<T, 8>(a, w, stream);
  } else if (a.topk <= 16) {
    e = launch_gate_k<T, 16>(a, w, stream);
  } else {
    e = launch_gate_k<T, 32>(a, w, stream);
  }
  trace_end(stream, slot);
  return e;
}

}  // namespace

size_t moba_gate_ws_bytes(int n_seq, int n_blocks, int hkv, int d, int block_size) {
  return carve_bytes(n_seq, n_blocks, hkv, d, block_size);
}

hipError_t launch_moba_gate(const MobaGateArgs& a, hipStream_t stream) {
  if (a.dtype == CSA_BF16) return launch_typed<__bf16>(a, stream);
  return launch_typed<float>(a, stream);
}

}  // namespace csa
