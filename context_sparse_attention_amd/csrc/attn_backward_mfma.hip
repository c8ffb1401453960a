// Block-mode backward on the matrix cores (bf16 MFMA, gfx950), D in {64, 128}.
//
// The same gradients as the vector-ALU kernels of attn_backward.hip ("Context
// parallel attention: exchange keys and merge softmax globally", masks
// paragraph: the backward returns key and value gradients to their owners;
// Megatron-LM issue #4878, "Strategy: allgather CP mode", backward step), over
// the same per-(key head, block) lists of flat slot ids in ascending order.
// P is recomputed from the forward's lse; P and dS enter the second products
// in bf16 (as P does in the forward), everything accumulates in fp32.
//
//   k_bwbm_dkdv  one workgroup per (list, 64-key subtile of the block): the
//                list's entries in chunks of 128 queries (32 per wave),
//                S = Q K^T and dP = dO V^T with the keys as columns, then
//                dV^T += dO^T P and dK^T += Q^T dS; the four waves' sums are
//                added in wave order at the end (no floating-point atomics)
//   k_bwbm_tiles the (list, first entry) table of 128-entry chunks
//   k_bwbm_dq    one workgroup per chunk: S^T = K Q^T and dP^T = V dO^T over
//                the block's 64-key subtiles with the queries in registers,
//                dQ^T += K^T dS^T; one fp32 partial per slot
//   k_bwbm_dq_sum per (row, head): the partials of its permitted block slots
//                added in slot order
#include <algorithm>

#include "attention.hpp"

namespace csa {

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kBT = 256;            // threads
constexpr int kBW = kBT / kWave;    // waves
constexpr int kBQ = 128;            // queries per chunk (32 per wave)
constexpr int kBK = 64;             // keys per subtile (dQ)
constexpr int kBKW = 128;           // keys per dK/dV workgroup (32 per wave)
constexpr float kL2e = 1.4426950408889634f;

__device__ __forceinline__ f32x16 mfma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// row-major bf16 tile with a pitch of P elements
template <int P>
__device__ __forceinline__ const bf16x8& row8(const __bf16* t, int r, int e) {
  return *reinterpret_cast<const bf16x8*>(t + r * P + e);
}

// transposing read: in a 16-lane group, lane c addressing [r0 + c/4][e0 + 4 (c % 4)]
// receives column e0 + t of rows r0 .. r0 + 3
__device__ __forceinline__ bf16x4 read_tr(const __bf16* base, int elem) {
  typedef __attribute__((address_space(3))) s16x4* lds_ptr;
  typedef __attribute__((address_space(3))) char* lds_bytes;
  const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_ptr)((lds_bytes)(const_cast<__bf16*>(base)) + elem * 2));
  return __builtin_bit_cast(bf16x4, x);
}

// A operand [32 columns x 16 rows] of the transposed tile: row block (16 st + perm)
// starting at row r0, columns c0 .. c0 + 31.  The contraction index is permuted
// like the accumulator rows of the first product (lane half h holds rows
// 16 st + 4 h + {0..3} and 16 st + 8 + 4 h + {0..3}), so that the first product's
// results feed the second as its B operand without moving between lanes.
template <int P>
__device__ __forceinline__ bf16x8 trfrag(const __bf16* t, int r0, int st, int c0, int lane) {
  const int half = lane >> 5, c16 = lane & 15, grp = lane >> 4;
  const int r = r0 + 16 * st + 4 * half + (c16 >> 2);
  const int c = c0 + 16 * (grp & 1) + 4 * (c16 & 3);
  const bf16x4 lo = read_tr(t, r * P + c);
  const bf16x4 hi = read_tr(t, (r + 8) * P + c);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// 8 consecutive elements of a row as bf16 (fp32 inputs rounded to nearest even)
__device__ __forceinline__ bf16x8 ld8bf(const View& t, int dtype, int64_t n, int h, int e) {
  if (dtype == CSA_BF16) return *reinterpret_cast<const bf16x8*>(elem_ptr<__bf16>(t, n, h) + e);
  float x[8];
  load8(elem_ptr<float>(t, n, h) + e, x);
  bf16x8 r;
#pragma unroll
  for (int k = 0; k < 8; ++k) r[k] = (__bf16)x[k];
  return r;
}

// ---- dK, dV ---------------------------------------------------------------------------
template <int D>
struct DkvLds {
  static constexpr int P = D + 8;
  __bf16 q[kBQ * P];
  __bf16 g[kBQ * P];  // dO
  const __bf16* qrow[kBQ];
  const void* grow[kBQ];
  float lse2[kBQ];
  float dl[kBQ];      // D = dO . O
  int pos[kBQ];
};

// Each wave owns 32 keys of the workgroup's 128 (its K and V rows stay in
// registers as the B operands of S and dP) and takes every query of each chunk,
// so no cross-wave sum is needed.
template <int D>
__global__ __launch_bounds__(kBT, 2) void k_bwbm_dkdv(BwMfmaArgs a) {
  using L = DkvLds<D>;
  constexpr int P = L::P;
  constexpr int KS = D / 16;   // k-steps over the head dimension
  constexpr int DB = D / 32;   // 32-row blocks of the head dimension
  constexpr int RU = D / 8;    // 16-byte pieces of a row
  __shared__ L s;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int half = lane >> 5;
  const int n_sub = a.n_sub;
  const int c = blockIdx.x / n_sub;
  const int st = blockIdx.x % n_sub;
  const int g = c / a.n_blocks;
  const int b = c % a.n_blocks;
  const int2 blk = a.bt.blocks[b];
  if (st * kBKW >= blk.y) return;
  const int k0 = blk.x + st * kBKW + 32 * wave;       // this wave's first key
  const int nk = min(32, blk.y - st * kBKW - 32 * wave);  // its keys (<= 0: none)
  const int hq = a.q.h;
  const int W = a.idx_width;

  // B operands: lane holds key (lane % 32); past nk it repeats a key of the block
  // (the last one, or the block's first for a wave without keys), masked below
  bf16x8 kf[KS], vf[KS];
  {
    const int key = nk > 0 ? k0 + min(lane & 31, nk - 1) : blk.x;
    const __bf16* kp = elem_ptr<__bf16>(a.k, key, g);
    const __bf16* vp = elem_ptr<__bf16>(a.v, key, g);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kf[ks] = *reinterpret_cast<const bf16x8*>(kp + 16 * ks + 8 * half);
      vf[ks] = *reinterpret_cast<const bf16x8*>(vp + 16 * ks + 8 * half);
    }
  }
  f32x16 dkt[DB], dvt[DB];  // [head-dim block]: rows = head dims, columns = the wave's keys
#pragma unroll
  for (int x = 0; x < DB; ++x) {
    dkt[x] = f32x16{};
    dvt[x] = f32x16{};
  }

  const int e0 = a.list_off[c];
  const int n = a.list_off[c + 1] - e0;
  for (int base = 0; base < n; base += kBQ) {
    __syncthreads();  // the previous chunk's reads are done
    if (threadIdx.x < kBQ) {
      const int t = threadIdx.x;
      const bool real = base + t < n;
      // rows past the list repeat its first entry of the chunk (masked by pos = -1)
      const int p = a.entries[e0 + base + (real ? t : 0)];
      const int e = p / W;
      const int i = e / hq, h = e % hq;
      const int64_t pair = (int64_t)i * hq + h;
      s.qrow[t] = elem_ptr<__bf16>(a.q, i, h);
      s.grow[t] = a.dout_dtype == CSA_BF16 ? (const void*)elem_ptr<__bf16>(a.dout, i, h)
                                           : (const void*)elem_ptr<float>(a.dout, i, h);
      s.lse2[t] = real ? a.lse[pair] * kL2e : -INFINITY;
      s.dl[t] = real ? a.delta[pair] : 0.f;
      s.pos[t] = real ? a.L.q_pos[i] : -1;
    }
    __syncthreads();
    // query rows, then dO rows: each pass issues all its loads before its stores
    {
      constexpr int PER = kBQ * RU / kBT;
      bf16x8 xv[PER];
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int t = threadIdx.x + u * kBT;
        xv[u] = *reinterpret_cast<const bf16x8*>(s.qrow[t / RU] + (t % RU) * 8);
      }
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int t = threadIdx.x + u * kBT;
        *reinterpret_cast<bf16x8*>(&s.q[(t / RU) * P + (t % RU) * 8]) = xv[u];
      }
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int t = threadIdx.x + u * kBT;
        const int r = t / RU, e = (t % RU) * 8;
        if (a.dout_dtype == CSA_BF16) {
          xv[u] = *reinterpret_cast<const bf16x8*>(static_cast<const __bf16*>(s.grow[r]) + e);
        } else {
          float x[8];
          load8(static_cast<const float*>(s.grow[r]) + e, x);
#pragma unroll
          for (int k = 0; k < 8; ++k) xv[u][k] = (__bf16)x[k];
        }
      }
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int t = threadIdx.x + u * kBT;
        *reinterpret_cast<bf16x8*>(&s.g[(t / RU) * P + (t % RU) * 8]) = xv[u];
      }
    }
    __syncthreads();
    if (nk <= 0) continue;
    const int nq = min(kBQ, n - base);
#pragma unroll 1
    for (int qb = 0; qb < (nq + 31) / 32; ++qb) {
      // S = Q K^T, dP = dO V^T: rows = 32 queries, columns = the wave's 32 keys
      const int qr = 32 * qb + (lane & 31);
      f32x16 sc = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int e = 16 * ks + 8 * half;
        sc = mfma(row8<P>(s.q, qr, e), kf[ks], sc);
        dp = mfma(row8<P>(s.g, qr, e), vf[ks], dp);
      }
      // P and dS; lane holds key (lane % 32), query rows 32 qb + 8 (j / 4) + 4 half + (j % 4)
      bf16x8 pb[2], db[2];
      const int kl = lane & 31;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int q = 32 * qb + 8 * (j >> 2) + 4 * half + (j & 3);
        const float l2 = s.lse2[q];
        const bool ok = kl < nk && k0 + kl <= s.pos[q];
        const float pv = ok ? exp2f(fmaf(sc[j], a.scale_log2, -l2)) : 0.f;
        pb[j >> 3][j & 7] = (__bf16)pv;
        db[j >> 3][j & 7] = (__bf16)(pv * (dp[j] - s.dl[q]) * a.scale);
      }
      // dV^T += dO^T P, dK^T += Q^T dS (contraction over the 32 queries)
#pragma unroll
      for (int qs = 0; qs < 2; ++qs)
#pragma unroll
        for (int x = 0; x < DB; ++x) {
          dvt[x] = mfma(trfrag<P>(s.g, 32 * qb, qs, 32 * x, lane), pb[qs], dvt[x]);
          dkt[x] = mfma(trfrag<P>(s.q, 32 * qb, qs, 32 * x, lane), db[qs], dkt[x]);
        }
    }
  }
  if (nk <= 0) return;
  // lane holds key (lane % 32), head dims 32 x + 8 (j / 4) + 4 half + (j % 4)
  const int kl = lane & 31;
  if (kl < nk) {
    const int64_t row = ((int64_t)(k0 + kl) * a.k.h + g) * D;
#pragma unroll
    for (int x = 0; x < DB; ++x)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int d = 32 * x + 8 * jj + 4 * half;
        *reinterpret_cast<float4*>(a.dk + row + d) =
            make_float4(dkt[x][4 * jj], dkt[x][4 * jj + 1], dkt[x][4 * jj + 2], dkt[x][4 * jj + 3]);
        *reinterpret_cast<float4*>(a.dv + row + d) =
            make_float4(dvt[x][4 * jj], dvt[x][4 * jj + 1], dvt[x][4 * jj + 2], dvt[x][4 * jj + 3]);
      }
  }
}

// ---- chunk table for dQ ---------------------------------------------------------------
// One workgroup: tiles[t] = (list, first entry of the chunk); tiles count in *n_tiles.
__global__ __launch_bounds__(1024) void k_bwbm_tiles(const int32_t* __restrict__ list_off,
                                                     int n_lists, int2* __restrict__ tiles,
                                                     int32_t* __restrict__ n_tiles) {
  __shared__ int s_wave[16];
  __shared__ int s_total;
  int carry = 0;
  for (int b0 = 0; b0 < n_lists; b0 += 1024) {
    const int c = b0 + threadIdx.x;
    int nt = 0;
    if (c < n_lists) nt = (list_off[c + 1] - list_off[c] + kBQ - 1) / kBQ;
    // inclusive scan over the workgroup
    const int lane = threadIdx.x & 63, wave = threadIdx.x / 64;
    int x = nt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off, 64);
      if (lane >= off) x += y;
    }
    if (lane == 63) s_wave[wave] = x;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; ++w) before += s_wave[w];
    if (threadIdx.x == 1023) s_total = before + x;
    const int first = carry + before + x - nt;
    for (int k = 0; k < nt; ++k) tiles[first + k] = make_int2(c, list_off[c] + k * kBQ);
    __syncthreads();
    carry += s_total;
    __syncthreads();
  }
  if (threadIdx.x == 0) *n_tiles = carry;
}

// ---- dQ ---------------------------------------------------------------------------------
template <int D>
struct DqLds {
  static constexpr int P = D + 8;
  __bf16 k[kBK * P];
  __bf16 v[kBK * P];
};

template <int D>
__global__ __launch_bounds__(kBT, 2) void k_bwbm_dq(BwMfmaArgs a) {
  using L = DqLds<D>;
  constexpr int P = L::P;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  __shared__ L s;
  const int t = blockIdx.x;
  if (t >= *a.n_tiles) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int half = lane >> 5;
  const int2 tl = a.tiles[t];
  const int c = tl.x;
  const int g = c / a.n_blocks;
  const int b = c % a.n_blocks;
  const int2 blk = a.bt.blocks[b];
  const int hq = a.q.h;
  const int W = a.idx_width;
  const int list_end = a.list_off[c + 1];
  // this lane's query: B-operand column (lane % 32) of the wave's 32
  const int ent = tl.y + 32 * wave + (lane & 31);
  const bool valid = ent < list_end;
  const int p = a.entries[valid ? ent : tl.y];
  const int e = p / W;
  const int i = e / hq, h = e % hq;
  const int64_t pair = (int64_t)i * hq + h;
  const float lse2 = valid ? a.lse[pair] * kL2e : -INFINITY;
  const float dl = a.delta[pair];
  const int pos = a.L.q_pos[i];
  bf16x8 qf[KS], gf[KS];
  {
    const __bf16* qp = elem_ptr<__bf16>(a.q, i, h);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[ks] = *reinterpret_cast<const bf16x8*>(qp + 16 * ks + 8 * half);
      gf[ks] = ld8bf(a.dout, a.dout_dtype, i, h, 16 * ks + 8 * half);
    }
  }
  f32x16 dqt[DB];  // dQ^T: head-dimension rows, the wave's queries as columns
#pragma unroll
  for (int x = 0; x < DB; ++x) dqt[x] = f32x16{};

  const int nsub = (blk.y + kBK - 1) / kBK;
  for (int st = 0; st < nsub; ++st) {
    const int k0 = blk.x + st * kBK;
    const int nk = min(kBK, blk.y - st * kBK);
    __syncthreads();
    for (int u0 = threadIdx.x; u0 < kBK * (D / 8); u0 += kBT) {
      const int r = u0 / (D / 8), u = u0 % (D / 8);
      const int key = k0 + min(r, nk - 1);
      *reinterpret_cast<bf16x8*>(&s.k[r * P + u * 8]) =
          *reinterpret_cast<const bf16x8*>(elem_ptr<__bf16>(a.k, key, g) + u * 8);
      *reinterpret_cast<bf16x8*>(&s.v[r * P + u * 8]) =
          *reinterpret_cast<const bf16x8*>(elem_ptr<__bf16>(a.v, key, g) + u * 8);
    }
    __syncthreads();
    // S^T = K Q^T, dP^T = V dO^T: rows = 32 keys, columns = the wave's queries
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 sc = f32x16{}, dp = f32x16{};
      const int kr = 32 * kb + (lane & 31);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int el = 16 * ks + 8 * half;
        sc = mfma(row8<P>(s.k, kr, el), qf[ks], sc);
        dp = mfma(row8<P>(s.v, kr, el), gf[ks], dp);
      }
      // dS^T; lane holds query column, key rows 32 kb + 8 (j / 4) + 4 half + (j % 4)
      bf16x8 db[2];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int kl = 32 * kb + 8 * (j >> 2) + 4 * half + (j & 3);
        const bool ok = kl < nk && k0 + kl <= pos && lse2 > -INFINITY;
        const float pv = ok ? exp2f(fmaf(sc[j], a.scale_log2, -lse2)) : 0.f;
        db[j >> 3][j & 7] = (__bf16)(pv * (dp[j] - dl) * a.scale);
      }
      // dQ^T += K^T dS^T over this key block
#pragma unroll
      for (int qs = 0; qs < 2; ++qs)
#pragma unroll
        for (int x = 0; x < DB; ++x)
          dqt[x] = mfma(trfrag<P>(s.k, 32 * kb, qs, 32 * x, lane), db[qs], dqt[x]);
    }
  }
  if (valid) {
    float* out = a.dq_part + (int64_t)p * D;
#pragma unroll
    for (int x = 0; x < DB; ++x)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        *reinterpret_cast<float4*>(out + 32 * x + 8 * jj + 4 * half) =
            make_float4(dqt[x][4 * jj], dqt[x][4 * jj + 1], dqt[x][4 * jj + 2],
                        dqt[x][4 * jj + 3]);
  }
}

// dq[i, h] = the partials of (i, h)'s permitted block slots, added in slot order.
template <int D>
__global__ __launch_bounds__(kBT) void k_bwbm_dq_sum(BwMfmaArgs a) {
  constexpr int kLanes = D / 4;
  const int64_t pair = (int64_t)blockIdx.x * (kBT / kLanes) + threadIdx.x / kLanes;
  if (pair >= (int64_t)a.L.n_q * a.q.h) return;
  const int d4 = (threadIdx.x % kLanes) * 4;
  const int i = (int)(pair / a.q.h);
  const RowKeys r = row_keys(a.L, i);
  const int W = a.idx_width;
  const int32_t* slots = a.idx + pair * W;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (r.valid) {
    for (int sl = 0; sl < W; ++sl) {
      const int s0 = slots[sl];
      if (s0 < r.lo || s0 > r.hi || (s0 - r.lo) % a.block_size) continue;
      const float4 x = *reinterpret_cast<const float4*>(a.dq_part + (pair * W + sl) * D + d4);
      acc.x += x.x;
      acc.y += x.y;
      acc.z += x.z;
      acc.w += x.w;
    }
  }
  *reinterpret_cast<float4*>(a.dq + pair * D + d4) = acc;
}

unsigned grid_of(int64_t items, int per) { return (unsigned)((items + per - 1) / per); }

template <int D>
hipError_t launch_d(const BwMfmaArgs& a, hipStream_t stream) {
  hipError_t e;
  int slot;
  if (a.n_lists > 0) {
    trace_begin(stream, "k_bwbm_dkdv", &slot);
    hipLaunchKernelGGL(k_bwbm_dkdv<D>, dim3((unsigned)((int64_t)a.n_lists * a.n_sub)), dim3(kBT),
                       0, stream, a);
    trace_end(stream, slot);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (a.L.n_q == 0) return hipSuccess;
  hipLaunchKernelGGL(k_bwbm_tiles, dim3(1), dim3(1024), 0, stream, a.list_off, a.n_lists,
                     a.tiles, a.n_tiles);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  trace_begin(stream, "k_bwbm_dq", &slot);
  if (a.max_tiles > 0)
    hipLaunchKernelGGL(k_bwbm_dq<D>, dim3((unsigned)a.max_tiles), dim3(kBT), 0, stream, a);
  trace_end(stream, slot);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t pairs = (int64_t)a.L.n_q * a.q.h;
  hipLaunchKernelGGL(k_bwbm_dq_sum<D>, dim3(grid_of(pairs, kBT / (D / 4))), dim3(kBT), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace

int attn_bwd_block_mfma_subtiles(int block_size) { return (block_size + kBKW - 1) / kBKW; }

int64_t attn_bwd_block_mfma_max_tiles(int64_t n_entries, int64_t n_lists) {
  return n_entries / kBQ + n_lists + 1;
}

bool attn_bwd_block_mfma_supported(int mode, int dtype, int dqk, int dv, int hq, int idx_heads,
                                   int block_size, int64_t n_lists, int64_t n_entries) {
  if (mode != CSA_SEL_BLOCK || dtype != CSA_BF16 || dqk != dv || (dqk != 64 && dqk != 128) ||
      idx_heads != hq || block_size < 1)
    return false;
  // grids within 2^23 workgroups
  return n_lists * attn_bwd_block_mfma_subtiles(block_size) < ((int64_t)1 << 23) &&
         attn_bwd_block_mfma_max_tiles(n_entries, n_lists) < ((int64_t)1 << 23);
}

hipError_t launch_attn_bwd_block_mfma(const BwMfmaArgs& a, hipStream_t stream) {
  if (a.q.d == 64) return launch_d<64>(a, stream);
  return launch_d<128>(a, stream);
}

}  // namespace csa
