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
//   k_bwbm_info   one 32-byte record per list entry (row offsets, lse, D, pos)
//   k_bwbm_dout16 dO rounded to bf16 when it arrives in fp32
//   k_bwbm_dkdv   one workgroup per (list, 128 keys of the block), one wave per
//                 SIMD owning 32 keys (K, V in registers); the list's entries in
//                 chunks of 128 queries copied global -> LDS a chunk ahead;
//                 S = Q K^T, dP = dO V^T, then dV^T += dO^T P, dK^T += Q^T dS
//                 (no cross-wave sums, no floating-point atomics)
//   k_bwbm_tiles  the (list, first entry) table of 128-entry chunks
//   k_bwbm_dq     one workgroup per chunk: S^T = K Q^T and dP^T = V dO^T over
//                 the block's 64-key subtiles with the queries in registers,
//                 dQ^T += K^T dS^T; one fp32 partial per slot
//   k_bwbm_dq_sum per (row, head): the partials of its permitted block slots
//                 added in slot order
#include <algorithm>

#include "backward.hpp"
#include "gather.hpp"
#include "mfma.hpp"

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
constexpr int kDW = 4;              // waves of a dK/dV workgroup
constexpr int kDT = kDW * kWave;    // its threads
constexpr int kBKW = 32 * kDW;      // its keys (32 per wave)
constexpr float kL2e = 1.4426950408889634f;

// 2^x by the hardware instruction: results below 2^-126 flush to zero (such
// probabilities are below bf16's smallest normal and far below the tolerances)
__device__ __forceinline__ float exp2_raw(float x) { return __builtin_amdgcn_exp2f(x); }

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

// ---- dK, dV ---------------------------------------------------------------------------
// Query and dO rows sit in LDS unpadded (rows of D bf16); 16-byte piece p of row
// r is stored at piece p ^ swz(r).  Both access patterns are then free of bank
// conflicts: 16 consecutive rows read at one piece (the A operands of S and dP),
// and 4 rows x 4 pieces read transposed (the A operands of dV and dK).
template <int D>
__device__ __forceinline__ int swz(int r) {
  if (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  const int x = (r >> 1) & 7;
  return ((x & 1) << 2) | ((x >> 1) & 3);
}

template <int D>
__device__ __forceinline__ int sw_off(int r, int e) {  // element offset of (r, e)
  return r * D + ((((e >> 3) ^ swz<D>(r))) << 3) + (e & 7);
}

template <int D>
__device__ __forceinline__ const bf16x8& sw_row8(const __bf16* t, int r, int e) {
  return *reinterpret_cast<const bf16x8*>(t + sw_off<D>(r, e));
}

// trfrag on the swizzled layout
template <int D>
__device__ __forceinline__ bf16x8 sw_trfrag(const __bf16* t, int r0, int st, int c0, int lane) {
  const int half = lane >> 5, c16 = lane & 15, grp = lane >> 4;
  const int r = r0 + 16 * st + 4 * half + (c16 >> 2);
  const int c = c0 + 16 * (grp & 1) + 4 * (c16 & 3);
  const bf16x4 lo = read_tr(t, sw_off<D>(r, c));
  const bf16x4 hi = read_tr(t, sw_off<D>(r + 8, c));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

template <int D>
struct DkvLds {
  __bf16 rows[2][2][kBQ * D];  // [stage][query, dO][128 rows]
  BwEntryInfo meta[3][kBQ];    // records of chunks m, m + 1, m + 2
};

// One record per list entry, and kBQ padding records past the last (so that a
// chunk's records are always 128 consecutive, in-bounds ones).
__global__ __launch_bounds__(kBT) void k_bwbm_info(BwMfmaArgs a) {
  const int64_t x = (int64_t)blockIdx.x * kBT + threadIdx.x;
  const int total = a.list_off[a.n_lists];
  if (x >= (int64_t)total + kBQ) return;
  BwEntryInfo r;
  r.pad = 0;
  if (x < total) {
    const int pair = a.entries[x] / a.idx_width;
    const int i = pair / a.q.h, h = pair % a.q.h;
    r.qoff = (int64_t)i * a.q.stride_n + (int64_t)h * a.q.stride_h;
    r.goff = (int64_t)i * a.g16.stride_n + (int64_t)h * a.g16.stride_h;
    r.lse2 = a.lse[pair] * kL2e;
    r.dl = a.delta[pair];
    r.pos = a.L.q_pos[i];
  } else {
    r.qoff = 0;
    r.goff = 0;
    r.lse2 = 0.f;
    r.dl = 0.f;
    r.pos = -1;
  }
  a.info[x] = r;
}

// dO rounded to bf16 (fp32 dO only): [n_q, Hq, D] contiguous
__global__ __launch_bounds__(kBT) void k_bwbm_dout16(BwMfmaArgs a, __bf16* g16) {
  const int64_t t = (int64_t)blockIdx.x * kBT + threadIdx.x;
  const int per_row = a.q.d / 8;
  const int64_t pair = t / per_row;
  if (pair >= (int64_t)a.L.n_q * a.q.h) return;
  const int e = (int)(t % per_row) * 8;
  float x[8];
  load8(elem_ptr<float>(a.dout, pair / a.q.h, (int)(pair % a.q.h)) + e, x);
  bf16x8 r;
#pragma unroll
  for (int k = 0; k < 8; ++k) r[k] = (__bf16)x[k];
  *reinterpret_cast<bf16x8*>(g16 + pair * a.q.d + e) = r;
}

// S = Q K^T and dP = dO V^T of 32 queries (rows qb * 32 ..) against the wave's
// 32 keys (B operands kf, vf): rows = queries, columns = keys
template <int D>
__device__ __forceinline__ void dkdv_sdp(const __bf16* sq, const __bf16* sg, int qb, int lane,
                                         const bf16x8 (&kf)[D / 16], const bf16x8 (&vf)[D / 16],
                                         f32x16& sc, f32x16& dp) {
  const int qr = 32 * qb + (lane & 31);
  const int half = lane >> 5;
  sc = f32x16{};
  dp = f32x16{};
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const int e = 16 * ks + 8 * half;
    sc = mfma(sw_row8<D>(sq, qr, e), kf[ks], sc);
    dp = mfma(sw_row8<D>(sg, qr, e), vf[ks], dp);
  }
}

// One workgroup per (list, 128 keys of its block), one wave per SIMD; each wave
// owns 32 keys (its K and V rows stay in registers as the B operands of S and
// dP) and takes every query of each chunk, so no cross-wave sum is needed.
// Chunk m + 1's rows and chunk m + 2's records are copied global -> LDS while
// chunk m is computed; within a chunk the S and dP products of the next 32
// queries are issued before the softmax of the current ones, so the matrix
// cores work while the vector ALUs take the exponentials.
template <int D>
__global__ __launch_bounds__(kDT, 1) void k_bwbm_dkdv(BwMfmaArgs a) {
  using L = DkvLds<D>;
  constexpr int KS = D / 16;       // k-steps over the head dimension
  constexpr int DB = D / 32;       // 32-row blocks of the head dimension
  constexpr int RU = D / 8;        // 16-byte pieces of a row
  constexpr int RPI = kWave / RU;  // rows per 1 KiB copy
  constexpr int NI = kBQ / RPI;    // copies per tensor per chunk
  constexpr int IPW = 2 * NI / kDW;  // copies per wave per chunk
  constexpr int MC = kBQ * (int)sizeof(BwEntryInfo) / 1024;  // 1 KiB copies of records
  static_assert(2 * NI % kDW == 0, "copies split evenly over the waves");
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
  const int k0 = blk.x + st * kBKW + 32 * wave;           // this wave's first key
  const int nk = min(32, blk.y - st * kBKW - 32 * wave);  // its keys (<= 0: none)

  const int e0 = a.list_off[c];
  const int n = a.list_off[c + 1] - e0;
  const int n_chunks = (n + kBQ - 1) / kBQ;
  const __bf16* qbase = static_cast<const __bf16*>(a.q.data);
  const __bf16* gbase = static_cast<const __bf16*>(a.g16.data);

  // the records of chunk m into meta stage m % 3 (wave 0)
  auto copy_meta = [&](int m) {
    if (wave != 0) return;
    const char* src = reinterpret_cast<const char*>(a.info + e0 + m * kBQ);
    const uint32_t dst = lds_addr(&s.meta[m % 3][0]);
#pragma unroll
    for (int u = 0; u < MC; ++u) gather16_addr(src + u * 1024 + lane * 16, dst + u * 1024);
  };
  // the query and dO rows of chunk m into row stage m & 1, from its records
  auto copy_rows = [&](int m) {
    const BwEntryInfo* meta = s.meta[m % 3];
#pragma unroll
    for (int u = 0; u < IPW; ++u) {
      const int ci = wave * IPW + u;  // copy index: tensor ci / NI, piece ci % NI
      const int tn = ci / NI, mm = ci % NI;
      const int r = mm * RPI + lane / RU;
      const int e = (((lane % RU) ^ swz<D>(r))) * 8;  // logical element of this lane's piece
      const __bf16* src = tn == 0 ? qbase + meta[r].qoff : gbase + meta[r].goff;
      gather16_addr(src + e, lds_addr(&s.rows[m & 1][tn][mm * RPI * D]));
    }
  };

  if (n_chunks > 0) {
    copy_meta(0);
    if (n_chunks > 1) copy_meta(1);
    wait_gathers();
    __syncthreads();
    copy_rows(0);
  }

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
  // [head-dim block]: rows = head dims, columns = the wave's keys; held in AGPRs
  // (the compiler otherwise copies them between register files every block)
  f32x16 dkt[DB], dvt[DB];
#pragma unroll
  for (int x = 0; x < DB; ++x) {
    to_agpr(dkt[x], f32x16{});
    to_agpr(dvt[x], f32x16{});
  }
  const int kl = lane & 31;
  // this lane's key, or one past every position when the lane holds no key
  const int key_l = kl < nk ? k0 + kl : 0x7fffffff;

  for (int m = 0; m < n_chunks; ++m) {
    // chunk m's rows and chunk m + 1's records have landed (this wave's copies),
    // and every wave is past chunk m - 1: stage (m + 1) & 1 and meta (m + 2) % 3
    // are free
    wait_gathers();
    __syncthreads();
    if (m + 1 < n_chunks) copy_rows(m + 1);
    if (m + 2 < n_chunks) copy_meta(m + 2);
    if (nk <= 0) continue;
    const __bf16* sq = s.rows[m & 1][0];
    const __bf16* sg = s.rows[m & 1][1];
    const BwEntryInfo* meta = s.meta[m % 3];
    const int nq = min(kBQ, n - m * kBQ);
    const int nqb = (nq + 31) / 32;
    f32x16 sc[2], dp[2];
    dkdv_sdp<D>(sq, sg, 0, lane, kf, vf, sc[0], dp[0]);
#pragma unroll
    for (int qb = 0; qb < kBQ / 32; ++qb) {
      if (qb >= nqb) break;
      if (qb + 1 < nqb) dkdv_sdp<D>(sq, sg, qb + 1, lane, kf, vf, sc[(qb + 1) & 1], dp[(qb + 1) & 1]);
      // P and dS / scale; lane holds key (lane % 32), query rows
      // 32 qb + 8 (j / 4) + 4 half + (j % 4); a masked element (a key past the
      // query's position, a lane without a key, a row past the chunk) takes an
      // exponent of -inf
      bf16x8 pb[2], db[2];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int q = 32 * qb + 8 * (j >> 2) + 4 * half + (j & 3);
        const float l2 = meta[q].lse2, dl = meta[q].dl;
        const int pos = meta[q].pos;
        const bool ok = (key_l <= pos) & (q < nq);
        const float pv = exp2_raw(fmaf(sc[qb & 1][j], a.scale_log2, ok ? -l2 : -INFINITY));
        pb[j >> 3][j & 7] = (__bf16)pv;
        db[j >> 3][j & 7] = (__bf16)(pv * (dp[qb & 1][j] - dl));
      }
      // dV^T += dO^T P, dK^T += Q^T dS (contraction over the 32 queries)
#pragma unroll
      for (int qs = 0; qs < 2; ++qs)
#pragma unroll
        for (int x = 0; x < DB; ++x) {
          mfma_a(dvt[x], sw_trfrag<D>(sg, 32 * qb, qs, 32 * x, lane), pb[qs]);
          mfma_a(dkt[x], sw_trfrag<D>(sq, 32 * qb, qs, 32 * x, lane), db[qs]);
        }
    }
  }
  if (nk <= 0) return;
  fence_a(dkt);
  fence_a(dvt);
  // lane holds key (lane % 32), head dims 32 x + 8 (j / 4) + 4 half + (j % 4)
  if (kl < nk) {
    const int64_t row = ((int64_t)(k0 + kl) * a.k.h + g) * D;
    const float scl = a.scale;  // dK sums dS / scale
#pragma unroll
    for (int x = 0; x < DB; ++x)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int d = 32 * x + 8 * jj + 4 * half;
        *reinterpret_cast<float4*>(a.dk + row + d) =
            make_float4(scl * dkt[x][4 * jj], scl * dkt[x][4 * jj + 1], scl * dkt[x][4 * jj + 2],
                        scl * dkt[x][4 * jj + 3]);
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
    const __bf16* gp = elem_ptr<__bf16>(a.g16, i, h);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[ks] = *reinterpret_cast<const bf16x8*>(qp + 16 * ks + 8 * half);
      gf[ks] = *reinterpret_cast<const bf16x8*>(gp + 16 * ks + 8 * half);
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
      // dS^T / scale; lane holds query column, key rows 32 kb + 8 (j / 4) + 4 half + (j % 4).
      // When the wave's queries are all real and see the 32 keys, nothing is masked.
      bf16x8 db[2];
      if (__all(valid && k0 + 32 * kb + 31 <= pos) && 32 * kb + 32 <= nk) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float pv = exp2_raw(fmaf(sc[j], a.scale_log2, -lse2));
          db[j >> 3][j & 7] = (__bf16)(pv * (dp[j] - dl));
        }
      } else {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int kl = 32 * kb + 8 * (j >> 2) + 4 * half + (j & 3);
          const bool ok = kl < nk && k0 + kl <= pos && lse2 > -INFINITY;
          const float pv = ok ? exp2_raw(fmaf(sc[j], a.scale_log2, -lse2)) : 0.f;
          db[j >> 3][j & 7] = (__bf16)(pv * (dp[j] - dl));
        }
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
    const float scl = a.scale;  // dQ sums dS / scale
#pragma unroll
    for (int x = 0; x < DB; ++x)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        *reinterpret_cast<float4*>(out + 32 * x + 8 * jj + 4 * half) =
            make_float4(scl * dqt[x][4 * jj], scl * dqt[x][4 * jj + 1],
                        scl * dqt[x][4 * jj + 2], scl * dqt[x][4 * jj + 3]);
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
hipError_t launch_d(const BwMfmaArgs& a0, hipStream_t stream) {
  hipError_t e;
  int slot;
  BwMfmaArgs a = a0;
  const int64_t pairs = (int64_t)a.L.n_q * a.q.h;
  if (a.dout_dtype == CSA_BF16) {
    a.g16 = a.dout;
  } else {
    a.g16 = View{a.dout16, (int64_t)a.q.h * D, D, a.L.n_q, a.q.h, D};
    if (pairs > 0) {
      hipLaunchKernelGGL(k_bwbm_dout16, dim3(grid_of(pairs * (D / 8), kBT)), dim3(kBT), 0, stream,
                         a, a.dout16);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  if (a.n_lists > 0) {
    hipLaunchKernelGGL(k_bwbm_info, dim3(grid_of(a.max_entries + kBQ, kBT)), dim3(kBT), 0,
                       stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    trace_begin(stream, "k_bwbm_dkdv", &slot);
    hipLaunchKernelGGL(k_bwbm_dkdv<D>, dim3((unsigned)((int64_t)a.n_lists * a.n_sub)), dim3(kDT),
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
