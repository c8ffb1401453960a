// Token-mode backward on the matrix cores: one selection per token (shared by
// every query head), bf16, Dqk = 576 and Dv = 512 (absorbed MLA: the value may be
// the key's first 512 columns), 32, 64 or 128 query heads per key head.
//
// "Context parallel attention: exchange keys and merge softmax globally", masks
// paragraph (key and value gradients go back to their owners); Megatron-LM issue
// #4878, "Strategy: allgather CP mode", backward step.  With the forward's lse,
// P = exp(scale q.k - lse) and dS' = P (dP - D), dP = dO.v, D = dO.O:
//
//   dq   = scale sum_slots dS' k          dv_j = sum_(slots holding j) sum_h P dO
//   dk_j = scale sum_(slots holding j) sum_h dS' q
//
//   k_bwtm_ds   per (row, key head): the row's selected keys gathered 32 slots at
//               a time, S^T and dP^T against the heads' q and dO (in registers);
//               dS' and P stored per slot in bf16
//   k_bwtm_dq   the same gathered tiles: dq = scale dS' K
//   k_bwtm_ckv  per (row, key head, 128 slots): each slot's contributions summed
//               over the heads, C_K = dS'^T q and C_V = P^T dO, in bf16
//   k_bwtm_kred per (key, key head): dk, dv = the sums of C_K, C_V over the key's
//               slots, in list order (the lists of attn_backward.hip)
// No floating-point atomics; results are bitwise reproducible.
#include <algorithm>

#include "backward.hpp"
#include "gather.hpp"

namespace csa {

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kTQ = 576;              // key / query width
constexpr int kTV = 512;              // value width
constexpr int kTQC = 32 * kTQ * 2 / 1024;  // 1 KiB copies of a 32-row key tile (36)
constexpr int kTGC = 32 * kTV * 2 / 1024;  // ... of a value tile (32)
constexpr float kL2e = 1.4426950408889634f;

__device__ __forceinline__ float exp2_raw(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ f32x16 mfma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Query rows (1152 bytes) and dO rows (1024 bytes) sit in LDS unpadded, 16-byte
// piece p of row r at p ^ swz(r).  Both access patterns are free of bank
// conflicts: 16 consecutive rows at one piece, and 4 rows x 4 pieces read
// transposed.  (A query row starts at bank 0 or 32 by row parity, so its swap
// works on row pairs; a dO row always starts at bank 0.)
__device__ __forceinline__ int swq(int r) {
  const int x = (r >> 1) & 7;
  return ((x & 1) << 2) | ((x >> 1) & 3);
}
__device__ __forceinline__ int swg(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int offq(int r, int e) {
  return r * kTQ + ((((e >> 3) ^ swq(r))) << 3) + (e & 7);
}
__device__ __forceinline__ int offg(int r, int e) {
  return r * kTV + ((((e >> 3) ^ swg(r))) << 3) + (e & 7);
}

__device__ __forceinline__ bf16x4 read_tr(const __bf16* base, int elem) {
  typedef __attribute__((address_space(3))) s16x4* lds_ptr;
  typedef __attribute__((address_space(3))) char* lds_bytes;
  const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_ptr)((lds_bytes)(const_cast<__bf16*>(base)) + elem * 2));
  return __builtin_bit_cast(bf16x4, x);
}

// ---- preparation --------------------------------------------------------------------------
__global__ void k_bwtm_fill(uint32_t* p, int64_t n) {
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < n;
       t += (int64_t)gridDim.x * blockDim.x)
    p[t] = 0u;
}

__global__ __launch_bounds__(256) void k_bwtm_dout16(BwTokArgs a, __bf16* g16) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t pair = t / (kTV / 8);
  if (pair >= (int64_t)a.L.n_q * a.q.h) return;
  const int e = (int)(t % (kTV / 8)) * 8;
  float x[8];
  load8(elem_ptr<float>(a.dout, pair / a.q.h, (int)(pair % a.q.h)) + e, x);
  bf16x8 r;
#pragma unroll
  for (int k = 0; k < 8; ++k) r[k] = (__bf16)x[k];
  *reinterpret_cast<bf16x8*>(g16 + pair * kTV + e) = r;
}

// ---- dQ -----------------------------------------------------------------------------------
// Two passes over each row's selected keys, 32 slots at a time gathered into LDS
// and shared by the row's query heads of one key head (32 heads per wave):
//   k_bwtm_ds  S^T = K Q^T and dP^T = V dO^T with the heads' Q and dO fragments in
//              registers; dS' = P (dP - D) stored per slot in bf16 (0 for a slot
//              that selects no permitted key)
//   k_bwtm_dq  dQ = scale dS' K with the heads' dQ accumulators in registers
// (one pass would need the Q, dO and dQ fragments of 32 heads at once: 560
// registers, more than a wave has)
constexpr int kDS = 32;       // slots per tile
constexpr int kMaxW = 4096;   // index width whose slots are staged in LDS

template <bool VA>
struct DsLds {
  __bf16 k[2][kDS * kTQ];
  __bf16 v[VA ? 1 : 2][VA ? 8 : kDS * kTV];
  int key[kMaxW];  // the row's slots: key, or -1 when it selects no permitted key
};

struct DqLds {
  __bf16 k[2][kDS * kTQ];
  __bf16 ds[2][4][32 * kDS];  // [stage][head block][head][slot]
  int key[kMaxW];
};

// the row's slots into LDS (permitted key or -1); returns a key every gather may read
__device__ __forceinline__ int stage_slots(const BwTokArgs& a, int i, int* key) {
  const RowKeys r = row_keys(a.L, i);
  for (int t = threadIdx.x; t < a.idx_width; t += blockDim.x) {
    const int k = a.idx[(int64_t)i * a.idx_width + t];
    key[t] = r.valid && k >= r.lo && k <= r.hi ? k : -1;
  }
  return r.valid ? r.lo : 0;
}

// gathers slot tile t's key rows (and value rows when V is not K's prefix) into
// stage st: copies c = wave, wave + NW, ...
template <bool VA>
__device__ __forceinline__ void gather_tile(const BwTokArgs& a, int g, const int* key, int kfb,
                                            int t, __bf16* kt, __bf16* vt, int nw, int wave,
                                            int lane) {
  const __bf16* kb = static_cast<const __bf16*>(a.k.data);
  const __bf16* vb = static_cast<const __bf16*>(a.v.data);
  constexpr int NC = kTQC + (VA ? 0 : kTGC);
  for (int c = wave; c < NC; c += nw) {
    if (c < kTQC) {
      const int byte = 1024 * c + 16 * lane;
      const int r = byte / (kTQ * 2);
      const int pp = (byte % (kTQ * 2)) / 16;
      const int slot = kDS * t + r;
      int k = slot < a.idx_width ? key[slot] : -1;
      k = k < 0 ? kfb : k;
      const __bf16* src = kb + (int64_t)k * a.k.stride_n + (int64_t)g * a.k.stride_h + (pp ^ swq(r)) * 8;
      gather16_addr(src, __builtin_amdgcn_readfirstlane(lds_addr(kt) + 1024 * c));
    } else {
      const int r = c - kTQC;
      const int slot = kDS * t + r;
      int k = slot < a.idx_width ? key[slot] : -1;
      k = k < 0 ? kfb : k;
      const __bf16* src = vb + (int64_t)k * a.v.stride_n + (int64_t)g * a.v.stride_h + (lane ^ swg(r)) * 8;
      gather16_addr(src, __builtin_amdgcn_readfirstlane(lds_addr(vt) + 1024 * r));
    }
  }
}

// Separate value rows: one workgroup per (row, key head); wave w takes query heads
// g G + 32 w .. and forms both S^T and dP^T (the K and V tiles leave no LDS for
// handing P between waves)
__global__ __launch_bounds__(256, 1) void k_bwtm_ds_v(BwTokArgs a) {
  constexpr bool VA = false;
  __shared__ DsLds<VA> s;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int nw = blockDim.x / kWave;
  const int half = lane >> 5;
  const int i = blockIdx.x / a.k.h, g = blockIdx.x % a.k.h;
  const int hq = a.q.h, G = hq / a.k.h;
  const int h = g * G + 32 * wave + (lane & 31);  // this lane's head (B-operand column)
  const int kfb = stage_slots(a, i, s.key);
  __syncthreads();
  const int n_t = (a.idx_width + kDS - 1) / kDS;
  gather_tile<VA>(a, g, s.key, kfb, 0, s.k[0], s.v[0], nw, wave, lane);

  // B operands: Q^T and dO^T fragments of head h
  bf16x8 qf[kTQ / 16], gf[kTV / 16];
  {
    const __bf16* qp = elem_ptr<__bf16>(a.q, i, h);
    const __bf16* gp = elem_ptr<__bf16>(a.g16, i, h);
#pragma unroll
    for (int ks = 0; ks < kTQ / 16; ++ks)
      qf[ks] = *reinterpret_cast<const bf16x8*>(qp + 16 * ks + 8 * half);
#pragma unroll
    for (int ks = 0; ks < kTV / 16; ++ks)
      gf[ks] = *reinterpret_cast<const bf16x8*>(gp + 16 * ks + 8 * half);
  }
  const int64_t pair = (int64_t)i * hq + h;
  const float lse2 = a.lse[pair] * kL2e;
  const float dl = a.delta[pair];
  __bf16* dsrow = a.ds + pair * a.wpad;
  __bf16* prow = a.pb + pair * a.wpad;
  // the previous tile's dS' and P, stored once the next tile is under way; lane
  // holds slots 32 t + 8 jj + 4 half + 0 .. 3 in [jj / 2][4 (jj % 2) ..]
  bf16x8 prev[2], prevp[2];
  auto store_prev = [&](int t) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      bf16x4 v, w;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        v[u] = prev[jj >> 1][4 * (jj & 1) + u];
        w[u] = prevp[jj >> 1][4 * (jj & 1) + u];
      }
      *reinterpret_cast<bf16x4*>(dsrow + kDS * t + 8 * jj + 4 * half) = v;
      *reinterpret_cast<bf16x4*>(prow + kDS * t + 8 * jj + 4 * half) = w;
    }
  };
  for (int t = 0; t < n_t; ++t) {
    wait_gathers();
    __syncthreads();
    if (t + 1 < n_t)
      gather_tile<VA>(a, g, s.key, kfb, t + 1, s.k[(t + 1) & 1], s.v[VA ? 0 : (t + 1) & 1], nw,
                      wave, lane);
    if (t > 0) store_prev(t - 1);
    const __bf16* kt = s.k[t & 1];
    const __bf16* vt = s.v[VA ? 0 : t & 1];
    // S^T and dP^T: rows = the tile's slots, columns = the wave's heads
    const int r = lane & 31;
    f32x16 s0 = f32x16{}, s1 = f32x16{}, p0 = f32x16{}, p1 = f32x16{};
#pragma unroll
    for (int ks = 0; ks < kTQ / 16; ks += 2) {
      s0 = mfma(*reinterpret_cast<const bf16x8*>(kt + offq(r, 16 * ks + 8 * half)), qf[ks], s0);
      s1 = mfma(*reinterpret_cast<const bf16x8*>(kt + offq(r, 16 * ks + 16 + 8 * half)), qf[ks + 1], s1);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int ks = 0; ks < kTV / 16; ks += 2) {
      const int e0 = 16 * ks + 8 * half, e1 = e0 + 16;
      const bf16x8& v0 = *reinterpret_cast<const bf16x8*>(VA ? kt + offq(r, e0) : vt + offg(r, e0));
      const bf16x8& v1 = *reinterpret_cast<const bf16x8*>(VA ? kt + offq(r, e1) : vt + offg(r, e1));
      p0 = mfma(v0, gf[ks], p0);
      p1 = mfma(v1, gf[ks + 1], p1);
      __builtin_amdgcn_sched_barrier(0);
    }
    // lane holds head h, slots 32 t + 8 (j / 4) + 4 half + (j % 4)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int slot = kDS * t + 8 * (j >> 2) + 4 * half + (j & 3);
      const bool ok = slot < a.idx_width && s.key[min(slot, a.idx_width - 1)] >= 0;
      const float pv = exp2_raw(fmaf(s0[j] + s1[j], a.scale_log2, ok ? -lse2 : -INFINITY));
      prev[j >> 3][j & 7] = (__bf16)(pv * (p0[j] + p1[j] - dl));
      prevp[j >> 3][j & 7] = (__bf16)pv;
    }
  }
  store_prev(n_t - 1);
}

// The value is the key's first 512 columns: one gathered tile serves both products,
// and each block of 32 heads gets two waves, one forming S^T (the heads' Q^T
// fragments in registers, 144 of them) and one forming dP^T (dO^T, 128), so neither
// runs out of registers at two waves per SIMD.  The S wave hands P (fp32) to the dP
// wave through LDS; the dP wave forms dS' = P (dP - D) one tile later, which keeps
// one barrier per tile: P of tile t is written after barrier t into stage t % 2 and
// read after barrier t + 1, before stage t % 2 is written again after barrier t + 2.
struct SdpLds {
  __bf16 k[2][kDS * kTQ];
  float4 xp[2][4][4][kWave];  // [stage][head block][j / 4][lane]: P in accumulator order
  int key[kMaxW];
};

template <bool SW>
__device__ __forceinline__ void sdp_role(const BwTokArgs& a, SdpLds& s, int i, int g, int hb,
                                         int kfb, int nw, int wave, int lane) {
  const int half = lane >> 5;
  const int hq = a.q.h, G = hq / a.k.h;
  const int h = g * G + 32 * hb + (lane & 31);  // this lane's head (B-operand column)
  constexpr int NF = (SW ? kTQ : kTV) / 16;
  bf16x8 f[NF];
  {
    const __bf16* fp = SW ? elem_ptr<__bf16>(a.q, i, h) : elem_ptr<__bf16>(a.g16, i, h);
#pragma unroll
    for (int ks = 0; ks < NF; ++ks)
      f[ks] = *reinterpret_cast<const bf16x8*>(fp + 16 * ks + 8 * half);
  }
  const int64_t pair = (int64_t)i * hq + h;
  const float lse2 = SW ? a.lse[pair] * kL2e : 0.f;
  const float dl = SW ? 0.f : a.delta[pair];
  __bf16* orow = (SW ? a.pb : a.ds) + pair * a.wpad;
  const int n_t = (a.idx_width + kDS - 1) / kDS;
  const int r = lane & 31;
  // lane holds head h, slots 32 t + 8 (j / 4) + 4 half + (j % 4); the previous tile's
  // results (P, or dP - D) wait here for the next iteration
  float prev[16];
  auto store = [&](int t, const float* x) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      bf16x4 v;
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = (__bf16)x[4 * jj + u];
      *reinterpret_cast<bf16x4*>(orow + kDS * t + 8 * jj + 4 * half) = v;
    }
  };
  for (int t = 0; t <= n_t; ++t) {
    wait_gathers();
    __syncthreads();
    if (t + 1 < n_t)
      gather_tile<true>(a, g, s.key, kfb, t + 1, s.k[(t + 1) & 1], nullptr, nw, wave, lane);
    if (t > 0) {
      if (SW) {
        store(t - 1, prev);
      } else {
        float ds[16];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const float4 pv = s.xp[(t - 1) & 1][hb][jj][lane];
          ds[4 * jj + 0] = pv.x * prev[4 * jj + 0];
          ds[4 * jj + 1] = pv.y * prev[4 * jj + 1];
          ds[4 * jj + 2] = pv.z * prev[4 * jj + 2];
          ds[4 * jj + 3] = pv.w * prev[4 * jj + 3];
        }
        store(t - 1, ds);
      }
    }
    if (t == n_t) break;
    // row r's piece 2 ks + half sits at (2 ks + half) ^ swq(r): for ks = 4 q + u that is
    // base u plus 8 q pieces, so four per-lane bases and immediate offsets suffice.
    // Fragments sit in a ring of four, read three MFMAs ahead of their use.
    const __bf16* kt = s.k[t & 1] + r * kTQ;
    auto af = [&](int ks) {
      return *reinterpret_cast<const bf16x8*>(kt + (((2 * (ks & 3) + half) ^ swq(r)) << 3) +
                                              64 * (ks >> 2));
    };
    f32x16 c0 = f32x16{}, c1 = f32x16{};
    bf16x8 fr[4];
#pragma unroll
    for (int ks = 0; ks < 3; ++ks) fr[ks] = af(ks);
#pragma unroll
    for (int ks = 0; ks < NF; ++ks) {
      if (ks + 3 < NF) fr[(ks + 3) & 3] = af(ks + 3);
      if (ks & 1) c1 = mfma(fr[ks & 3], f[ks], c1);
      else c0 = mfma(fr[ks & 3], f[ks], c0);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (SW) {
      // slots past the width or selecting no permitted key get P = 0
      const int sl = kDS * t + r;
      const int kk = s.key[min(sl, a.idx_width - 1)];
      const uint64_t ok = __ballot(sl < a.idx_width && kk >= 0);
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const bool on = (ok >> (8 * (j >> 2) + 4 * half + (j & 3))) & 1;
        prev[j] = exp2_raw(fmaf(c0[j] + c1[j], a.scale_log2, on ? -lse2 : -INFINITY));
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        s.xp[t & 1][hb][jj][lane] = make_float4(prev[4 * jj], prev[4 * jj + 1],
                                                prev[4 * jj + 2], prev[4 * jj + 3]);
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) prev[j] = c0[j] + c1[j] - dl;
    }
  }
}

// one workgroup per (row, key head): waves 0 .. G/32 - 1 form S^T for head block w,
// waves G/32 .. G/16 - 1 dP^T for head block w - G/32
__global__ __launch_bounds__(512, 1) void k_bwtm_ds(BwTokArgs a) {
  __shared__ SdpLds s;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int nw = blockDim.x / kWave, nb = nw / 2;
  const int i = blockIdx.x / a.k.h, g = blockIdx.x % a.k.h;
  const int kfb = stage_slots(a, i, s.key);
  __syncthreads();
  gather_tile<true>(a, g, s.key, kfb, 0, s.k[0], nullptr, nw, wave, lane);
  if (wave < nb) sdp_role<true>(a, s, i, g, wave, kfb, nw, wave, lane);
  else sdp_role<false>(a, s, i, g, wave - nb, kfb, nw, wave, lane);
}

// B operand [16 slots x 32 columns] of a gathered key tile, slots in natural order
// (16 qs + 8 half + 0 .. 7), columns c0 .. c0 + 31
__device__ __forceinline__ bf16x8 trnat(const __bf16* t, int qs, int c0, int lane) {
  const int half = lane >> 5, c16 = lane & 15, grp = lane >> 4;
  const int r = 16 * qs + 8 * half + (c16 >> 2);
  const int c = c0 + 16 * (grp & 1) + 4 * (c16 & 3);
  const bf16x4 lo = read_tr(t, offq(r, c));
  const bf16x4 hi = read_tr(t, offq(r + 4, c));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// one workgroup per (row, key head); wave w takes head block w % (G/32) and dQ
// columns 288 (w / (G/32)) .. + 287: 144 accumulators per wave, two waves per SIMD
__global__ __launch_bounds__(512, 1) void k_bwtm_dq(BwTokArgs a) {
  __shared__ DqLds s;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int nw = blockDim.x / kWave, nb = nw / 2;
  const int hb = wave % nb, ch = wave / nb;
  const int half = lane >> 5;
  const int i = blockIdx.x / a.k.h, g = blockIdx.x % a.k.h;
  const int hq = a.q.h, G = hq / a.k.h;
  const int h0 = g * G + 32 * hb;  // this wave's first head
  const int kfb = stage_slots(a, i, s.key);
  __syncthreads();
  const int n_t = (a.idx_width + kDS - 1) / kDS;
  // half ch of head block hb's dS' tile t (32 heads x 32 slots, 2 KiB) into stage st
  auto copy_ds = [&](int t, int st) {
    const int byte = 1024 * ch + 16 * lane;
    const int hl = byte / (2 * kDS), sl = (byte % (2 * kDS)) / 2;
    const __bf16* src = a.ds + ((int64_t)i * hq + h0 + hl) * a.wpad + kDS * t + sl;
    gather16_addr(src, __builtin_amdgcn_readfirstlane(lds_addr(&s.ds[st][hb][0]) + 1024 * ch));
  };
  gather_tile<true>(a, g, s.key, kfb, 0, s.k[0], nullptr, nw, wave, lane);
  copy_ds(0, 0);
  constexpr int NB = kTQ / 64;  // 9 column blocks of 32 per wave
  const int cb = 32 * NB * ch;  // the wave's first column
  f32x16 acc[NB];
#pragma unroll
  for (int x = 0; x < NB; ++x) acc[x] = f32x16{};
  for (int t = 0; t < n_t; ++t) {
    wait_gathers();
    __syncthreads();
    if (t + 1 < n_t) {
      gather_tile<true>(a, g, s.key, kfb, t + 1, s.k[(t + 1) & 1], nullptr, nw, wave, lane);
      copy_ds(t + 1, (t + 1) & 1);
    }
    const __bf16* kt = s.k[t & 1];
    const __bf16* dt = s.ds[t & 1][hb];
    // A operands: dS' rows of the wave's heads (m = head lane % 32), slots 16 qs + 8 half ..
    const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(dt + (lane & 31) * kDS + 8 * half);
    const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(dt + (lane & 31) * kDS + 16 + 8 * half);
    bf16x8 f0 = trnat(kt, 0, cb, lane), f1 = trnat(kt, 0, cb + 32, lane);
#pragma unroll
    for (int u = 0; u < 2 * NB; ++u) {  // u = NB qs + x
      bf16x8 nf;
      if (u + 2 < 2 * NB) nf = trnat(kt, (u + 2) / NB, cb + 32 * ((u + 2) % NB), lane);
      acc[u % NB] = mfma(u < NB ? a0 : a1, f0, acc[u % NB]);
      f0 = f1;
      f1 = nf;
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // lane holds column cb + 32 x + lane % 32, heads h0 + 8 (j / 4) + 4 half + (j % 4)
  const float scl = a.scale;  // dQ sums dS' = dS / scale
#pragma unroll
  for (int x = 0; x < NB; ++x)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int hh = h0 + 8 * (j >> 2) + 4 * half + (j & 3);
      a.dq[((int64_t)i * hq + hh) * kTQ + cb + 32 * x + (lane & 31)] = scl * acc[x][j];
    }
}

// ---- dK, dV -------------------------------------------------------------------------------
// Row-centric: each selected slot's contributions, summed over the heads of its
// key head, then added per key over the key's list of slots:
//   k_bwtm_ckv  per (row, key head, 128 slots): C_K[slot] = sum_h dS'[h, slot] q[h]
//               (576) and C_V[slot] = sum_h P[h, slot] dO[h] (512), bf16, as MFMA
//               products over the heads with the slots' dS' and P and 64-column
//               chunks of the heads' q and dO rows in LDS
//   k_bwtm_kred per (key, key head): dk = scale sum C_K, dv = sum C_V over the
//               key's slots in list order (no floating-point atomics)
constexpr int kCS = 128;  // slots per k_bwtm_ckv workgroup
constexpr int kCC = 64;   // columns per chunk

__device__ __forceinline__ int sw128(int r) { return ((r >> 1) & 1) << 2; }
__device__ __forceinline__ int sw256(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int offx(int r, int e) {  // [head][64 columns], 128-byte rows
  return r * kCC + ((((e >> 3) ^ sw128(r))) << 3) + (e & 7);
}
__device__ __forceinline__ int offs(int r, int e) {  // [head][128 slots], 256-byte rows
  return r * kCS + ((((e >> 3) ^ sw256(r))) << 3) + (e & 7);
}

// dS' and P of the G heads for the 128 slots are staged (one after the other) and read
// into each wave's registers (the B operands of its 32 slots); their LDS then holds
// the double-buffered q / dO chunks and the output tile
union CkLds {
  __bf16 b[128 * kCS];  // dS', then P, of the group's heads for the 128 slots
  struct {
    __bf16 x[2][128 * kCC];  // a 64-column chunk of the heads' q (chunks 0 .. 8) or dO (9 .. 16)
    __bf16 out[kCS * kCC];   // the chunk's results, slot-major, on their way out
  } c;
};

// the output tile: 128-byte slot rows, piece p of row s at p ^ ((s / 2) % 8)
__device__ __forceinline__ int offo(int s, int e) {
  return s * kCC + ((((e >> 3) ^ ((s >> 1) & 7))) << 3) + (e & 7);
}

// operand [16 heads (natural order) x 32 columns] read transposed from a [head][...] tile
template <bool S>
__device__ __forceinline__ bf16x8 trh(const __bf16* t, int ks, int c0, int lane) {
  const int half = lane >> 5, c16 = lane & 15, grp = lane >> 4;
  const int r = 16 * ks + 8 * half + (c16 >> 2);
  const int c = c0 + 16 * (grp & 1) + 4 * (c16 & 3);
  const bf16x4 lo = read_tr(t, S ? offs(r, c) : offx(r, c));
  const bf16x4 hi = read_tr(t, S ? offs(r + 4, c) : offx(r + 4, c));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// one workgroup per (row, key head, 128 slots); wave w takes slots 32 w .. 32 w + 31
// and both 32-column blocks of every chunk
template <int G>
__global__ __launch_bounds__(256, 3) void k_bwtm_ckv(BwTokArgs a) {
  __shared__ CkLds s;
  constexpr int KS = G / 16;  // k-steps over the heads
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int half = lane >> 5;
  const int hkv = a.k.h, hq = a.q.h;
  const int n_st = a.wpad / kCS;
  const int i = blockIdx.x / (hkv * n_st);
  const int g = (blockIdx.x / n_st) % hkv;
  const int st = blockIdx.x % n_st;
  const int W = a.idx_width;
  if (kCS * st >= W) return;
  const int h0 = g * G;
  const __bf16* qb = static_cast<const __bf16*>(a.q.data);
  const __bf16* gb = static_cast<const __bf16*>(a.g16.data);

  // dS', then P, of the G heads for the 128 slots (4 heads per 1 KiB copy) through one
  // 32 KiB area, so that the workgroup's LDS stays at 48 KiB (three workgroups a CU)
  auto stage = [&](const __bf16* src0) {
    for (int m = wave; m < G / 4; m += 4) {
      const int hh = 4 * m + lane / 16, pp = lane % 16;
      const __bf16* src = src0 + ((int64_t)i * hq + h0 + hh) * a.wpad + kCS * st + 8 * (pp ^ sw256(hh));
      gather16_addr(src, __builtin_amdgcn_readfirstlane(lds_addr(s.b) + 1024 * m));
    }
    wait_gathers();
    __syncthreads();
  };
  bf16x8 bd[KS], bp[KS];  // B operands [heads 16 ks .. x the wave's 32 slots]
  stage(a.ds);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) bd[ks] = trh<true>(s.b, ks, 32 * wave, lane);
  __syncthreads();
  stage(a.pb);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) bp[ks] = trh<true>(s.b, ks, 32 * wave, lane);
  __syncthreads();
  // chunk c of the heads' q (c < 9) or dO rows: 8 heads per 1 KiB copy
  auto copy_chunk = [&](int c) {
    const bool qq = c < kTQ / kCC;
    const int col = kCC * (qq ? c : c - kTQ / kCC);
    for (int m = wave; m < G / 8; m += 4) {
      const int hh = 8 * m + lane / 8, pp = lane % 8;
      const __bf16* src =
          qq ? qb + (int64_t)i * a.q.stride_n + (int64_t)(h0 + hh) * a.q.stride_h
             : gb + (int64_t)i * a.g16.stride_n + (int64_t)(h0 + hh) * a.g16.stride_h;
      gather16_addr(src + col + 8 * (pp ^ sw128(hh)),
                    __builtin_amdgcn_readfirstlane(lds_addr(s.c.x[c & 1]) + 1024 * m));
    }
  };
  copy_chunk(0);
  constexpr int NCH = kTQ / kCC + kTV / kCC;  // 17
  const int sl = 32 * wave + (lane & 31);      // the lane's slot in the tile
  for (int c = 0; c < NCH; ++c) {
    wait_gathers();
    __syncthreads();
    if (c + 1 < NCH) copy_chunk(c + 1);
    const bool qq = c < kTQ / kCC;
    const __bf16* xt = s.c.x[c & 1];
    // C^T [32 columns x 32 slots] = X^T [columns x heads] . B [heads x slots], per
    // 32-column block
    f32x16 acc0 = f32x16{}, acc1 = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8& b = qq ? bd[ks] : bp[ks];
      acc0 = mfma(trh<false>(xt, ks, 0, lane), b, acc0);
      acc1 = mfma(trh<false>(xt, ks, 32, lane), b, acc1);
    }
    // lane holds slot sl, columns 32 u + 8 (j / 4) + 4 half + (j % 4) of the chunk:
    // through LDS, then out as whole 128-byte rows
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const f32x16& acc = u == 0 ? acc0 : acc1;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        bf16x4 v;
#pragma unroll
        for (int t = 0; t < 4; ++t) v[t] = (__bf16)acc[4 * jj + t];
        *reinterpret_cast<bf16x4*>(&s.c.out[offo(sl, 32 * u + 8 * jj + 4 * half)]) = v;
      }
    }
    __syncthreads();
    __bf16* outb = qq ? a.ck : a.cv;
    const int D = qq ? kTQ : kTV;
    const int col = kCC * (qq ? c : c - kTQ / kCC);
#pragma unroll
    for (int t = threadIdx.x; t < kCS * (kCC / 8); t += 256) {
      const int ts = t / (kCC / 8), pc = t % (kCC / 8);
      const int slot = kCS * st + ts;
      if (slot < W)
        *reinterpret_cast<bf16x8*>(outb + (((int64_t)i * W + slot) * hkv + g) * D + col + 8 * pc) =
            *reinterpret_cast<const bf16x8*>(&s.c.out[offo(ts, 8 * pc)]);
    }
  }
}

// one workgroup per (key, key head): wave w adds the key's list entries w, w + 4, ..
// (four entries' rows in flight at a time, their ids fetched 64 at a time), and the
// four partial sums are added in wave order: a fixed order, so bitwise reproducible
constexpr int kKC = kTQ + kTV;  // contribution columns per slot

__device__ __forceinline__ void add8(float* acc, const bf16x8& v) {
#pragma unroll
  for (int t = 0; t < 8; ++t) acc[t] += (float)v[t];
}

__global__ __launch_bounds__(256) void k_bwtm_kred(BwTokArgs a) {
  __shared__ float part[4][kKC];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int hkv = a.k.h;
  const int64_t kp = blockIdx.x;
  const int j = (int)(kp / hkv), g = (int)(kp % hkv);
  const int e0 = a.list_off[j], e1 = a.list_off[j + 1];
  const bool tail = lane < kTQ / 8 - kWave;  // lanes holding C_K columns 512 .. 575
  float ak[8] = {}, ak2[8] = {}, av[8] = {};
  for (int base = e0 + wave; base < e1; base += 4 * kWave) {
    // this wave's entries base, base + 4, .. (up to 64 of them), lane t holding the t-th
    const int n = min(kWave, (e1 - base + 3) / 4);
    const int mine = lane < n ? a.entries[base + 4 * lane] : 0;
    int u = 0;
    for (; u + 4 <= n; u += 4) {
      bf16x8 k0[4], k1[4], v0[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int64_t p = (int64_t)__builtin_amdgcn_readlane(mine, u + x) * hkv + g;
        k0[x] = *reinterpret_cast<const bf16x8*>(a.ck + p * kTQ + 8 * lane);
        if (tail) k1[x] = *reinterpret_cast<const bf16x8*>(a.ck + p * kTQ + 8 * (kWave + lane));
        v0[x] = *reinterpret_cast<const bf16x8*>(a.cv + p * kTV + 8 * lane);
      }
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        add8(ak, k0[x]);
        if (tail) add8(ak2, k1[x]);
        add8(av, v0[x]);
      }
    }
    for (; u < n; ++u) {
      const int64_t p = (int64_t)__builtin_amdgcn_readlane(mine, u) * hkv + g;
      add8(ak, *reinterpret_cast<const bf16x8*>(a.ck + p * kTQ + 8 * lane));
      if (tail) add8(ak2, *reinterpret_cast<const bf16x8*>(a.ck + p * kTQ + 8 * (kWave + lane)));
      add8(av, *reinterpret_cast<const bf16x8*>(a.cv + p * kTV + 8 * lane));
    }
  }
  float* pw = part[wave];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    pw[8 * lane + t] = ak[t];
    if (tail) pw[8 * (kWave + lane) + t] = ak2[t];
    pw[kTQ + 8 * lane + t] = av[t];
  }
  __syncthreads();
  float* dk = a.dk + kp * kTQ;
  float* dv = a.dv + kp * kTV;
  const float scl = a.scale;  // dK sums dS' = dS / scale
  for (int c = threadIdx.x; c < kKC; c += 256) {
    const float x = ((part[0][c] + part[1][c]) + part[2][c]) + part[3][c];
    if (c < kTQ) dk[c] = scl * x;
    else dv[c - kTQ] = x;
  }
}

unsigned grid_of(int64_t items, int per) { return (unsigned)((items + per - 1) / per); }

}  // namespace

bool attn_bwd_token_mfma_supported(int mode, int dtype, int dqk, int dv, int hq, int hkv,
                                   int idx_heads, int idx_width) {
  if (mode != CSA_SEL_TOKEN || dtype != CSA_BF16 || dqk != kTQ || dv != kTV ||
      idx_heads != 1 || idx_width > kMaxW || hq % hkv)
    return false;
  const int G = hq / hkv;
  return G == 32 || G == 64 || G == 128;
}

int attn_bwd_token_wpad(int idx_width) { return (idx_width + kCS - 1) / kCS * kCS; }

hipError_t launch_attn_bwd_token(const BwTokArgs& a0, hipStream_t stream) {
  hipError_t e;
  BwTokArgs a = a0;
  const int64_t pairs = (int64_t)a.L.n_q * a.q.h;
  if (a.dout_dtype == CSA_BF16) {
    a.g16 = a.dout;
  } else {
    a.g16 = View{a.dout16, (int64_t)a.q.h * kTV, kTV, a.L.n_q, a.q.h, kTV};
    if (pairs > 0) {
      hipLaunchKernelGGL(k_bwtm_dout16, dim3(grid_of(pairs * (kTV / 8), 256)), dim3(256), 0,
                         stream, a, a.dout16);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  if (a.L.n_kv == 0) {  // no keys: dQ is zero (dK, dV have no rows)
    const int64_t words = pairs * kTQ;
    if (words > 0) {
      hipLaunchKernelGGL(k_bwtm_fill, dim3((unsigned)std::min<int64_t>(4096, grid_of(words, 256))),
                         dim3(256), 0, stream, reinterpret_cast<uint32_t*>(a.dq), words);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
  }
  int slot;
  const int G = a.q.h / a.k.h;
  if (a.L.n_q > 0) {
    const dim3 grid((unsigned)((int64_t)a.L.n_q * a.k.h)), block((unsigned)(G / 32 * kWave));
    const bool va = a.v.data == a.k.data && a.v.stride_n == a.k.stride_n &&
                    a.v.stride_h == a.k.stride_h;
    trace_begin(stream, "k_bwtm_ds", &slot);
    if (va) hipLaunchKernelGGL(k_bwtm_ds, grid, dim3(2 * block.x), 0, stream, a);
    else hipLaunchKernelGGL(k_bwtm_ds_v, grid, block, 0, stream, a);
    trace_end(stream, slot);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    trace_begin(stream, "k_bwtm_dq", &slot);
    hipLaunchKernelGGL(k_bwtm_dq, grid, dim3(2 * block.x), 0, stream, a);
    trace_end(stream, slot);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    trace_begin(stream, "k_bwtm_ckv", &slot);
    const dim3 cgrid((unsigned)((int64_t)a.L.n_q * a.k.h * (a.wpad / kCS)));
    if (G == 32) hipLaunchKernelGGL(k_bwtm_ckv<32>, cgrid, dim3(256), 0, stream, a);
    else if (G == 64) hipLaunchKernelGGL(k_bwtm_ckv<64>, cgrid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL(k_bwtm_ckv<128>, cgrid, dim3(256), 0, stream, a);
    trace_end(stream, slot);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  trace_begin(stream, "k_bwtm_kred", &slot);
  hipLaunchKernelGGL(k_bwtm_kred, dim3((unsigned)((int64_t)a.L.n_kv * a.k.h)), dim3(256), 0,
                     stream, a);
  trace_end(stream, slot);
  return hipGetLastError();
}

}  // namespace csa
