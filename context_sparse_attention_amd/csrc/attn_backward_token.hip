// Token-mode backward of dK and dV on the matrix cores: one selection per
// token (shared by every query head), bf16, Dqk = 576 and Dv = 512 (absorbed
// MLA: the value may be the key's first 512 columns).
//
// "Context parallel attention: exchange keys and merge softmax globally", masks
// paragraph (key and value gradients go back to their owners); Megatron-LM issue
// #4878, "Strategy: allgather CP mode", backward step.  With the forward's lse,
// c(i, j) the number of times row i's index row holds key j (only permitted
// keys count) and dS' = P (dP - D):
//
//   dv_j = sum_(i, h) c(i, j) P dO[i, h]      dk_j = scale sum_(i, h) c(i, j) dS' q[i, h]
//
// The keys a token selects share no structure with its neighbours', so a key
// tile has no common set of rows.  The kernel therefore runs key tiles against
// every row whose permitted range meets the tile, masked by c: more products
// than the selection needs (about 1 / density), but each one a dense MFMA tile
// with its operands in LDS, instead of scattered per-key work.
//
//   k_bwtm_count  c(i, j) as a uint16 map [n_q, n_kv rounded up to 64]
//   k_bwtm_rec    per (row, 32-head block): lse * log2(e) and D, 256 bytes
//   k_bwtm_dout16 dO rounded to bf16 when it arrives in fp32
//   k_bwtm_dkdv   one workgroup per (key head, 32 keys, 512 rows), four waves.
//                 Per block of 32 items (32 heads of one row), waves 0 and 1 each
//                 take half of S = Q K^T's contraction (half K rows in registers)
//                 and waves 2 and 3 half of dP = dO V^T's; the partial sums meet
//                 in LDS; waves 0 and 1 form P and each accumulates half of
//                 dV^T += dO^T P, waves 2 and 3 form dS' and each half of
//                 dK^T += Q^T dS'.  The next
//                 block's rows, record and counts are copied global -> LDS while
//                 the current one is computed.  Partial sums per row chunk.
//   k_bwtm_reduce the row chunks' partial sums in chunk order
#include <algorithm>

#include "attention.hpp"
#include "gather.hpp"

namespace csa {

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kTQ = 576;              // key / query width
constexpr int kTV = 512;              // value width
constexpr int kTI = 32;               // items (heads of one row) per block
constexpr int kTK = 32;               // keys per workgroup
constexpr int kTRows = 512;           // rows per workgroup
constexpr int kTW = 4;                // waves
constexpr int kTT = kTW * kWave;      // threads
constexpr int kTQC = kTI * kTQ * 2 / 1024;  // 1 KiB copies of a block's query rows (36)
constexpr int kTGC = kTI * kTV * 2 / 1024;  // ... of its dO rows (32)
constexpr int kTC = kTQC + kTGC + 1;        // with the record / counts copy
constexpr int kTPart = kTQ + kTV;     // floats per (chunk, key, key head) partial
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

// A operand [32 columns x 16 items] of a transposed item tile: items (16 st +
// the permutation of the first product's accumulator rows), columns c0 .. c0 + 31.
template <bool Q>
__device__ __forceinline__ bf16x8 trfrag(const __bf16* t, int st, int c0, int lane) {
  const int half = lane >> 5, c16 = lane & 15, grp = lane >> 4;
  const int r = 16 * st + 4 * half + (c16 >> 2);
  const int c = c0 + 16 * (grp & 1) + 4 * (c16 & 3);
  const bf16x4 lo = read_tr(t, Q ? offq(r, c) : offg(r, c));
  const bf16x4 hi = read_tr(t, Q ? offq(r + 8, c) : offg(r + 8, c));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// acc0 + acc1 = sum over k-steps of A rows (item tile t, row `it`, columns from e0)
// times B[ks]: two
// accumulator chains, each step's A fragments read two steps ahead, with a
// scheduling fence per step so that the reads are not hoisted further (the
// registers are spoken for).
template <bool Q, int NKS>
__device__ __forceinline__ void row_chains(const __bf16* t, int it, int half, int e0,
                                           const bf16x8 (&bf)[kTQ / 32], f32x16& acc0,
                                           f32x16& acc1) {
  auto ld = [&](int ks) {
    const int e = e0 + 16 * ks + 8 * half;
    return *reinterpret_cast<const bf16x8*>(t + (Q ? offq(it, e) : offg(it, e)));
  };
  bf16x8 a0 = ld(0), a1 = ld(1);
#pragma unroll
  for (int ks = 0; ks < NKS; ks += 2) {
    bf16x8 n0, n1;
    if (ks + 2 < NKS) {
      n0 = ld(ks + 2);
      n1 = ld(ks + 3);
    }
    acc0 = mfma(a0, bf[ks], acc0);
    acc1 = mfma(a1, bf[ks + 1], acc1);
    a0 = n0;
    a1 = n1;
    __builtin_amdgcn_sched_barrier(0);
  }
}

// ---- preparation --------------------------------------------------------------------------
__global__ void k_bwtm_fill(uint32_t* p, int64_t n) {
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < n;
       t += (int64_t)gridDim.x * blockDim.x)
    p[t] = 0u;
}

// c(i, j): one thread per index slot; repeated slots add again
__global__ __launch_bounds__(256) void k_bwtm_count(BwTokArgs a) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= (int64_t)a.L.n_q * a.idx_width) return;
  const int i = (int)(t / a.idx_width);
  const RowKeys r = row_keys(a.L, i);
  const int s = a.idx[t];
  if (!r.valid || s < r.lo || s > r.hi) return;
  const int64_t e = (int64_t)i * a.n_kvp + s;
  uint32_t* w = reinterpret_cast<uint32_t*>(a.cmap) + (e >> 1);
  atomicAdd(w, (e & 1) ? 0x10000u : 1u);
}

// per (row, 32-head block): lse * log2(e) for the 32 heads, then their D
__global__ __launch_bounds__(256) void k_bwtm_rec(BwTokArgs a) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= (int64_t)a.L.n_q * a.q.h) return;
  const int64_t i = t / a.q.h;
  const int h = (int)(t % a.q.h);
  float* rec = a.rec + (i * (a.q.h / kTI) + h / kTI) * 64;
  rec[h % kTI] = a.lse[t] * kL2e;
  rec[kTI + h % kTI] = a.delta[t];
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

// ---- dK, dV -------------------------------------------------------------------------------
struct TkLds {
  __bf16 q[2][kTI * kTQ];
  __bf16 g[2][kTI * kTV];
  float xs[kTW][kWave * 16];   // [wave][lane * 16 + j]: partial S or dP
  float meta[2][256];          // [stage]: lse2[32], D[32], counts (32 x uint16), unused
  int rows[kTRows];            // the chunk's rows that meet the key tile
};

__global__ __launch_bounds__(kTT, 1) void k_bwtm_dkdv(BwTokArgs a) {
  __shared__ TkLds s;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int half = lane >> 5;
  // waves 0, 1: halves of S's contraction (K rows in registers), then P and half
  // of dV^T each; waves 2, 3: halves of dP's (V rows), then P, dS' and half of dK^T
  const int role = wave >> 1;  // 0: S / dV^T, 1: dP / dK^T
  const int hf = wave & 1;     // which half
  const int n_tiles = a.n_kvp / kTK;
  const int g = blockIdx.x / (n_tiles * a.n_chunks);
  const int rem = blockIdx.x % (n_tiles * a.n_chunks);
  const int kt = rem / a.n_chunks;
  const int chunk = rem % a.n_chunks;
  const int tk0 = kt * kTK;
  const int hq = a.q.h;
  const int G = hq / a.k.h;
  const int nhb = G / kTI;
  float* part = a.part + (((int64_t)chunk * a.n_kvp + tk0) * a.k.h + g) * kTPart;

  // the chunk's rows whose permitted keys meet [tk0, tk0 + 64)
  const int c0 = chunk * kTRows;
  int nvis;
  {
    __shared__ int s_wave[kTW];
    const int t0 = 2 * threadIdx.x;
    int f[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = c0 + t0 + u;
      f[u] = 0;
      if (i < a.L.n_q) {
        const RowKeys r = row_keys(a.L, i);
        f[u] = r.valid && r.lo < tk0 + kTK && r.hi >= tk0;
      }
    }
    const int cnt = f[0] + f[1];
    int incl = cnt;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int y = __shfl_up(incl, off, kWave);
      if (lane >= off) incl += y;
    }
    if (lane == kWave - 1) s_wave[wave] = incl;
    __syncthreads();
    int before = 0;
    nvis = 0;
    for (int w = 0; w < kTW; ++w) {
      if (w < wave) before += s_wave[w];
      nvis += s_wave[w];
    }
    int at = before + incl - cnt;
    if (f[0]) s.rows[at++] = c0 + t0;
    if (f[1]) s.rows[at] = c0 + t0 + 1;
  }
  const int n_blk = nvis * nhb;
  if (n_blk == 0) {  // no row meets the tile: the partial sums are zero
    for (int t = threadIdx.x; t < kTK * kTPart / 4; t += kTT) {
      const int key = t / (kTPart / 4), d4 = t % (kTPart / 4);
      *reinterpret_cast<float4*>(part + (int64_t)key * a.k.h * kTPart + 4 * d4) =
          make_float4(0.f, 0.f, 0.f, 0.f);
    }
    return;
  }
  __syncthreads();  // s.rows complete

  const __bf16* qb = static_cast<const __bf16*>(a.q.data);
  const __bf16* gb = static_cast<const __bf16*>(a.g16.data);
  // block b: row rows[b / nhb], heads g G + 32 (b % nhb) ..
  auto copy_block = [&](int b) {
    const int i = s.rows[b / nhb];
    const int h0 = g * G + kTI * (b % nhb);
    const int stg = b & 1;
    for (int c = wave; c < kTC; c += kTW) {
      if (c < kTQC) {
        const int byte = 1024 * c + 16 * lane;
        const int r = byte / (kTQ * 2);
        const int pp = (byte % (kTQ * 2)) / 16;
        const int e = (pp ^ swq(r)) * 8;
        const __bf16* src = qb + (int64_t)i * a.q.stride_n + (int64_t)(h0 + r) * a.q.stride_h + e;
        gather16_addr(src, __builtin_amdgcn_readfirstlane(lds_addr(&s.q[stg][0]) + 1024 * c));
      } else if (c < kTQC + kTGC) {
        const int r = c - kTQC;
        const int e = (lane ^ swg(r)) * 8;
        const __bf16* src =
            gb + (int64_t)i * a.g16.stride_n + (int64_t)(h0 + r) * a.g16.stride_h + e;
        gather16_addr(src, __builtin_amdgcn_readfirstlane(lds_addr(&s.g[stg][0]) + 1024 * r));
      } else {
        const float* rec = a.rec + ((int64_t)i * (hq / kTI) + h0 / kTI) * 64;
        const void* src;
        if (lane < 16) src = rec + 4 * lane;
        else if (lane < 20) src = a.cmap + (int64_t)i * a.n_kvp + tk0 + 8 * (lane - 16);
        else src = rec;
        gather16_addr(src, __builtin_amdgcn_readfirstlane(lds_addr(&s.meta[stg][0])));
      }
    }
  };
  copy_block(0);

  // B operands: half of the K row (role 0: 18 k-steps) or of the V row (role 1:
  // 16) of key tk0 + lane % 32 (past the last key: the last one, counts are 0)
  constexpr int NKS = kTQ / 32;  // 18
  bf16x8 bf[NKS];
  {
    const int key = min(tk0 + (lane & 31), a.L.n_kv - 1);
    const __bf16* src = role == 0 ? elem_ptr<__bf16>(a.k, key, g) + hf * (kTQ / 2)
                                  : elem_ptr<__bf16>(a.v, key, g) + hf * (kTV / 2);
    const int nks = role == 0 ? kTQ / 32 : kTV / 32;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      if (ks < nks) bf[ks] = *reinterpret_cast<const bf16x8*>(src + 16 * ks + 8 * half);
  }
  // role 0: dV^T rows 256 hf .. (8 blocks); role 1: dK^T rows 288 hf .. (9 blocks)
  constexpr int NB = kTQ / 64;  // 9
  f32x16 acc[NB];
#pragma unroll
  for (int x = 0; x < NB; ++x) acc[x] = f32x16{};
  const int kl = lane & 31;

  for (int b = 0; b < n_blk; ++b) {
    // block b's copies have landed and every wave is past block b - 1
    wait_gathers();
    __syncthreads();
    if (b + 1 < n_blk) copy_block(b + 1);
    const int stg = b & 1;
    const __bf16* sq = s.q[stg];
    const __bf16* sg = s.g[stg];
    const float* meta = s.meta[stg];
    // partial S (role 0) or dP (role 1) over this wave's half of the contraction:
    // rows = the block's 32 items, columns = the keys; lane holds key kl, items
    // 8 (j / 4) + 4 half + (j % 4)
    f32x16 acc0 = f32x16{}, acc1 = f32x16{};
    const int it = lane & 31;
    if (role == 0) row_chains<true, kTQ / 32>(sq, it, half, hf * (kTQ / 2), bf, acc0, acc1);
    else row_chains<false, kTV / 32>(sg, it, half, hf * (kTV / 2), bf, acc0, acc1);
#pragma unroll
    for (int j = 0; j < 16; ++j) acc0[j] += acc1[j];
    float* xw = &s.xs[wave][lane * 16];
#pragma unroll
    for (int j = 0; j < 16; j += 4)
      *reinterpret_cast<float4*>(xw + j) = make_float4(acc0[j], acc0[j + 1], acc0[j + 2], acc0[j + 3]);
    __syncthreads();
    // P = c exp(S scale - lse) (a key the row does not select: exponent -inf);
    // role 1 also dS' = P (dP - D); both in the B layout
    const float cnt = (float)reinterpret_cast<const uint16_t*>(meta + 64)[kl];
    const float bias_off = cnt > 0.f ? 0.f : -INFINITY;
    bf16x8 ob[2];
    const float* s0 = &s.xs[0][lane * 16];
    const float* s1 = &s.xs[1][lane * 16];
    const float* po = &s.xs[role == 1 ? (wave ^ 1) : 0][lane * 16];  // role 1: the other dP half
#pragma unroll
    for (int j = 0; j < 16; j += 4) {
      float sv[4], dv4[4];
      if (role == 0) {
        const float4 o = *reinterpret_cast<const float4*>((hf ? s0 : s1) + j);
        sv[0] = acc0[j] + o.x; sv[1] = acc0[j + 1] + o.y;
        sv[2] = acc0[j + 2] + o.z; sv[3] = acc0[j + 3] + o.w;
      } else {
        const float4 x0 = *reinterpret_cast<const float4*>(s0 + j);
        const float4 x1 = *reinterpret_cast<const float4*>(s1 + j);
        const float4 o = *reinterpret_cast<const float4*>(po + j);
        sv[0] = x0.x + x1.x; sv[1] = x0.y + x1.y; sv[2] = x0.z + x1.z; sv[3] = x0.w + x1.w;
        dv4[0] = acc0[j] + o.x; dv4[1] = acc0[j + 1] + o.y;
        dv4[2] = acc0[j + 2] + o.z; dv4[3] = acc0[j + 3] + o.w;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int jj = j + u;
        const int q = 8 * (jj >> 2) + 4 * half + (jj & 3);
        const float pv = cnt * exp2_raw(fmaf(sv[u], a.scale_log2, bias_off - meta[q]));
        ob[jj >> 3][jj & 7] =
            role == 0 ? (__bf16)pv : (__bf16)(pv * (dv4[u] - meta[kTI + q]));
      }
    }
    // role 0: dV^T += dO^T P on rows 256 hf + 32 x (8 blocks); role 1: dK^T += Q^T dS'
    // on rows 288 hf + 32 x (9 blocks); each A fragment read two steps ahead
    const int nb = role == 0 ? kTV / 64 : kTQ / 64;
    auto frag = [&](int u) {  // u = NB qs + x; role 0's step x = 8 reads block 7 (unused)
      const int qs = u / NB, x = min(u % NB, nb - 1);
      return role == 0 ? trfrag<false>(sg, qs, 256 * hf + 32 * x, lane)
                       : trfrag<true>(sq, qs, 288 * hf + 32 * x, lane);
    };
    bf16x8 f0 = frag(0), f1 = frag(1);
#pragma unroll
    for (int u = 0; u < 2 * NB; ++u) {
      bf16x8 nf;
      if (u + 2 < 2 * NB) nf = frag(u + 2);
      const int qs = u / NB, x = u % NB;
      if (x < nb) acc[x] = mfma(f0, ob[qs], acc[x]);
      f0 = f1;
      f1 = nf;
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // lane holds key tk0 + kl, rows 32 x + 8 (j / 4) + 4 half + (j % 4) of its part
  float* out = part + (int64_t)kl * a.k.h * kTPart +
               (role == 0 ? kTQ + 256 * hf : 288 * hf);
  const float scl = role == 0 ? 1.f : a.scale;  // dK sums dS' = dS / scale
  const int nb = role == 0 ? kTV / 64 : kTQ / 64;
#pragma unroll
  for (int x = 0; x < NB; ++x)
    if (x < nb) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        *reinterpret_cast<float4*>(out + 32 * x + 8 * jj + 4 * half) =
            make_float4(scl * acc[x][4 * jj], scl * acc[x][4 * jj + 1], scl * acc[x][4 * jj + 2],
                        scl * acc[x][4 * jj + 3]);
    }
}

// dk, dv = the row chunks' partial sums, added in chunk order
__global__ __launch_bounds__(256) void k_bwtm_reduce(BwTokArgs a) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t per = kTPart / 4;
  const int64_t kh = t / per;  // key * Hkv + g
  if (kh >= (int64_t)a.L.n_kv * a.k.h) return;
  const int d4 = (int)(t % per) * 4;
  const int64_t stride = (int64_t)a.n_kvp * a.k.h * kTPart;
  const float* p = a.part + kh * kTPart + d4;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int c = 0; c < a.n_chunks; ++c) {
    const float4 x = *reinterpret_cast<const float4*>(p + c * stride);
    acc.x += x.x;
    acc.y += x.y;
    acc.z += x.z;
    acc.w += x.w;
  }
  if (d4 < kTQ) *reinterpret_cast<float4*>(a.dk + kh * kTQ + d4) = acc;
  else *reinterpret_cast<float4*>(a.dv + kh * kTV + (d4 - kTQ)) = acc;
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
  __bf16 ds[2][4][32 * kDS];  // [stage][wave][head][slot]
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

// one workgroup per (row, key head); wave w takes query heads g G + 32 w ..
template <bool VA>
__global__ __launch_bounds__(256, 1) void k_bwtm_ds(BwTokArgs a) {
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
  __bf16* dsrow = a.ds + pair * a.w32;
  bf16x8 prev[2];  // the previous tile's dS', stored once the next tile is under way
  // lane holds slots 32 t + 8 jj + 4 half + 0 .. 3 in prev[jj / 2][4 (jj % 2) ..]
  auto store_prev = [&](int t) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      bf16x4 v;
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = prev[jj >> 1][4 * (jj & 1) + u];
      *reinterpret_cast<bf16x4*>(dsrow + kDS * t + 8 * jj + 4 * half) = v;
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
    }
  }
  store_prev(n_t - 1);
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

__global__ __launch_bounds__(256, 1) void k_bwtm_dq(BwTokArgs a) {
  __shared__ DqLds s;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int nw = blockDim.x / kWave;
  const int half = lane >> 5;
  const int i = blockIdx.x / a.k.h, g = blockIdx.x % a.k.h;
  const int hq = a.q.h, G = hq / a.k.h;
  const int h0 = g * G + 32 * wave;  // this wave's first head
  const int kfb = stage_slots(a, i, s.key);
  __syncthreads();
  const int n_t = (a.idx_width + kDS - 1) / kDS;
  // this wave's dS' tile t (32 heads x 32 slots, 2 KiB) into stage st
  auto copy_ds = [&](int t, int st) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int byte = 1024 * u + 16 * lane;
      const int hl = byte / (2 * kDS), sl = (byte % (2 * kDS)) / 2;
      const __bf16* src = a.ds + ((int64_t)i * hq + h0 + hl) * a.w32 + kDS * t + sl;
      gather16_addr(src, __builtin_amdgcn_readfirstlane(lds_addr(&s.ds[st][wave][0]) + 1024 * u));
    }
  };
  gather_tile<true>(a, g, s.key, kfb, 0, s.k[0], nullptr, nw, wave, lane);
  copy_ds(0, 0);
  constexpr int NB = kTQ / 32;  // 18 column blocks of dQ
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
    const __bf16* dt = s.ds[t & 1][wave];
    // A operands: dS' rows of the wave's heads (m = head lane % 32), slots 16 qs + 8 half ..
    const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(dt + (lane & 31) * kDS + 8 * half);
    const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(dt + (lane & 31) * kDS + 16 + 8 * half);
    bf16x8 f0 = trnat(kt, 0, 0, lane), f1 = trnat(kt, 0, 32, lane);
#pragma unroll
    for (int u = 0; u < 2 * NB; ++u) {  // u = NB qs + x
      bf16x8 nf;
      if (u + 2 < 2 * NB) nf = trnat(kt, (u + 2) / NB, 32 * ((u + 2) % NB), lane);
      acc[u % NB] = mfma(u < NB ? a0 : a1, f0, acc[u % NB]);
      f0 = f1;
      f1 = nf;
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // lane holds column 32 x + lane % 32, heads h0 + 8 (j / 4) + 4 half + (j % 4)
  const float scl = a.scale;  // dQ sums dS' = dS / scale
#pragma unroll
  for (int x = 0; x < NB; ++x)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int hh = h0 + 8 * (j >> 2) + 4 * half + (j & 3);
      a.dq[((int64_t)i * hq + hh) * kTQ + 32 * x + (lane & 31)] = scl * acc[x][j];
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

int attn_bwd_token_chunks(int n_q) { return (n_q + kTRows - 1) / kTRows; }
int attn_bwd_token_kvp(int n_kv) { return (n_kv + kTK - 1) / kTK * kTK; }
int attn_bwd_token_w32(int idx_width) { return (idx_width + kDS - 1) / kDS * kDS; }

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
  const int64_t words = (int64_t)a.L.n_q * a.n_kvp / 2;
  if (words > 0) {
    hipLaunchKernelGGL(k_bwtm_fill, dim3((unsigned)std::min<int64_t>(4096, grid_of(words, 256))),
                       dim3(256), 0, stream, reinterpret_cast<uint32_t*>(a.cmap), words);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (pairs > 0) {
    hipLaunchKernelGGL(k_bwtm_count, dim3(grid_of((int64_t)a.L.n_q * a.idx_width, 256)),
                       dim3(256), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(k_bwtm_rec, dim3(grid_of(pairs, 256)), dim3(256), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
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
  const int64_t wgs = (int64_t)a.k.h * (a.n_kvp / kTK) * a.n_chunks;
  int slot;
  trace_begin(stream, "k_bwtm_dkdv", &slot);
  hipLaunchKernelGGL(k_bwtm_dkdv, dim3((unsigned)wgs), dim3(kTT), 0, stream, a);
  trace_end(stream, slot);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_bwtm_reduce,
                     dim3(grid_of((int64_t)a.L.n_kv * a.k.h * (kTPart / 4), 256)), dim3(256), 0,
                     stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (a.L.n_q == 0) return hipSuccess;
  const int G = a.q.h / a.k.h;
  const dim3 grid((unsigned)((int64_t)a.L.n_q * a.k.h)), block((unsigned)(G / 32 * kWave));
  const bool va = a.v.data == a.k.data && a.v.stride_n == a.k.stride_n &&
                  a.v.stride_h == a.k.stride_h;
  trace_begin(stream, "k_bwtm_ds", &slot);
  if (va) hipLaunchKernelGGL(k_bwtm_ds<true>, grid, block, 0, stream, a);
  else hipLaunchKernelGGL(k_bwtm_ds<false>, grid, block, 0, stream, a);
  trace_end(stream, slot);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  trace_begin(stream, "k_bwtm_dq", &slot);
  hipLaunchKernelGGL(k_bwtm_dq, grid, block, 0, stream, a);
  trace_end(stream, slot);
  return hipGetLastError();
}

}  // namespace csa
