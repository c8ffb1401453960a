// Token-mode sparse shard attention on the matrix cores (bf16 MFMA, gfx950).
//
// Megatron-LM PR #3674 ("[1/2] Enable DSA CP, THD with absorbed MLA",
// Description and sequence diagram): each query token attends to the top-k key
// tokens its indexer picked, and with absorbed MLA all query heads share one
// latent key head whose first columns are also the value.  Megatron-LM issue
// #4878 ("Strategy: allgather CP mode"): the sparse kernel iterates only over
// the top-k indices, never materialising the full score matrix.
//
// One workgroup per (query token, key head) with the G = Hq / Hkv query heads
// of that key head as the 32-wide query tiles of G / 32 waves.  The token's
// selected keys are gathered 32 at a time into a row-major LDS tile (padded
// rows plus a one-bit unit swizzle on row bit 3: conflict-free for both read
// patterns).
// S^T = K Q^T runs on 32x32x16 bf16 MFMA with Q^T in registers; the softmax
// state lives in the lane of its query.  O^T = V^T P^T reads V^T straight from
// the row-major tile with the transposing LDS read (ds_read_b64_tr_b16): in a
// 16-lane group, lane c addressing 4 values of key kb + c/4 at value column
// dvb + 4 (c % 4) makes lane t receive column dvb + t of keys kb .. kb + 3.
// When the value aliases the key (absorbed MLA) no second tile exists at all.
// The running maximum is raised only when a score exceeds it by 2^8 (scores
// stay bounded by 2^8 in between), so the 16 x Dv/32 accumulators are rarely
// rescaled.  Chunk summaries merge exactly as in "Context parallel attention:
// exchange keys and merge softmax globally" (chunk summary paragraph).
#include <type_traits>

#include "attention.hpp"
#include "gather.hpp"
#include "mfma.hpp"

namespace csa {

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kTK = 32;          // gathered keys per tile
constexpr int kKD = 2;           // key (and LDS query) fragment reads in flight ahead of use
constexpr int kVD = 2;           // transposed value fragment reads in flight ahead of use
constexpr float kLazy = 8.0f;    // log2 headroom before the running max moves
constexpr float kLn2 = 0.69314718055994531f;

// Query fragments kept in LDS instead of registers (the 576-wide shape would
// otherwise not fit its query, accumulators and fragment pipeline in 512 registers).
template <int DQK, bool ALIAS>
constexpr int q_in_lds() { return DQK == 576 ? (ALIAS ? 8 : 4) : 0; }

template <int DQK, int DV, bool ALIAS, int NW>
struct TokLds {
  static constexpr int kPitch = DQK + 16;  // bf16 elements per K row
  static constexpr int kVPitch = DV + 16;
  static constexpr int kQL = q_in_lds<DQK, ALIAS>();
  __bf16 k[2][kTK * kPitch];
  __bf16 v[ALIAS ? 1 : 2][ALIAS ? 8 : kTK * kVPitch];
  bf16x8 q[NW][kQL > 0 ? kQL : 1][kWave];  // [wave][fragment][lane]
};

// byte offset of element e (a multiple of 4) of row r in a padded, swizzled tile.
// The 16-byte units of rows 8..15 of every 16 are swapped in pairs: with a
// pitch of an even number of units (2 (D + 16) bytes) the sixteen rows that one
// phase of a ds_read_b128 touches then fall on distinct banks (measured on
// gfx950: 152 B/clk per CU against 113 with the swap on rows 4..7 of every 8),
// and the transposing value reads stay conflict-free.
// The 16-heads-a-wave kernel's read patterns (16 rows x 4 units per ds_read_b128, 4
// rows x 32 bytes per 16-lane group of the transposing read) are conflict-free with
// the swap on row bit 2 instead (SQ_LDS_BANK_CONFLICT 0 for both; bit 3 costs ~4
// conflict cycles per ds_read_b128).
template <int PITCH, int SB = 3>
__device__ __forceinline__ int tile_off(int r, int e) {
  const int unit = (e >> 3) ^ ((r >> SB) & 1);
  return r * PITCH * 2 + unit * 16 + (e & 7) * 2;
}

__device__ __forceinline__ bf16x4 read_tr(const __bf16* lds_base, int byte_off) {
  typedef __attribute__((address_space(3))) s16x4* lds_ptr;
  typedef __attribute__((address_space(3))) char* lds_bytes;
  const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_ptr)((lds_bytes)(const_cast<__bf16*>(lds_base)) + byte_off));
  return __builtin_bit_cast(bf16x4, x);
}

// x * s for an accumulator value that stays in an accumulator register
// (VALU instructions cannot read accumulator registers directly).
__device__ __forceinline__ float acc_scale(float x, float s) {
  float y, t;
  asm volatile(
      "v_accvgpr_read_b32 %1, %2\n\t"
      "v_mul_f32 %1, %1, %3\n\t"
      "v_accvgpr_write_b32 %0, %1"
      : "=a"(y), "=&v"(t)
      : "a"(x), "v"(s));
  return y;
}

// Gathers one tile straight into LDS with global_load_lds_dwordx4: an
// instruction fills 1 KiB of LDS, lane l writing bytes [16 l, 16 l + 16) of
// it, so each lane loads the 16 bytes that the padded, swizzled layout puts at
// its destination (pad slots re-read unit 0 of their row).  The tile sizes are
// whole KiBs (32 rows of 2 (D + 16) bytes).  No registers hold the data.
// (gather16_addr of gather.hpp: one instruction per KiB, the source as a
// 64-bit address per lane, since a chunk spans rows of different tokens).
template <int D, int SB = 3>
__device__ __forceinline__ void issue_tile(const View& T, int g, const int* keys, __bf16* tile,
                                           int wave, int nwaves) {
  constexpr int kPitchB = 2 * (D + 16);
  constexpr int kChunks = kTK * kPitchB / 1024;
  static_assert(kTK * kPitchB % 1024 == 0, "tile must be whole KiBs");
  const int lane = threadIdx.x & (kWave - 1);
  typedef __attribute__((address_space(3))) char* lds_bytes;
  for (int ch = wave; ch < kChunks; ch += nwaves) {
    const int byte = ch * 1024 + lane * 16;
    const int row = byte / kPitchB;
    const int pu = (byte - row * kPitchB) >> 4;
    const int u = pu < D / 8 ? (pu ^ ((row >> SB) & 1)) : 0;
    const __bf16* src = elem_ptr<__bf16>(T, keys[row], g) + u * 8;
    const uint32_t dst = static_cast<uint32_t>(
        reinterpret_cast<uintptr_t>((lds_bytes)(void*)tile + ch * 1024));
    gather16_addr(src, __builtin_amdgcn_readfirstlane(dst));
  }
}

template <int DQK, int DV, bool ALIAS, int NW, typename TO>
__global__ __launch_bounds__(NW * kWave, 1) void k_tok_attn(AttnKernelArgs a) {
  using Lds = TokLds<DQK, DV, ALIAS, NW>;
  constexpr int NQR = DQK / 16 - Lds::kQL;  // query fragments held in registers
  __shared__ Lds s;
  // slot keys of tiles kt, kt + 1 and kt + 2 live in distinct slots (kt % 3)
  __shared__ int s_keys[3][kTK];
  __shared__ int s_valid[3][kTK];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // uniform: scalar branches
  const int half = lane >> 5;
  const int hkv = a.k.h;
  const int i = blockIdx.x / hkv;
  const int g = blockIdx.x % hkv;
  const int G = a.q.h / hkv;
  const int head = g * G + wave * 32 + (lane & 31);
  const RowKeys r = row_keys(a.L, i);
  const int W = a.idx_width;
  const int32_t* slots = a.idx + (int64_t)i * W;
  const float c = a.scale_log2;

  bf16x8 qf[NQR];
  {
    const __bf16* qp = elem_ptr<__bf16>(a.q, i, head);
#pragma unroll
    for (int ks = 0; ks < NQR; ++ks)
      qf[ks] = *reinterpret_cast<const bf16x8*>(qp + 16 * ks + 8 * half);
#pragma unroll
    for (int ks = NQR; ks < DQK / 16; ++ks)
      s.q[wave][ks - NQR][lane] = *reinterpret_cast<const bf16x8*>(qp + 16 * ks + 8 * half);
  }
  f32x16 o[DV / 32];  // in AGPRs
#pragma unroll
  for (int dt = 0; dt < DV / 32; ++dt) to_agpr(o[dt], f32x16{});
  float m = -INFINITY, l = 0.f;

  const int n_kt = r.valid ? (W + kTK - 1) / kTK : 0;
  // slot key of tile kt for thread t < kTK (loaded a tile ahead of its store,
  // so that the load's latency hides under a tile of MFMAs)
  auto load_key = [&](int kt) {
    const int j = kt * kTK + threadIdx.x;
    return (threadIdx.x < kTK && j < W) ? slots[j] : -1;
  };
  auto store_key = [&](int kt, int key) {
    if (threadIdx.x < kTK) {
      const bool ok = key >= r.lo && key <= r.hi;
      s_keys[kt % 3][threadIdx.x] = ok ? key : r.lo;  // masked slots read a valid row
      s_valid[kt % 3][threadIdx.x] = ok;
    }
  };
  auto fetch_keys = [&](int kt) { store_key(kt, load_key(kt)); };
  auto issue = [&](int kt) {
    issue_tile<DQK>(a.k, g, s_keys[kt % 3], s.k[kt & 1], wave, NW);
    if constexpr (!ALIAS) issue_tile<DV>(a.v, g, s_keys[kt % 3], s.v[ALIAS ? 0 : (kt & 1)], wave, NW);
  };
  if (n_kt > 0) {
    fetch_keys(0);
    if (n_kt > 1) fetch_keys(1);
    __syncthreads();
    issue(0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  for (int kt = 0; kt < n_kt; ++kt) {
    const int buf = kt & 1;
    const int ks3 = kt % 3;
    const int key2 = kt + 2 < n_kt ? load_key(kt + 2) : -1;
    // S^T = K Q^T: lane holds keys 8 (j / 4) + 4 half + (j % 4) of its query.
    // Two accumulators (even and odd steps) keep consecutive MFMAs independent;
    // fragment reads run two MFMAs ahead.
    const char* kb = reinterpret_cast<const char*>(s.k[buf]);
    f32x16 sc;
    {
      constexpr int NK = DQK / 16;
      const int row = lane & 31;
      auto kfrag = [&](int ks) {
        return *reinterpret_cast<const bf16x8*>(kb + tile_off<Lds::kPitch>(row, 16 * ks + 8 * half));
      };
      // query fragments past NQR come from LDS, read along with the key fragment
      auto qlds = [&](int ks) { return s.q[wave][ks - NQR][lane]; };
      f32x16 sab[2];  // even and odd steps
      bf16x8 ka[kKD + 1], qa[kKD + 1];
#pragma unroll
      for (int t = 0; t < kKD; ++t) {
        ka[t] = kfrag(t);
        if (t >= NQR) qa[t] = qlds(t);
      }
#pragma unroll
      for (int ks = 0; ks < NK; ++ks) {
        if (ks + kKD < NK) {
          ka[(ks + kKD) % (kKD + 1)] = kfrag(ks + kKD);
          if (ks + kKD >= NQR) qa[(ks + kKD) % (kKD + 1)] = qlds(ks + kKD);
        }
        const bf16x8 q = ks < NQR ? qf[ks < NQR ? ks : 0] : qa[ks % (kKD + 1)];
        if (ks < 2)
          mfma_v0(sab[ks], ka[ks % (kKD + 1)], q);
        else
          mfma_v(sab[ks & 1], ka[ks % (kKD + 1)], q);
        // the next tile's gather (into the other buffer) is issued once the
        // first MFMAs run, so that its address work overlaps them
        if (ks == 3 && kt + 1 < n_kt) issue(kt + 1);
        __builtin_amdgcn_sched_barrier(0);
      }
      fence_v(sab);
#pragma unroll
      for (int j = 0; j < 16; ++j) sc[j] = sab[0][j] + sab[1][j];
    }
    // O^T += V^T P^T with V^T read transposed from the row-major tile: the first
    // kVD fragment reads are issued before the softmax, and each MFMA has the
    // reads of the next kVD in flight
    const __bf16* vbase = ALIAS ? s.k[buf] : s.v[ALIAS ? 0 : buf];
    constexpr int VP = ALIAS ? Lds::kPitch : Lds::kVPitch;
    constexpr int NO = 2 * (DV / 32);  // MFMA i: key step i / (DV / 32), value block i % (DV / 32)
    const int c16 = lane & 15;
    const int grp = lane >> 4;
    auto vfrag = [&](int i) {
      const int st = i / (DV / 32), dt = i % (DV / 32);
      const int ka_ = 16 * st + 4 * half + (c16 >> 2);
      const int dv = dt * 32 + 16 * (grp & 1) + 4 * (c16 & 3);
      const bf16x4 lo = read_tr(vbase, tile_off<VP>(ka_, dv));
      const bf16x4 hi = read_tr(vbase, tile_off<VP>(ka_ + 8, dv));
      return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    bf16x8 va[kVD + 1];
#pragma unroll
    for (int t = 0; t < kVD; ++t) va[t] = vfrag(t);

    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int kl = 8 * (j >> 2) + 4 * half + (j & 3);
      if (!s_valid[ks3][kl]) sc[j] = -INFINITY;
      mx = fmaxf(mx, sc[j]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave)) * c;
    const bool need = mx > m + kLazy || (m == -INFINITY && mx > -INFINITY);
    if (__any(need)) {
      fence_a(o);
      const float mn = need ? mx : m;
      const float alpha = (m == -INFINITY) ? 0.f : exp2f(m - mn);
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < DV / 32; ++dt)
#pragma unroll
        for (int j = 0; j < 16; ++j) o[dt][j] = acc_scale(o[dt][j], alpha);
      m = mn;
    }
    const float mu = (m == -INFINITY) ? 0.f : m;
    float rs = 0.f;
    bf16x8 pb[2];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float p = __builtin_amdgcn_exp2f(fmaf(sc[j], c, -mu));
      rs += p;
      pb[j >> 3][j & 7] = (__bf16)p;
    }
    rs += __shfl_xor(rs, 32, kWave);
    l += rs;
    {
#pragma unroll
      for (int i = 0; i < NO; ++i) {
        if (i + kVD < NO) va[(i + kVD) % (kVD + 1)] = vfrag(i + kVD);
        const int st = i / (DV / 32), dt = i % (DV / 32);
        mfma_a(o[dt], va[i % (kVD + 1)], pb[st]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (kt + 2 < n_kt) store_key(kt + 2, key2);
    __builtin_amdgcn_s_waitcnt(0);  // the next tile's direct loads have landed
    __syncthreads();
  }

  fence_a(o);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  if (a.lse && half == 0)
    a.lse[(int64_t)i * a.q.h + head] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
  // bf16: the wave's 32 heads are 32 consecutive output rows.  Where the key
  // tiles are large enough, they go through the wave's part of that (now free)
  // buffer, at most 256 columns at a time, and out as whole row pieces, 16 bytes
  // a lane, where 8-byte stores would spread each row over many instructions.
  constexpr int kPart = DV > 256 ? 256 : DV;
  constexpr int kRowB = kPart * 2 + 16;  // staged row pitch in bytes (padded)
  constexpr bool kStage = sizeof(TO) == 2 && NW * 32 * kRowB <= (int)sizeof(s.k);
  if constexpr (kStage) {
    constexpr int kUnits = kPart / 8;  // 16-byte units of a row piece
    char* st = reinterpret_cast<char*>(&s.k[0][0]) + wave * 32 * kRowB;
    __bf16* wout = reinterpret_cast<__bf16*>(a.out) +
                   ((int64_t)i * a.q.h + g * G + wave * 32) * DV;
#pragma unroll
    for (int pc = 0; pc < DV / kPart; ++pc) {
#pragma unroll
      for (int dt = pc * kPart / 32; dt < (pc + 1) * kPart / 32; ++dt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const bf16x4 x = {(__bf16)(o[dt][4 * jj] * inv), (__bf16)(o[dt][4 * jj + 1] * inv),
                            (__bf16)(o[dt][4 * jj + 2] * inv), (__bf16)(o[dt][4 * jj + 3] * inv)};
          *reinterpret_cast<bf16x4*>(st + (lane & 31) * kRowB +
                                     (dt * 32 + 8 * jj + 4 * half - pc * kPart) * 2) = x;
        }
#pragma unroll
      for (int e0 = 0; e0 < 32 * kUnits; e0 += kWave) {
        const int r = (e0 + lane) / kUnits, un = (e0 + lane) % kUnits;
        *reinterpret_cast<uint4*>(wout + (int64_t)r * DV + pc * kPart + un * 8) =
            *reinterpret_cast<const uint4*>(st + r * kRowB + un * 16);
      }
    }
    return;
  }
  TO* out = reinterpret_cast<TO*>(a.out) + ((int64_t)i * a.q.h + head) * DV;
#pragma unroll
  for (int dt = 0; dt < DV / 32; ++dt)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int d = dt * 32 + 8 * jj + 4 * half;
      if constexpr (sizeof(TO) == 4) {
        *reinterpret_cast<float4*>(out + d) =
            make_float4(o[dt][4 * jj] * inv, o[dt][4 * jj + 1] * inv, o[dt][4 * jj + 2] * inv,
                        o[dt][4 * jj + 3] * inv);
      } else {
        bf16x4 x = {(__bf16)(o[dt][4 * jj] * inv), (__bf16)(o[dt][4 * jj + 1] * inv),
                    (__bf16)(o[dt][4 * jj + 2] * inv), (__bf16)(o[dt][4 * jj + 3] * inv)};
        *reinterpret_cast<bf16x4*>(out + d) = x;
      }
    }
}

// Max and sum over lanes l and l ^ 16 (or l ^ 32) with the VALU lane swaps of gfx950:
// each swap returns the pair (value of the lower, value of the upper 16- or 32-lane
// group) in both lanes, so both lanes compute the same result in the same order.
// (__shfl_xor goes through ds_bpermute, which queues behind the other wave's LDS reads.)
__device__ __forceinline__ float pair16_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair16_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Absorbed-MLA widths (Dqk = 576, Dv = 512, V = the key's first 512 columns): 16 query
// heads per wave on 16x16x32 MFMAs, so that a wave's Q^T fragments (72 registers) and
// output accumulators (128) fit in half a SIMD's register file and two waves share
// each SIMD: one wave's gather issue and softmax then run under the other's MFMAs
// (a single wave per SIMD, as with 32 heads a wave, leaves the matrix core idle
// through both).  This kernel serves 32 and 64 heads a key head (two workgroups a CU
// at 64); 128 heads take the paired form below.  Per 32-key tile each wave forms S^T = K Q^T over 18 column steps
// for two 16-key halves, the softmax of its heads, and O^T += V^T P^T with the keys
// in the order its score accumulators hold them: key k of step position 8 quad + t
// is 4 quad + t (t < 4) or 16 + 4 quad + t - 4.
template <int NW, typename TO>
__global__ __launch_bounds__(NW * kWave, NW == 4 ? 2 : 1) void k_tok_attn16(AttnKernelArgs a) {
  constexpr int DQK = 576, DV = 512;
  constexpr int kPitch = DQK + 16;
  constexpr int NKS = DQK / 32;  // score steps
  constexpr int NDB = DV / 16;   // output blocks of 16 columns
  constexpr int NBUF = 2;
  __shared__ __bf16 s_k[NBUF][kTK * kPitch];
  __shared__ int s_keys[3][kTK];
  __shared__ __align__(16) float s_bias[3][kTK];  // 0: permitted key; -inf: masked slot
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int quad = lane >> 4, c16 = lane & 15;
  const int hkv = a.k.h;
  const int i = blockIdx.x / hkv;
  const int g = blockIdx.x % hkv;
  const int G = a.q.h / hkv;
  const int head = g * G + wave * 16 + c16;
  const RowKeys r = row_keys(a.L, i);
  const int W = a.idx_width;
  const int32_t* slots = a.idx + (int64_t)i * W;
  const float c = a.scale_log2;

  // B operands: Q^T [32 columns x 16 heads], lane: head c16, columns 32 ks + 8 quad ..
  bf16x8 qf[NKS];
  {
    const __bf16* qp = elem_ptr<__bf16>(a.q, i, head);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      qf[ks] = *reinterpret_cast<const bf16x8*>(qp + 32 * ks + 8 * quad);
  }
  f32x4 o[NDB];  // O^T: lane holds head c16, columns 16 db + 4 quad + 0 .. 3
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;

  const int n_kt = r.valid ? (W + kTK - 1) / kTK : 0;
  auto load_key = [&](int kt) {
    const int j = kt * kTK + threadIdx.x;
    return (threadIdx.x < kTK && j < W) ? slots[j] : -1;
  };
  auto store_key = [&](int kt, int key) {
    if (threadIdx.x < kTK) {
      const bool ok = key >= r.lo && key <= r.hi;
      s_keys[kt % 3][threadIdx.x] = ok ? key : r.lo;  // masked slots read a valid row
      s_bias[kt % 3][threadIdx.x] = ok ? 0.f : -INFINITY;
    }
  };
  auto issue = [&](int kt) { issue_tile<DQK, 2>(a.k, g, s_keys[kt % 3], s_k[kt % NBUF], wave, NW); };
  if (n_kt > 0) {
    store_key(0, load_key(0));
    if (n_kt > 1) store_key(1, load_key(1));
    __syncthreads();
    issue(0);
  }
  // on every path, so that no wait for the Q fragments stays inside the loop (where
  // it would also wait for the next tile's gather)
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // per-lane byte offsets: score A operands (rows c16 and 16 + c16, column unit
  // 4 ks + quad, swapped on row bit 2: the swap stays within the low two unit bits,
  // so step ks adds 64 ks bytes) and value A operands (the two 4-key groups)
  const int ka0 = tile_off<kPitch, 2>(c16, 8 * quad);
  const int ka1 = tile_off<kPitch, 2>(16 + c16, 8 * quad);
  const int va0 = tile_off<kPitch, 2>(4 * quad + (c16 >> 2), 4 * (c16 & 3));
  const int va1 = tile_off<kPitch, 2>(16 + 4 * quad + (c16 >> 2), 4 * (c16 & 3));
  bf16x8 pb;  // P^T of the tile
  // O^T += V^T P^T over tile buffer b.  Value A operand of block db: columns
  // 16 db + c16 of the lane's two key groups, read transposed (lane c16 of a 16-lane
  // group addresses key base + c16 / 4 at column 16 db + 4 (c16 % 4) and receives
  // column 16 db + c16 of the 4 keys); each MFMA has the next kVF in flight.
  auto pv = [&](int b) {
    constexpr int kVF = 3;
    const __bf16* vt = s_k[b];
    auto vf = [&](int db) {
      const bf16x4 lo = read_tr(vt, va0 + 32 * db);
      const bf16x4 hi = read_tr(vt, va1 + 32 * db);
      return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    bf16x8 vfr[kVF + 1];
#pragma unroll
    for (int t = 0; t < kVF; ++t) vfr[t] = vf(t);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      if (db + kVF < NDB) vfr[(db + kVF) % (kVF + 1)] = vf(db + kVF);
      o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vfr[db % (kVF + 1)], pb, o[db], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  for (int kt = 0; kt < n_kt; ++kt) {
    const int buf = kt % NBUF;
    const int ks3 = kt % 3;
    const int key2 = kt + 2 < n_kt ? load_key(kt + 2) : -1;
    const char* kb = reinterpret_cast<const char*>(s_k[buf]);
    // the scores start from the slots' bias: a masked slot's score is -inf exactly
    // (its key row is a valid one, so every product is finite)
    f32x4 s0 = *reinterpret_cast<const f32x4*>(&s_bias[ks3][4 * quad]);
    f32x4 s1 = *reinterpret_cast<const f32x4*>(&s_bias[ks3][16 + 4 * quad]);
    {
      // MFMA j = 2 ks + half takes the key fragment of rows 16 half + c16 at step ks;
      // fragments sit in a ring of four, read three MFMAs ahead of their use
      auto kf = [&](int j) {
        return *reinterpret_cast<const bf16x8*>(kb + ((j & 1) ? ka1 : ka0) + 64 * (j >> 1));
      };
      bf16x8 fr[4];
#pragma unroll
      for (int j = 0; j < 3; ++j) fr[j] = kf(j);
#pragma unroll
      for (int j = 0; j < 2 * NKS; ++j) {
        if (j + 3 < 2 * NKS) fr[(j + 3) & 3] = kf(j + 3);
        if (j & 1)
          s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fr[j & 3], qf[j >> 1], s1, 0, 0, 0);
        else
          s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fr[j & 3], qf[j >> 1], s0, 0, 0, 0);
        if (j == 3 && kt + 1 < n_kt) issue(kt + 1);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // lane: head c16, keys 4 quad + t (s0) and 16 + 4 quad + t (s1)
    float x[8];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      x[t] = s0[t];
      x[4 + t] = s1[t];
    }
    float mx = x[0];
#pragma unroll
    for (int t = 1; t < 8; ++t) mx = fmaxf(mx, x[t]);
    mx = pair32_max(pair16_max(mx)) * c;
    const bool need = mx > m + kLazy || (m == -INFINITY && mx > -INFINITY);
    if (__any(need)) {
      const float mn = need ? mx : m;
      const float alpha = (m == -INFINITY) ? 0.f : exp2f(m - mn);
      l *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int t = 0; t < 4; ++t) o[db][t] *= alpha;
      m = mn;
    }
    const float mu = (m == -INFINITY) ? 0.f : m;
    float rs = 0.f;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float p = __builtin_amdgcn_exp2f(fmaf(x[t], c, -mu));
      rs += p;
      pb[t] = (__bf16)p;
    }
    l += pair32_sum(pair16_sum(rs));
    pv(buf);
    if (kt + 2 < n_kt) store_key(kt + 2, key2);
    __builtin_amdgcn_s_waitcnt(0);  // the next tile's direct loads have landed
    __syncthreads();
  }

  const float inv = l > 0.f ? 1.f / l : 0.f;
  if (a.lse && quad == 0)
    a.lse[(int64_t)i * a.q.h + head] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
  if constexpr (sizeof(TO) == 2) {
    // the wave's 16 heads are 16 consecutive output rows: through the (now free) key
    // tiles 256 columns at a time, then out as whole 16-byte row pieces
    constexpr int kPart = 256;
    constexpr int kRowB = kPart * 2 + 16;
    static_assert(NW * 16 * kRowB <= (int)sizeof(s_k), "staging fits the key tiles");
    char* st = reinterpret_cast<char*>(&s_k[0][0]) + wave * 16 * kRowB;
    __bf16* wout = reinterpret_cast<__bf16*>(a.out) + ((int64_t)i * a.q.h + g * G + wave * 16) * DV;
#pragma unroll
    for (int pc = 0; pc < DV / kPart; ++pc) {
#pragma unroll
      for (int db = pc * kPart / 16; db < (pc + 1) * kPart / 16; ++db) {
        const bf16x4 x4 = {(__bf16)(o[db][0] * inv), (__bf16)(o[db][1] * inv),
                           (__bf16)(o[db][2] * inv), (__bf16)(o[db][3] * inv)};
        *reinterpret_cast<bf16x4*>(st + c16 * kRowB + (16 * db + 4 * quad - pc * kPart) * 2) = x4;
      }
#pragma unroll
      for (int e0 = 0; e0 < 16 * (kPart / 8); e0 += kWave) {
        const int rr = (e0 + lane) / (kPart / 8), un = (e0 + lane) % (kPart / 8);
        *reinterpret_cast<uint4*>(wout + (int64_t)rr * DV + pc * kPart + un * 8) =
            *reinterpret_cast<const uint4*>(st + rr * kRowB + un * 16);
      }
    }
  } else {
    float* out = reinterpret_cast<float*>(a.out) + ((int64_t)i * a.q.h + head) * DV;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      *reinterpret_cast<float4*>(out + 16 * db + 4 * quad) =
          make_float4(o[db][0] * inv, o[db][1] * inv, o[db][2] * inv, o[db][3] * inv);
  }
}

// 128 query heads a key head: waves w and w + 4 (one SIMD) form S^T and the softmax
// of their own 16 heads as above and publish P (bf16) and their heads' running-maximum
// factors in LDS; one tile later each of the two forms O^T += V^T P^T for all 32 heads
// of the pair on 32x32x16 MFMAs, wave w over output columns 0 .. 255 and wave w + 4
// over 256 .. 511, so that every transposing value read serves 32 heads (half the
// value reads of 16 heads a wave).  Both waves form S and the softmax of tile t and
// then the pair's P V of tile t - 1, except that wave w + 4 runs the first kPre of
// the 16 P V steps before its scores: the small offset keeps the two waves' softmaxes
// apart (a whole P V ahead, or none, measured slower).
//   Key order of the P V step st (keys 16 st .. 16 st + 15): lane half h takes keys
// 16 st + h + 2 j (j < 4) and 16 st + h + 8 + 2 (j - 4): rows two apart start 16
// banks apart at this pitch, so each 32-lane half of a transposing read covers the 64
// banks once; P sits in LDS in that order (per step: even keys, then odd keys).
template <typename TO>
__global__ __launch_bounds__(512, 1) void k_tok_attn16p(AttnKernelArgs a) {
  constexpr int DQK = 576, DV = 512, NW = 8;
  constexpr int kPitch = DQK + 16;
  constexpr int NKS = DQK / 32;  // score steps
  constexpr int kPP = 40;        // P row pitch (bf16): 32 key positions + pad
  constexpr int kPre = 4;        // P V steps wave w + 4 runs before its scores
  __shared__ __bf16 s_k[3][kTK * kPitch];
  __shared__ __bf16 s_p[2][4][32 * kPP];  // [tile parity][pair][pair head][key position]
  __shared__ float s_al[2][4][32];        // [tile parity][pair][pair head]: factor
  __shared__ float s_l[4][32];
  __shared__ int s_keys[3][kTK];
  __shared__ __align__(16) float s_bias[3][kTK];  // 0: permitted key; -inf: masked slot
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int quad = lane >> 4, c16 = lane & 15, half = lane >> 5;
  const int pr = wave & 3, side = wave >> 2;  // pair, and which half of the columns
  const int hcol = 16 * side + c16;           // the lane's own head as a pair column
  const int hkv = a.k.h;
  const int i = blockIdx.x / hkv;
  const int g = blockIdx.x % hkv;
  const int G = a.q.h / hkv;
  const int head = g * G + wave * 16 + c16;
  const RowKeys r = row_keys(a.L, i);
  const int W = a.idx_width;
  const int32_t* slots = a.idx + (int64_t)i * W;
  const float c = a.scale_log2;

  bf16x8 qf[NKS];  // B operands Q^T [32 columns x 16 heads]
  {
    const __bf16* qp = elem_ptr<__bf16>(a.q, i, head);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      qf[ks] = *reinterpret_cast<const bf16x8*>(qp + 32 * ks + 8 * quad);
  }
  // O^T of the pair: lane holds pair head lane % 32, columns 256 side + 32 db + 8 (j / 4)
  // + 4 half + (j % 4)
  f32x16 o[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) o[db] = f32x16{};
  float m = -INFINITY, l = 0.f;

  const int n_kt = r.valid ? (W + kTK - 1) / kTK : 0;
  auto load_key = [&](int kt) {
    const int j = kt * kTK + threadIdx.x;
    return (threadIdx.x < kTK && j < W) ? slots[j] : -1;
  };
  auto store_key = [&](int kt, int key) {
    if (threadIdx.x < kTK) {
      const bool ok = key >= r.lo && key <= r.hi;
      s_keys[kt % 3][threadIdx.x] = ok ? key : r.lo;  // masked slots read a valid row
      s_bias[kt % 3][threadIdx.x] = ok ? 0.f : -INFINITY;
    }
  };
  auto issue = [&](int kt) { issue_tile<DQK, 2>(a.k, g, s_keys[kt % 3], s_k[kt % 3], wave, NW); };
  if (n_kt > 0) {
    store_key(0, load_key(0));
    if (n_kt > 1) store_key(1, load_key(1));
    __syncthreads();
    issue(0);
  }
  __builtin_amdgcn_s_waitcnt(0);  // on every path: no wait for the Q loads in the loop
  __syncthreads();
  const int ka0 = tile_off<kPitch, 2>(c16, 8 * quad);
  const int ka1 = tile_off<kPitch, 2>(16 + c16, 8 * quad);
  // value A operand (V^T [32 columns x 16 keys]) of step st and 32-column block db:
  // lane c16 of a 16-lane group addresses key 16 st + half + 2 (c16 / 4) (+ 8) at
  // column 256 side + 32 db + 16 (group % 2) + 4 (c16 % 4), and receives column
  // ... + c16 of the 4 keys; steps add 16 rows, blocks 64 bytes (the row-bit-2 swap
  // stays inside the unit's low bit)
  const int vcol = 256 * side + 16 * ((lane >> 4) & 1) + 4 * (c16 & 3);
  const int vb0 = tile_off<kPitch, 2>(half + 2 * (c16 >> 2), vcol);
  const int vb1 = tile_off<kPitch, 2>(8 + half + 2 * (c16 >> 2), vcol);
  // P V steps [U0, U1) of the 16 (step u: keys 16 (u / 8) .., output block u % 8); the
  // accumulators are rescaled by the part that starts at step 0
  auto pv_steps = [&](int b, int par, auto U0c, auto U1c) {
    constexpr int U0 = decltype(U0c)::value, U1 = decltype(U1c)::value;
    // the pair heads' factors for this tile (1 unless the running maximum moved)
    const float al = s_al[par][pr][lane & 31];
    if (U0 == 0 && __any(al != 1.f)) {
#pragma unroll
      for (int db = 0; db < 8; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) o[db][j] *= al;
    }
    const __bf16* pp = &s_p[par][pr][(lane & 31) * kPP + 8 * half];
    const bf16x8 pb0 = *reinterpret_cast<const bf16x8*>(pp);
    const bf16x8 pb1 = *reinterpret_cast<const bf16x8*>(pp + 16);
    const __bf16* vt = s_k[b];
    auto vf = [&](int u) {  // u = 8 st + db
      const int off = (u >> 3) * 16 * kPitch * 2 + 64 * (u & 7);
      const bf16x4 lo = read_tr(vt, vb0 + off);
      const bf16x4 hi = read_tr(vt, vb1 + off);
      return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    bf16x8 vfr[3];
#pragma unroll
    for (int u = U0; u < U0 + 2 && u < U1; ++u) vfr[u % 3] = vf(u);
#pragma unroll
    for (int u = U0; u < U1; ++u) {
      if (u + 2 < U1) vfr[(u + 2) % 3] = vf(u + 2);
      o[u & 7] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfr[u % 3], u < 8 ? pb0 : pb1,
                                                         o[u & 7], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  const std::integral_constant<int, 0> first;
  const std::integral_constant<int, kPre> pre;
  const std::integral_constant<int, 16> all;
  for (int kt = 0; kt < n_kt; ++kt) {
    const int buf = kt % 3;
    const int par = kt & 1;
    const int key2 = kt + 2 < n_kt ? load_key(kt + 2) : -1;
    if (side == 1 && kt > 0) pv_steps((kt - 1) % 3, par ^ 1, first, pre);
    const char* kb = reinterpret_cast<const char*>(s_k[buf]);
    // scores start from the slots' bias (masked slot: -inf)
    f32x4 s0 = *reinterpret_cast<const f32x4*>(&s_bias[buf][4 * quad]);
    f32x4 s1 = *reinterpret_cast<const f32x4*>(&s_bias[buf][16 + 4 * quad]);
    // the score loop runs at a raised wave priority: where both waves of a SIMD can
    // issue, the one feeding score MFMAs goes first (~1% faster than equal priority)
    __builtin_amdgcn_s_setprio(1);
    {
      auto kf = [&](int j) {
        return *reinterpret_cast<const bf16x8*>(kb + ((j & 1) ? ka1 : ka0) + 64 * (j >> 1));
      };
      bf16x8 fr[4];
#pragma unroll
      for (int j = 0; j < 3; ++j) fr[j] = kf(j);
#pragma unroll
      for (int j = 0; j < 2 * NKS; ++j) {
        if (j + 3 < 2 * NKS) fr[(j + 3) & 3] = kf(j + 3);
        if (j & 1)
          s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fr[j & 3], qf[j >> 1], s1, 0, 0, 0);
        else
          s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fr[j & 3], qf[j >> 1], s0, 0, 0, 0);
        if (j == 3 && kt + 1 < n_kt) issue(kt + 1);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    // softmax of the own heads: lane holds head c16, keys 4 quad + t (s0) and
    // 16 + 4 quad + t (s1)
    float x[8];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      x[t] = s0[t];
      x[4 + t] = s1[t];
    }
    float mx = x[0];
#pragma unroll
    for (int t = 1; t < 8; ++t) mx = fmaxf(mx, x[t]);
    mx = pair32_max(pair16_max(mx)) * c;
    float al = 1.f;
    if (mx > m + kLazy || (m == -INFINITY && mx > -INFINITY)) {
      al = (m == -INFINITY) ? 0.f : exp2f(m - mx);
      l *= al;
      m = mx;
    }
    const float mu = (m == -INFINITY) ? 0.f : m;
    float pv[8], rs = 0.f;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      pv[t] = __builtin_amdgcn_exp2f(fmaf(x[t], c, -mu));
      rs += pv[t];
    }
    l += pair32_sum(pair16_sum(rs));
    {
      // key 4 quad + t of a step sits at position 2 quad + t / 2 (t even) or
      // 8 + 2 quad + t / 2 (t odd)
      typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
      __bf16* prow = &s_p[par][pr][hcol * kPP + 2 * quad];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const float* q4 = pv + 4 * st;
        *reinterpret_cast<bf16x2*>(prow + 16 * st) = bf16x2{(__bf16)q4[0], (__bf16)q4[2]};
        *reinterpret_cast<bf16x2*>(prow + 16 * st + 8) = bf16x2{(__bf16)q4[1], (__bf16)q4[3]};
      }
      if (quad == 0) s_al[par][pr][hcol] = al;
    }
    if (side == 0 && kt > 0) pv_steps((kt - 1) % 3, par ^ 1, first, all);
    if (side == 1 && kt > 0) pv_steps((kt - 1) % 3, par ^ 1, pre, all);
    if (kt + 2 < n_kt) store_key(kt + 2, key2);
    __builtin_amdgcn_s_waitcnt(0);  // the next tile's direct loads have landed
    __syncthreads();
  }
  if (n_kt > 0) pv_steps((n_kt - 1) % 3, (n_kt - 1) & 1, first, all);
  if (quad == 0) s_l[pr][hcol] = l;
  if (a.lse && quad == 0)
    a.lse[(int64_t)i * a.q.h + head] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
  __syncthreads();  // the pair's row sums; every wave is done with the tiles
  const float lp = s_l[pr][lane & 31];
  const float inv = lp > 0.f ? 1.f / lp : 0.f;
  const int n = lane & 31;
  const int hout = g * G + 16 * (pr + 4 * (n >> 4)) + (n & 15);  // pair column n's head
  if constexpr (sizeof(TO) == 2) {
    // the pair's 32 heads x 128 columns at a time through the (now free) key tiles,
    // then out as whole 16-byte row pieces
    constexpr int kPart = 128;
    constexpr int kRowB = kPart * 2 + 16;
    static_assert(NW * 32 * kRowB <= (int)sizeof(s_k), "staging fits the key tiles");
    char* st = reinterpret_cast<char*>(&s_k[0][0]) + wave * 32 * kRowB;
#pragma unroll
    for (int pc = 0; pc < 2; ++pc) {
#pragma unroll
      for (int db = 4 * pc; db < 4 * pc + 4; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const bf16x4 x4 = {(__bf16)(o[db][4 * jj] * inv), (__bf16)(o[db][4 * jj + 1] * inv),
                             (__bf16)(o[db][4 * jj + 2] * inv), (__bf16)(o[db][4 * jj + 3] * inv)};
          *reinterpret_cast<bf16x4*>(st + n * kRowB + (32 * db + 8 * jj + 4 * half - kPart * pc) * 2) = x4;
        }
#pragma unroll
      for (int e0 = 0; e0 < 32 * (kPart / 8); e0 += kWave) {
        const int rr = (e0 + lane) / (kPart / 8), un = (e0 + lane) % (kPart / 8);
        const int hr = g * G + 16 * (pr + 4 * (rr >> 4)) + (rr & 15);
        *reinterpret_cast<uint4*>(reinterpret_cast<__bf16*>(a.out) + ((int64_t)i * a.q.h + hr) * DV +
                                  256 * side + kPart * pc + un * 8) =
            *reinterpret_cast<const uint4*>(st + rr * kRowB + un * 16);
      }
    }
  } else {
    float* out = reinterpret_cast<float*>(a.out) + ((int64_t)i * a.q.h + hout) * DV + 256 * side;
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        *reinterpret_cast<float4*>(out + 32 * db + 8 * jj + 4 * half) =
            make_float4(o[db][4 * jj] * inv, o[db][4 * jj + 1] * inv, o[db][4 * jj + 2] * inv,
                        o[db][4 * jj + 3] * inv);
  }
}

template <int DQK, int DV, bool ALIAS, typename TO>
hipError_t launch_shape(const AttnKernelArgs& a, hipStream_t stream) {
  const int G = a.q.h / a.k.h;
  const dim3 grid((unsigned)a.L.n_q * a.k.h);
  int slot;
  constexpr bool k16 = DQK == 576 && DV == 512 && ALIAS;
  trace_begin(stream, !k16 ? "k_tok_attn" : G == 128 ? "k_tok_attn16p" : "k_tok_attn16", &slot);
  if constexpr (k16) {
    if (G == 32)
      hipLaunchKernelGGL((k_tok_attn16<2, TO>), grid, dim3(128), 0, stream, a);
    else if (G == 64)
      hipLaunchKernelGGL((k_tok_attn16<4, TO>), grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((k_tok_attn16p<TO>), grid, dim3(512), 0, stream, a);
    trace_end(stream, slot);
    return hipGetLastError();
  }
  if (G == 32)
    hipLaunchKernelGGL((k_tok_attn<DQK, DV, ALIAS, 1, TO>), grid, dim3(64), 0, stream, a);
  else if (G == 64)
    hipLaunchKernelGGL((k_tok_attn<DQK, DV, ALIAS, 2, TO>), grid, dim3(128), 0, stream, a);
  else
    hipLaunchKernelGGL((k_tok_attn<DQK, DV, ALIAS, 4, TO>), grid, dim3(256), 0, stream, a);
  trace_end(stream, slot);
  return hipGetLastError();
}

template <int DQK, int DV, typename TO>
hipError_t launch_alias(const AttnKernelArgs& a, hipStream_t stream) {
  const bool alias = a.v.data == a.k.data && a.v.stride_n == a.k.stride_n &&
                     a.v.stride_h == a.k.stride_h;
  if (alias) return launch_shape<DQK, DV, true, TO>(a, stream);
  return launch_shape<DQK, DV, false, TO>(a, stream);
}

template <typename TO>
hipError_t launch_out(const AttnKernelArgs& a, hipStream_t stream) {
  const int dqk = a.q.d, dv = a.v.d;
  if (dqk == 576 && dv == 512) return launch_alias<576, 512, TO>(a, stream);
  if (dqk == 128 && dv == 128) return launch_alias<128, 128, TO>(a, stream);
  return launch_alias<64, 64, TO>(a, stream);
}

}  // namespace

bool attn_token_mfma_supported(const AttnKernelArgs& a) {
  const int G = a.q.h / a.k.h;
  const int dqk = a.q.d, dv = a.v.d;
  const bool shape = (dqk == 576 && dv == 512) || (dqk == 128 && dv == 128) ||
                     (dqk == 64 && dv == 64);
  return a.mode == CSA_SEL_TOKEN && a.dtype == CSA_BF16 && a.idx_heads == 1 && shape &&
         (G == 32 || G == 64 || G == 128) && a.scale_log2 > 0.f &&
         (int64_t)a.L.n_q * a.k.h < (int64_t)1 << 31;
}

hipError_t launch_attn_token_mfma(const AttnKernelArgs& a, hipStream_t stream) {
  if (a.L.n_q == 0) return hipSuccess;
  if (a.out_dtype == CSA_BF16) return launch_out<__bf16>(a, stream);
  return launch_out<float>(a, stream);
}

}  // namespace csa
