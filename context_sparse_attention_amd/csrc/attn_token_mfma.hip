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
#include "attention.hpp"
#include "gather.hpp"
#include "mfma.hpp"

namespace csa {

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
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
template <int PITCH>
__device__ __forceinline__ int tile_off(int r, int e) {
  const int unit = (e >> 3) ^ ((r >> 3) & 1);
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
template <int D>
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
    const int u = pu < D / 8 ? (pu ^ ((row >> 3) & 1)) : 0;
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

template <int DQK, int DV, bool ALIAS, typename TO>
hipError_t launch_shape(const AttnKernelArgs& a, hipStream_t stream) {
  const int G = a.q.h / a.k.h;
  const dim3 grid((unsigned)a.L.n_q * a.k.h);
  int slot;
  trace_begin(stream, "k_tok_attn", &slot);
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
