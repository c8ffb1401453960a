// Absorbed-MLA value up-projection after sparse attention.
//
// Megatron-LM PR #3674, "[1/2] Enable DSA CP, THD with absorbed MLA": the
// earlier PR description quoted on that page (with matrix absorption the value
// up-projection is applied after sparse attention) and the review summary's
// sequence diagram (an einsum with up_v_weight after the sparse attention,
// giving [sq, b, np, v_channels]).  Reading: for each query head h,
//
//   out[i, h, d] = sum_c o[i, h, c] * w[h, d, c],
//
// o the latent attention output, w[h] the head's up-projection stored as a
// linear layer's weight (row d = output channel d).
//
// k_mla_v_up: per head a plain [n_q x Dl] x [Dl x Dv] product, bound by HBM
// (the latent output is read once; the weights, Dv * Dl per head, stay in L2).
// Workgroup b takes head b % Hq and 128 consecutive rows: the workgroups on one
// XCD (b % 8) serve the heads of one residue class mod 8, whose weights fit its
// L2.  The rows' latent outputs and the head's weight rows are staged 64
// channels at a time into LDS by direct loads (eight lanes cover a row's 128
// bytes, so every load instruction reads whole cache lines), double-buffered,
// at a pitch of 9 16-byte units (an odd count: the fragment reads of 32 rows
// fall on distinct banks; the pad slot re-reads unit 0).  Wave w computes out^T
// for 32 rows with 32x32x16 bf16 MFMA: the A operand is the weight (rows =
// output channels, shared by the four waves), the B operand the rows' latent
// outputs, so a lane ends with 4 consecutive output channels of one row per
// accumulator group (8- or 16-byte stores).
#include "common.hpp"
#include "gather.hpp"

namespace csa {

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

constexpr int kUpWaves = 4;
constexpr int kUpRows = 32 * kUpWaves;  // rows of one workgroup
constexpr int kUpKC = 64;        // latent channels per staged slice
constexpr int kUpPitch = 9;      // 16-byte units per staged row (8 + 1 pad)
constexpr int kUpChunks = kUpRows * kUpPitch / 64;  // 1 KiB pieces of a slice
static_assert(kUpRows * kUpPitch % 64 == 0, "slices must be whole KiBs");

template <int NM, typename TO>
__global__ __launch_bounds__(kUpWaves * kWave) void k_mla_v_up(View o, View w, int n_q,
                                                               TO* __restrict__ out) {
  // weight rows (output channels) padded to a multiple of 64 so that a slice is
  // whole KiBs; pad rows repeat the last channel and are never used
  constexpr int kWRows = (NM * 32 + 63) / 64 * 64;
  constexpr int kWChunks = kWRows * kUpPitch / 64;
  __shared__ __attribute__((aligned(16))) char s_o[2][kUpRows * kUpPitch * 16];
  __shared__ __attribute__((aligned(16))) char s_w[2][kWRows * kUpPitch * 16];
  const int hq = o.h;
  const int dl = o.d;
  const int h = blockIdx.x % hq;
  const int rw = (blockIdx.x / hq) * kUpRows;  // first row of the workgroup
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x & (kWave - 1);
  const int half = lane >> 5;
  // staging: lane slot -> (row, unit) of the slice; rows past the shard repeat
  // its last row (computed, not stored)
  constexpr int kPer = (kUpChunks + kUpWaves - 1) / kUpWaves;
  uint32_t goff[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int slot = (wave + kUpWaves * j) * 64 + lane;
    const int r = min(slot / kUpPitch, n_q - 1 - rw);
    const int u = slot % kUpPitch;
    goff[j] = (uint32_t)(((int64_t)r * o.stride_n + (u < 8 ? u : 0) * 8) * 2);
  }
  constexpr int kWPer = (kWChunks + kUpWaves - 1) / kUpWaves;
  uint32_t woff[kWPer];
#pragma unroll
  for (int j = 0; j < kWPer; ++j) {
    const int slot = (wave + kUpWaves * j) * 64 + lane;
    const int r = min(slot / kUpPitch, NM * 32 - 1);
    const int u = slot % kUpPitch;
    woff[j] = (uint32_t)(((int64_t)r * w.stride_h + (u < 8 ? u : 0) * 8) * 2);
  }
  const char* obase = reinterpret_cast<const char*>(elem_ptr<__bf16>(o, rw, h));
  const char* wbase = reinterpret_cast<const char*>(elem_ptr<__bf16>(w, h, 0));
  auto issue = [&](int kc, int buf) {
    const char* ob = obase + kc * kUpKC * 2;
    const char* wb = wbase + kc * kUpKC * 2;
    const uint32_t l0 = lds_addr(&s_o[buf][0]);
    const uint32_t w0 = lds_addr(&s_w[buf][0]);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int c = wave + kUpWaves * j;
      if (c < kUpChunks) gather16(goff[j], ob, __builtin_amdgcn_readfirstlane(l0 + c * 1024));
    }
#pragma unroll
    for (int j = 0; j < kWPer; ++j) {
      const int c = wave + kUpWaves * j;
      if (c < kWChunks) gather16(woff[j], wb, __builtin_amdgcn_readfirstlane(w0 + c * 1024));
    }
  };
  const int arow = (lane & 31) * kUpPitch * 16 + half * 16;  // + 32 rows per M tile
  const int brow = (wave * 32 + (lane & 31)) * kUpPitch * 16 + half * 16;
  f32x16 acc[NM];
#pragma unroll
  for (int mt = 0; mt < NM; ++mt) acc[mt] = f32x16{};
  const int nk = dl / kUpKC;
  issue(0, 0);
  wait_gathers();
  __syncthreads();
  for (int kc = 0; kc < nk; ++kc) {
    const int buf = kc & 1;
    if (kc + 1 < nk) issue(kc + 1, buf ^ 1);
#pragma unroll
    for (int s = 0; s < kUpKC / 16; ++s) {
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(&s_o[buf][brow + s * 32]);
#pragma unroll
      for (int mt = 0; mt < NM; ++mt) {
        const bf16x8 a =
            *reinterpret_cast<const bf16x8*>(&s_w[buf][arow + mt * 32 * kUpPitch * 16 + s * 32]);
        acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[mt], 0, 0, 0);
      }
    }
    wait_gathers();
    __syncthreads();  // the next slice has landed; this buffer is free again
  }
  const int dv = NM * 32;
  if constexpr (sizeof(TO) == 2) {
    // bf16: the wave's 32 output rows go through its own part of the (now
    // free) slice buffer, then out as whole rows, 16 bytes a lane: stores of 8
    // bytes spread over a row made the L2 fetch the lines they partly wrote
    constexpr int kRowB = NM * 64 + 16;  // staged row pitch in bytes (padded)
    static_assert(kUpWaves * 32 * kRowB <= 2 * kUpRows * kUpPitch * 16, "staging fits");
    char* st = &s_o[0][0] + wave * 32 * kRowB;
#pragma unroll
    for (int mt = 0; mt < NM; ++mt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const bf16x4 x = {(__bf16)acc[mt][4 * jj], (__bf16)acc[mt][4 * jj + 1],
                          (__bf16)acc[mt][4 * jj + 2], (__bf16)acc[mt][4 * jj + 3]};
        *reinterpret_cast<bf16x4*>(st + (lane & 31) * kRowB + (mt * 32 + 8 * jj + 4 * half) * 2) = x;
      }
    constexpr int kUnits = NM * 4;  // 16-byte units per output row
#pragma unroll
    for (int i = 0; i < 32 * kUnits / kWave; ++i) {
      const int e = i * kWave + lane;
      const int r = e / kUnits, un = e % kUnits;
      const int row = rw + wave * 32 + r;
      if (row < n_q)
        *reinterpret_cast<uint4*>(out + ((int64_t)row * hq + h) * dv + un * 8) =
            *reinterpret_cast<const uint4*>(st + r * kRowB + un * 16);
    }
    return;
  }
  const int row = rw + wave * 32 + (lane & 31);
  if (row >= n_q) return;
  TO* op = out + ((int64_t)row * hq + h) * dv + 4 * half;
  // lane holds output channels mt * 32 + 8 jj + 4 half + (0..3) of its row
#pragma unroll
  for (int mt = 0; mt < NM; ++mt)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      TO* p = op + mt * 32 + 8 * jj;
      if constexpr (sizeof(TO) == 4) {
        *reinterpret_cast<float4*>(p) = make_float4(acc[mt][4 * jj], acc[mt][4 * jj + 1],
                                                    acc[mt][4 * jj + 2], acc[mt][4 * jj + 3]);
      } else {
        const bf16x4 x = {(__bf16)acc[mt][4 * jj], (__bf16)acc[mt][4 * jj + 1],
                          (__bf16)acc[mt][4 * jj + 2], (__bf16)acc[mt][4 * jj + 3]};
        *reinterpret_cast<bf16x4*>(p) = x;
      }
    }
}

template <int NM>
hipError_t launch_nm(const MlaUpArgs& a, hipStream_t stream) {
  const int tiles = (a.n_q + kUpRows - 1) / kUpRows;
  const dim3 grid((unsigned)(tiles * a.o.h));
  if (a.out_dtype == CSA_BF16)
    hipLaunchKernelGGL((k_mla_v_up<NM, __bf16>), grid, dim3(kUpWaves * kWave), 0, stream, a.o,
                       a.w, a.n_q, static_cast<__bf16*>(a.out));
  else
    hipLaunchKernelGGL((k_mla_v_up<NM, float>), grid, dim3(kUpWaves * kWave), 0, stream, a.o,
                       a.w, a.n_q, static_cast<float*>(a.out));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mla_v_up_proj(const MlaUpArgs& a, hipStream_t stream) {
  if (a.n_q == 0) return hipSuccess;
  int slot;
  trace_begin(stream, "k_mla_v_up", &slot);
  hipError_t e;
  switch (a.w.h / 32) {
    case 1: e = launch_nm<1>(a, stream); break;
    case 2: e = launch_nm<2>(a, stream); break;
    case 3: e = launch_nm<3>(a, stream); break;
    default: e = launch_nm<4>(a, stream); break;
  }
  trace_end(stream, slot);
  return e;
}

}  // namespace csa
