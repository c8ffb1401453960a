// Block-mode sparse shard attention on the matrix cores (bf16 MFMA, gfx950).
//
// MoBA issue #34 (opening question): every query attends only to its own
// top-k key blocks.  With independent per-query, per-head choices a
// query-tile-centric kernel would visit the union of its rows' blocks, so the
// selection is inverted instead: every fully permitted block slot of every
// (row, head) is appended to the list of its (key head, block); each list is
// cut into tiles of 128 gathered queries that share the block's keys, and each
// tile yields one (m, l, z) chunk summary per slot ("Context parallel
// attention: exchange keys and merge softmax globally", chunk summary).  The
// own block, partially masked by the causal diagonal at the row's global
// position (Megatron-LM issue #4878, shifted causal diagonal), is computed in
// the same persistent kernel over diagonal tiles of consecutive rows.  A merge
// kernel then combines the summaries of each (row, head) by rescaling to the
// larger maximum and finalizes the output (neutral summary and zero-output
// convention for rows with no permitted key: same article, masking paragraph).
//
// Kernels (in stream order):
//   k_block_table  (layout.hip) block table + zeroed list counters, only for
//                  more than kLocalSeqs sequences (otherwise k_bm_hist does it)
//   k_bm_hist      LDS histogram of full block slots per list for each range of
//                  (row, head) pairs, own-block multiplicity per (row, head)
//   k_bm_colscan   one wave per list: prefix of the histogram over the ranges
//   k_bm_scan      one workgroup: list offsets and the query-tile table
//                  (for small matrices the fill workgroups derive both themselves)
//   k_bm_fill      place slot ids into the lists (counting sort)
//   k_bm_attn      persistent, per-XCD work queues: list tiles, then diagonal
//                  tiles; S^T = K Q^T and O^T = V^T P^T on LDS-staged key/value
//                  tiles (32x32x16 bf16 MFMA), fp32 online softmax in registers,
//                  one summary per chunk (fp32 m, l; bf16 z / l)
//   k_bm_merge     per (row, head): merge the summaries in slot order, finalize
//
// Layout of the math: the MFMA computes S^T (keys x queries) so that a lane
// owns one query and its scores sit in that lane's registers; the softmax row
// reduction is then in-lane plus one cross-half exchange, and P^T is already
// in the B-operand layout of the O^T = V^T P^T product (the contraction index
// is permuted consistently on both operands).  V is stored transposed in LDS.
#include "attention.hpp"
#include "gather.hpp"

namespace csa {

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

constexpr int kTN = 64;                  // keys per LDS tile
constexpr int kQW = 32;                  // queries per wave
constexpr int kWaves = 4;
constexpr int kTM = kQW * kWaves;        // queries per workgroup tile
constexpr int kThreads = kWaves * kWave;
constexpr int kScanThreads = 1024;
constexpr int kHistThreads = 256;
constexpr int kHistPairs = 256;        // (row, head) pairs per bucketing workgroup (one a thread)
constexpr int kMaxHistWgs = 512;
constexpr int64_t kHistCells = 1 << 21;  // bound on workgroups x lists
constexpr int kMaxLists = 16384;      // LDS histogram bins (64 KiB)
constexpr int kXcds = 8;              // accelerator complex dies; workgroup b runs on b % 8
constexpr int kQueue0 = 8;            // totals[kQueue0 + x]: work-queue counter of XCD x
constexpr float kLn2 = 0.69314718055994531f;

struct BmWs {
  BlockTable bt;
  int32_t* counts;    // [n_lists]  slots per list
  int32_t* hist;      // [n_lists, n_hist]  per-range counts, then prefixes
  int32_t* list_off;  // [n_lists + 1]
  int4* tiles;        // [max_tiles]  (list, first entry in entries[], slots, 0)
  int32_t* totals;    // [16]  [0] list tiles, [kQueue0 + x] work-queue counter of XCD x
  int4* pinfo;        // [n_q * hq]  own-block multiplicity, full-block slot mask (lo, hi),
                      //             first own-block slot (-1 if none)
  int4* rowinfo;      // [n_q]  own block (-1 if the row has no key), position, own block's
                      //        first key, 0
  int32_t* entries;   // [n_q * hq * W]  flat slot ids
  float2* part_ml;    // [n_q * hq * W]  (m in log2 units, l)
  __bf16* part_o;     // [n_q * hq * W * D]  normalized partial output z / l
};

int64_t max_query_tiles(int64_t slots, int64_t n_lists) { return slots / kTM + n_lists + 1; }

// Number of bucketing workgroups (ranges of (row, head) pairs), a multiple of
// 4 so that a list's row of the histogram matrix is read in 16-byte pieces.
int hist_wgs(int64_t pairs, int64_t n_lists) {
  int64_t w = (pairs + kHistPairs - 1) / kHistPairs;
  w = std::min<int64_t>(w, kMaxHistWgs);
  w = std::min<int64_t>(w, std::max<int64_t>(16, kHistCells / std::max<int64_t>(n_lists, 1)));
  return (int)((std::max<int64_t>(w, 1) + 3) / 4 * 4);
}

template <bool CARVE>
size_t carve_bm(void* base, int n_q, int n_seq, int n_blocks, int hq, int hkv, int dv, int W,
                BmWs* w) {
  Carver c(base);
  const int64_t n_lists = (int64_t)hkv * n_blocks;
  const int64_t slots = (int64_t)n_q * hq * W;
  BmWs t;
  t.bt.blk_off = c.take<int32_t>(n_seq + 1);
  t.bt.blocks = c.take<int2>(n_blocks);
  t.bt.blk_seq = c.take<int32_t>(n_blocks);
  t.counts = c.take<int32_t>(n_lists);
  t.hist = c.take<int32_t>((size_t)hist_wgs((int64_t)n_q * hq, n_lists) * n_lists);
  t.list_off = c.take<int32_t>(n_lists + 1);
  t.tiles = c.take<int4>(max_query_tiles(slots, n_lists));
  t.totals = c.take<int32_t>(16);
  t.pinfo = c.take<int4>((size_t)n_q * hq);
  t.rowinfo = c.take<int4>((size_t)n_q);
  t.entries = c.take<int32_t>(slots);
  t.part_ml = c.take<float2>(slots);
  t.part_o = c.take<__bf16>(slots * dv);
  if (CARVE) *w = t;
  return align_up(c.used, 256);
}

__device__ inline const int32_t* slot_row(const AttnKernelArgs& a, int i, int h) {
  return a.idx + ((int64_t)i * a.idx_heads + (a.idx_heads == 1 ? 0 : h)) * a.idx_width;
}

// Slot classes: 0 = no permitted key, 1 = full block strictly before pos_i, 2 = own block.
__device__ inline int slot_class(int s, const RowKeys& r, int B) {
  if (s < r.lo || s > r.hi || (s - r.lo) % B) return 0;
  return (s + B - 1 < r.hi) ? 1 : 2;
}

// The (row, head) pairs are cut into gridDim.x contiguous ranges.  Each range
// is bucketed by one workgroup with an LDS histogram (no global atomics), so
// list building is a counting sort: hist[list][w] counts, a scan turns the
// matrix into per-list offsets, and the fill pass places each slot at
// list_off[list] + prefix[list][w] + its LDS-local rank.
__device__ inline void pair_range(int64_t pairs, int64_t* b, int64_t* e) {
  const int64_t per = (pairs + gridDim.x - 1) / gridDim.x;
  *b = min(pairs, (int64_t)blockIdx.x * per);
  *e = min(pairs, *b + per);
}

// Sequences whose block offsets the bucketing workgroups build in LDS themselves
// (then no separate block-table kernel runs); more go through k_block_table.
constexpr int kLocalSeqs = 4096;

// First global block of every sequence, blk_off[0 .. n_seq], into s_off by the
// workgroup's kHistThreads threads (an exclusive scan of the block counts).
__device__ inline void local_blk_off(const int32_t* __restrict__ cu, int n_seq, int B,
                                     int* s_off) {
  __shared__ int s_wave[kHistThreads / kWave];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  int carry = 0;
  for (int base = 0; base < n_seq; base += kHistThreads) {
    const int s = base + threadIdx.x;
    const int nb = s < n_seq ? (cu[s + 1] - cu[s] + B - 1) / B : 0;
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
    for (int w = 0; w < kHistThreads / kWave; ++w) {
      before += w < wave ? s_wave[w] : 0;
      all += s_wave[w];
    }
    if (s < n_seq) s_off[s] = carry + before + incl - nb;
    carry += all;
    __syncthreads();
  }
  if (threadIdx.x == 0) s_off[n_seq] = carry;
  __syncthreads();
}

// LOCAL: the workgroup builds the sequences' block offsets in LDS, and
// workgroup 0 also writes the block table for the later kernels and clears the
// list-tile total and the work-queue counters (in place of k_block_table).
template <bool LOCAL>
__global__ __launch_bounds__(kHistThreads) void k_bm_hist(AttnKernelArgs a, BlockTable bt,
                                                          int n_blocks, int n_lists,
                                                          int32_t* __restrict__ hist,
                                                          int4* __restrict__ pinfo,
                                                          int4* __restrict__ rowinfo,
                                                          int32_t* __restrict__ totals) {
  extern __shared__ int s_bins[];
  const int* blk_off = bt.blk_off;
  if (LOCAL) {
    int* s_off = s_bins + n_lists;
    local_blk_off(a.L.cu, a.L.n_seq, a.block_size, s_off);
    blk_off = s_off;
    if (blockIdx.x == 0) {
      if (threadIdx.x < 16) totals[threadIdx.x] = 0;
      for (int s = threadIdx.x; s <= a.L.n_seq; s += kHistThreads) bt.blk_off[s] = s_off[s];
      for (int b = threadIdx.x; b < n_blocks; b += kHistThreads) {
        int lo = 0, hi = a.L.n_seq - 1;  // last sequence whose first block is <= b
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (s_off[mid] <= b) lo = mid; else hi = mid - 1;
        }
        const int start = a.L.cu[lo] + (b - s_off[lo]) * a.block_size;
        bt.blocks[b] = make_int2(start, min(a.block_size, a.L.cu[lo + 1] - start));
        bt.blk_seq[b] = lo;
      }
    }
  }
  for (int l = threadIdx.x; l < n_lists; l += kHistThreads) s_bins[l] = 0;
  __syncthreads();
  const int hq = a.q.h;
  int64_t b, e;
  pair_range((int64_t)a.L.n_q * hq, &b, &e);
  for (int64_t pair = b + threadIdx.x; pair < e; pair += kHistThreads) {
    const int i = (int)(pair / hq), h = (int)(pair % hq);
    const int g = h / (hq / a.k.h);
    const RowKeys r = row_keys(a.L, i);
    int mult = 0, own_slot = -1;
    uint64_t full = 0;
    if (r.valid) {
      const int32_t* slots = slot_row(a, i, h);
      const int base = g * n_blocks + blk_off[r.seq];
      for (int s = 0; s < a.idx_width; ++s) {
        const int st = slots[s];
        const int c = slot_class(st, r, a.block_size);
        if (c == 1) {
          atomicAdd(&s_bins[base + (st - r.lo) / a.block_size], 1);
          full |= (uint64_t)1 << s;
        } else if (c == 2) {
          if (mult++ == 0) own_slot = s;
        }
      }
    }
    pinfo[pair] = make_int4(mult, (int)(uint32_t)full, (int)(uint32_t)(full >> 32), own_slot);
    if (h == 0) {
      const int ob = r.valid ? blk_off[r.seq] + (r.hi - r.lo) / a.block_size : -1;
      const int ostart = r.valid ? r.lo + (r.hi - r.lo) / a.block_size * a.block_size : 0;
      rowinfo[i] = make_int4(ob, r.hi, ostart, 0);
    }
  }
  __syncthreads();
  for (int l = threadIdx.x; l < n_lists; l += kHistThreads)
    hist[(int64_t)l * gridDim.x + blockIdx.x] = s_bins[l];
}

// SCAN (small histogram matrices, in place of k_bm_colscan and k_bm_scan): the
// workgroup reads the whole matrix, one list a thread, and derives its own
// list offsets (exclusive scan of the list totals) and per-range prefixes;
// workgroup 0 also writes the list totals, offsets, the list-tile table and
// the tile count for the attention kernel.
template <bool LOCAL, bool SCAN>
__global__ __launch_bounds__(kHistThreads) void k_bm_fill(AttnKernelArgs a, BlockTable bt,
                                                          int n_blocks, int n_lists,
                                                          int32_t* __restrict__ list_off,
                                                          const int32_t* __restrict__ hist,
                                                          int32_t* __restrict__ entries,
                                                          int32_t* __restrict__ counts,
                                                          int4* __restrict__ tiles,
                                                          int32_t* __restrict__ totals) {
  extern __shared__ int s_bins[];
  const int* blk_off = bt.blk_off;
  if (LOCAL) {
    local_blk_off(a.L.cu, a.L.n_seq, a.block_size, s_bins + n_lists + (SCAN ? n_lists : 0));
    blk_off = s_bins + n_lists + (SCAN ? n_lists : 0);
  }
  if (SCAN) {
    __shared__ int s_wave[kHistThreads / kWave];
    __shared__ int s_carry[2];
    int* s_cnt = s_bins + n_lists;  // list totals, then the list offsets
    const int n_hist = gridDim.x;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int bx = blockIdx.x;
    for (int l = threadIdx.x; l < n_lists; l += kHistThreads) {
      // n_hist is a multiple of 4; sixteen 16-byte loads in flight
      const int4* h = reinterpret_cast<const int4*>(hist + (int64_t)l * n_hist);
      int tot = 0, pre = 0;
#pragma unroll 16
      for (int w4 = 0; w4 < n_hist / 4; ++w4) {
        const int4 v = h[w4];
        const int w = 4 * w4;
        tot += v.x + v.y + v.z + v.w;
        pre += (w < bx ? v.x : 0) + (w + 1 < bx ? v.y : 0) + (w + 2 < bx ? v.z : 0) +
               (w + 3 < bx ? v.w : 0);
      }
      s_cnt[l] = tot;
      s_bins[l] = pre;
    }
    __syncthreads();
    if (threadIdx.x == 0) s_carry[0] = s_carry[1] = 0;
    for (int base = 0; base < n_lists; base += kHistThreads) {
      const int l = base + threadIdx.x;
      const int c = l < n_lists ? s_cnt[l] : 0;
      const int nt = (c + kTM - 1) / kTM;
      int incl = c, tincl = nt;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const int y = __shfl_up(incl, off, kWave), ty = __shfl_up(tincl, off, kWave);
        if (lane >= off) {
          incl += y;
          tincl += ty;
        }
      }
      if (lane == kWave - 1) s_wave[wave] = incl;
      __syncthreads();
      int before = 0, all = 0;
#pragma unroll
      for (int w = 0; w < kHistThreads / kWave; ++w) {
        before += w < wave ? s_wave[w] : 0;
        all += s_wave[w];
      }
      __syncthreads();
      if (lane == kWave - 1) s_wave[wave] = tincl;
      __syncthreads();
      int tbefore = 0, tall = 0;
#pragma unroll
      for (int w = 0; w < kHistThreads / kWave; ++w) {
        tbefore += w < wave ? s_wave[w] : 0;
        tall += s_wave[w];
      }
      const int off = s_carry[0] + before + incl - c;
      const int first = s_carry[1] + tbefore + tincl - nt;
      if (l < n_lists) {
        s_bins[l] += off;
        if (blockIdx.x == 0) {
          counts[l] = c;
          list_off[l] = off;
          for (int j = 0; j < nt; ++j)
            tiles[first + j] = make_int4(l, off + j * kTM, min(kTM, c - j * kTM), 0);
        }
      }
      __syncthreads();
      if (threadIdx.x == 0) {
        s_carry[0] += all;
        s_carry[1] += tall;
      }
    }
    __syncthreads();
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      list_off[n_lists] = s_carry[0];
      totals[0] = s_carry[1];
    }
  } else {
    for (int l = threadIdx.x; l < n_lists; l += kHistThreads)
      s_bins[l] = list_off[l] + hist[(int64_t)l * gridDim.x + blockIdx.x];
  }
  __syncthreads();
  const int hq = a.q.h;
  int64_t b, e;
  pair_range((int64_t)a.L.n_q * hq, &b, &e);
  for (int64_t pair = b + threadIdx.x; pair < e; pair += kHistThreads) {
    const int i = (int)(pair / hq), h = (int)(pair % hq);
    const int g = h / (hq / a.k.h);
    const RowKeys r = row_keys(a.L, i);
    if (!r.valid) continue;
    const int32_t* slots = slot_row(a, i, h);
    const int base = g * n_blocks + blk_off[r.seq];
    for (int s = 0; s < a.idx_width; ++s) {
      const int st = slots[s];
      if (slot_class(st, r, a.block_size) != 1) continue;
      const int at = atomicAdd(&s_bins[base + (st - r.lo) / a.block_size], 1);
      entries[at] = (int32_t)(pair * a.idx_width + s);
    }
  }
}

// Workgroup-wide inclusive scan (kScanThreads threads).
__device__ int scan_incl(int x, int* s_wave, int* s_total) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(x, off, kWave);
    if (lane >= off) x += y;
  }
  if (lane == kWave - 1) s_wave[wave] = x;
  __syncthreads();
  int before = 0, all = 0;
  for (int w = 0; w < kScanThreads / kWave; ++w) {
    if (w < wave) before += s_wave[w];
    all += s_wave[w];
  }
  __syncthreads();
  *s_total = all;
  return x + before;
}

// One wave per list: exclusive prefix of the list's per-range counts, and the
// list total.
__global__ __launch_bounds__(kHistThreads) void k_bm_colscan(int n_lists, int n_hist,
                                                             int32_t* __restrict__ hist,
                                                             int32_t* __restrict__ counts) {
  const int lane = threadIdx.x & (kWave - 1);
  const int l = blockIdx.x * (kHistThreads / kWave) + threadIdx.x / kWave;
  if (l >= n_lists) return;
  int32_t* h = hist + (int64_t)l * n_hist;
  int carry = 0;
  for (int w0 = 0; w0 < n_hist; w0 += kWave) {
    const int w = w0 + lane;
    const int x = w < n_hist ? h[w] : 0;
    int incl = x;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int y = __shfl_up(incl, off, kWave);
      if (lane >= off) incl += y;
    }
    if (w < n_hist) h[w] = carry + incl - x;
    carry += __shfl(incl, kWave - 1, kWave);
  }
  if (lane == 0) counts[l] = carry;
}

// Histogram matrices of at most this many cells (and lists) are scanned by the
// fill workgroups themselves; larger ones by k_bm_colscan then k_bm_scan.
constexpr int64_t kFillScanCells = 1 << 15;
constexpr int kFillScanLists = 4096;

__global__ __launch_bounds__(kScanThreads) void k_bm_scan(int n_lists,
                                                          const int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ list_off,
                                                          int4* __restrict__ tiles,
                                                          int32_t* __restrict__ totals) {
  __shared__ int s_wave[kScanThreads / kWave];
  __shared__ int s_tfirst[kMaxLists + 1];  // first tile of each list
  __shared__ int s_loff[kMaxLists];        // first entry of each list
  int carry = 0, tcarry = 0, tot = 0;
  for (int base = 0; base < n_lists; base += kScanThreads) {
    const int l = base + threadIdx.x;
    const int c = l < n_lists ? counts[l] : 0;
    const int incl = scan_incl(c, s_wave, &tot);
    const int ctot = tot;
    const int nt = (c + kTM - 1) / kTM;
    const int tincl = scan_incl(nt, s_wave, &tot);
    if (l < n_lists) {
      list_off[l] = s_loff[l] = carry + incl - c;
      s_tfirst[l] = tcarry + tincl - nt;
    }
    carry += ctot;
    tcarry += tot;
  }
  if (threadIdx.x == 0) {
    list_off[n_lists] = carry;
    totals[0] = tcarry;
    s_tfirst[n_lists] = tcarry;
  }
  __syncthreads();
  // the tile table: each thread writes a run of consecutive tiles, finding the
  // list of its first tile by binary search over the lists' first tiles
  const int per = (tcarry + kScanThreads - 1) / kScanThreads;
  const int t0 = threadIdx.x * per, t1 = min(tcarry, t0 + per);
  if (t0 < t1) {
    int lo = 0, hi = n_lists - 1;  // last list whose first tile is <= t0
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_tfirst[mid] <= t0) lo = mid; else hi = mid - 1;
    }
    for (int t = t0; t < t1; ++t) {
      while (s_tfirst[lo + 1] <= t) ++lo;  // empty lists have no tiles
      const int j = t - s_tfirst[lo];
      const int cnt = (lo + 1 < n_lists ? s_loff[lo + 1] : carry) - s_loff[lo];
      tiles[t] = make_int4(lo, s_loff[lo] + j * kTM, min(kTM, cnt - j * kTM), 0);
    }
  }
}

// ---------------------------------------------------------------------------
// MFMA tile machinery
// ---------------------------------------------------------------------------

// LDS tiles are row-major with padded row pitches, filled straight from global
// memory by the gather instructions (no staging registers, no VALU work):
//   K [kTN][D + 8]: pitch 4 mod 32 banks, so eight consecutive rows read at one
//       column (the S^T operand reads) cover all 32 banks once;
//   V [kTN][D + 16]: pitch 8 mod 32 banks, so the four rows one transposing
//       read touches (ds_read_b64_tr_b16) cover all 32 banks once.
// Every fragment read is one per-lane base address plus a compile-time offset.
template <int D>
struct Lds {
  static constexpr int kKP = D + 8;
  static constexpr int kVR = D + 16;
  __bf16 k[2][kTN * kKP];
  __bf16 v[2][kTN * kVR];
};

// The gather of one key/value tile, split over the workgroup's waves in 1 KiB
// chunks: chunk c of a tile is issued by wave c % kWaves.  Lane l of chunk c
// fills 16-byte slot 64 c + l of the padded tile, i.e. unit (slot % units) of
// row (slot / units); pad slots re-read unit 0 of their row.  The per-lane
// byte offsets from the tile's first key do not change from tile to tile.
template <int D>
struct Gather {
  static constexpr int kKU = Lds<D>::kKP / 8;   // 16-byte slots per K row
  static constexpr int kVU = Lds<D>::kVR / 8;   // 16-byte slots per V row
  static constexpr int kKC = kTN * kKU / 64;    // 1 KiB chunks per K tile
  static constexpr int kVC = kTN * kVU / 64;
  static constexpr int kKPer = (kKC + kWaves - 1) / kWaves;
  static constexpr int kVPer = (kVC + kWaves - 1) / kWaves;
  static_assert(kTN * kKU % 64 == 0 && kTN * kVU % 64 == 0, "tiles must be whole KiBs");
  uint32_t ko[kKPer], vo[kVPer];

  // rows at or beyond `rows` repeat row rows - 1 (their scores are masked)
  __device__ __forceinline__ void init(const View& K, const View& V, int rows) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // uniform: scalar branches
#pragma unroll
    for (int j = 0; j < kKPer; ++j) {
      const int slot = (wave + kWaves * j) * 64 + lane;
      const int row = min(slot / kKU, rows - 1);
      const int u = slot % kKU;
      ko[j] = (uint32_t)((row * K.stride_n + (u < D / 8 ? u : 0) * 8) * (int64_t)sizeof(__bf16));
    }
#pragma unroll
    for (int j = 0; j < kVPer; ++j) {
      const int slot = (wave + kWaves * j) * 64 + lane;
      const int row = min(slot / kVU, rows - 1);
      const int u = slot % kVU;
      vo[j] = (uint32_t)((row * V.stride_n + (u < D / 8 ? u : 0) * 8) * (int64_t)sizeof(__bf16));
    }
  }

  __device__ __forceinline__ void issue(const char* kb, const char* vb, Lds<D>& s, int buf) const {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // uniform: scalar branches
    const uint32_t kl = lds_addr(&s.k[buf][0]), vl = lds_addr(&s.v[buf][0]);
#pragma unroll
    for (int j = 0; j < kKPer; ++j) {
      const int c = wave + kWaves * j;
      if (c < kKC) gather16(ko[j], kb, __builtin_amdgcn_readfirstlane(kl + c * 1024));
    }
#pragma unroll
    for (int j = 0; j < kVPer; ++j) {
      const int c = wave + kWaves * j;
      if (c < kVC) gather16(vo[j], vb, __builtin_amdgcn_readfirstlane(vl + c * 1024));
    }
  }
};

__device__ __forceinline__ bf16x4 read_tr(const __bf16* p) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s16x4* lds_ptr;
  const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_ptr)(const_cast<__bf16*>(p)));
  return __builtin_bit_cast(bf16x4, x);
}

// Per-wave online-softmax state for 32 queries (one per lane pair).  m is the
// reference maximum the exponentials are taken against (log2 units); it is
// raised only when a tile's maximum exceeds it by more than kLazy, so the
// probabilities stay below 2^kLazy and the accumulators are rescaled rarely.
template <int D>
struct WaveState {
  f32x16 o[D / 32];  // O^T: rows = value columns, columns = queries
  float m, l;        // reference max (log2 units) and denominator of this lane's query
};

constexpr float kLazy = 8.f;

// lane l and lane l ^ 32 hold the two key halves of one query
__device__ inline float halves_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                  false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float halves_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                  false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// One key tile for one wave: S^T = K Q^T, online softmax, O^T += V^T P^T.
// kvalid: number of valid keys in the tile; qpos: mask keys > qpos (MASK only).
// Fragment reads run three MFMAs ahead of their use, and the probabilities of
// key step ks + 1 are computed while the MFMAs of key step ks run.
template <int D, bool MASK>
__device__ __forceinline__ void wave_tile(const Lds<D>& s, int buf, const bf16x8* qf, float c,
                                          WaveState<D>& st, int tile_key0, int kvalid,
                                          int qpos) {
  constexpr int KP = Lds<D>::kKP, VR = Lds<D>::kVR;
  constexpr int NS = 2 * (D / 16);  // S^T MFMAs: MFMA i takes key block i & 1, step i >> 1
  constexpr int NDT = D / 32;       // value blocks
  constexpr int NO = 4 * NDT;       // O^T MFMAs: MFMA i takes value block i % NDT, step i / NDT
  const int lane = threadIdx.x & (kWave - 1);
  const int half = lane >> 5;
  const __bf16* kp = &s.k[buf][(lane & 31) * KP + 8 * half];
  // V^T fragment: in a 16-lane group, lane c addresses 4 values of key
  // kb + c / 4 at value column dvb + 4 (c % 4) and receives column dvb + c of
  // keys kb .. kb + 3; lanes 16..31 take the next 16 columns, lanes 32..63 the
  // keys 4 further on
  const int c16 = lane & 15;
  const __bf16* vp = &s.v[buf][(4 * half + (c16 >> 2)) * VR + 16 * ((lane >> 4) & 1) + 4 * (c16 & 3)];
  auto kfrag = [&](int i) {
    return *reinterpret_cast<const bf16x8*>(kp + (i & 1) * 32 * KP + (i >> 1) * 16);
  };
  auto vfrag = [&](int i) {  // value block i % NDT, keys 16 (i / NDT) + 4 half + (0..3, 8..11)
    const __bf16* p = vp + (i / NDT) * 16 * VR + (i % NDT) * 32;
    const bf16x4 lo = read_tr(p), hi = read_tr(p + 8 * VR);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };

  f32x16 sc[2] = {f32x16{}, f32x16{}};
  bf16x8 ka[4];
#pragma unroll
  for (int i = 0; i < 3; ++i) ka[i] = kfrag(i);
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    if (i + 3 < NS) ka[(i + 3) & 3] = kfrag(i + 3);
    sc[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[i & 3], qf[i >> 1], sc[i & 1], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
  // the first value fragments load while the softmax runs
  bf16x8 va[4];
#pragma unroll
  for (int i = 0; i < 3; ++i) va[i] = vfrag(i);

  // lane holds keys m*32 + 8*(j/4) + 4*half + (j%4) of its query (column lane&31)
  float mx = -INFINITY;
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (MASK) {
        const int kl = m * 32 + 8 * (j >> 2) + 4 * half + (j & 3);
        if (kl >= kvalid || tile_key0 + kl > qpos) sc[m][j] = -INFINITY;
      }
      mx = fmaxf(mx, sc[m][j]);
    }
  mx = halves_max(mx) * c;
  // wave-uniform branch: some query's maximum moved past the reference
  if (__builtin_amdgcn_ballot_w64(mx > st.m + kLazy)) {
    const float m_new = fmaxf(st.m, mx);
    // equal references (both -inf included) need no rescale
    const float alpha = (m_new == st.m) ? 1.f : __builtin_amdgcn_exp2f(st.m - m_new);
    st.l *= alpha;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int j = 0; j < 16; ++j) st.o[dt][j] *= alpha;
    st.m = m_new;
  }
  const float m_use = (st.m == -INFINITY) ? 0.f : st.m;

  // P^T for key step ks: pb[ks] holds keys 16ks + 4*half + (0..3) and
  // 16ks + 8 + 4*half + (0..3), i.e. elements (ks & 1) * 8 .. + 7 of sc[ks >> 1]
  bf16x8 pb[4];
  float rs = 0.f;
  auto probs = [&](int ks, int e0, int e1) {
#pragma unroll
    for (int e = e0; e < e1; ++e) {
      const float p =
          __builtin_amdgcn_exp2f(fmaf(sc[ks >> 1][(ks & 1) * 8 + e], c, -m_use));
      rs += p;
      pb[ks][e] = (__bf16)p;
    }
  };
  probs(0, 0, 8);
  constexpr int kSlice = 8 / NDT;
#pragma unroll
  for (int i = 0; i < NO; ++i) {
    if (i + 3 < NO) va[(i + 3) & 3] = vfrag(i + 3);
    const int dt = i % NDT, ks = i / NDT;
    st.o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[i & 3], pb[ks], st.o[dt], 0, 0, 0);
    if (ks + 1 < 4) probs(ks + 1, dt * kSlice, (dt + 1) * kSlice);
    __builtin_amdgcn_sched_barrier(0);
  }
  st.l += halves_sum(rs);
}

// Runs every key tile of [key0, key0 + nkeys) through the workgroup.  Tile kt
// is gathered into LDS buffer kt & 1 while tile kt - 1 is computed; each tile
// ends with a wait for this wave's gathers and a barrier, which makes the next
// tile visible and orders every read of a buffer before its next gather.
// Without MASK every tile is full (nkeys is a multiple of kTN).
// active: this wave has work; wave_max_pos: skip tiles entirely past it (MASK).
template <int D, bool MASK>
__device__ __forceinline__ void run_keys(Lds<D>& s, const View& K, const View& V, int g,
                                         int key0, int nkeys, bool active, const bf16x8* qf,
                                         float c, WaveState<D>& st, int qpos,
                                         int wave_max_pos) {
  key0 = __builtin_amdgcn_readfirstlane(key0);
  nkeys = __builtin_amdgcn_readfirstlane(nkeys);
  const int n_kt = (nkeys + kTN - 1) / kTN;
  Gather<D> gt;
  gt.init(K, V, MASK ? min(kTN, nkeys) : kTN);
  const char* kb = reinterpret_cast<const char*>(elem_ptr<__bf16>(K, key0, g));
  const char* vb = reinterpret_cast<const char*>(elem_ptr<__bf16>(V, key0, g));
  const int64_t kstep = kTN * K.stride_n * (int64_t)sizeof(__bf16);
  const int64_t vstep = kTN * V.stride_n * (int64_t)sizeof(__bf16);
  gt.issue(kb, vb, s, 0);
  wait_gathers();
  __syncthreads();
  for (int kt = 0; kt < n_kt; ++kt) {
    const int buf = kt & 1;
    const int tk0 = key0 + kt * kTN;
    if (kt + 1 < n_kt) {
      kb += kstep;
      vb += vstep;
      if (MASK && nkeys - (kt + 1) * kTN < kTN) gt.init(K, V, nkeys - (kt + 1) * kTN);
      gt.issue(kb, vb, s, buf ^ 1);
    }
    if (active && (!MASK || tk0 <= wave_max_pos))
      wave_tile<D, MASK>(s, buf, qf, c, st, tk0, min(kTN, nkeys - kt * kTN), qpos);
    wait_gathers();
    __syncthreads();
  }
}

template <int D>
__device__ __forceinline__ void load_q(const View& Q, int row, int head, bf16x8* qf) {
  const int half = (threadIdx.x & (kWave - 1)) >> 5;
  const __bf16* qp = elem_ptr<__bf16>(Q, row, head);
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
    qf[ks] = *reinterpret_cast<const bf16x8*>(qp + 16 * ks + 8 * half);
}

__device__ inline void store4(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}
__device__ inline void store4(__bf16* p, float a, float b, float c, float d) {
  bf16x4 x = {(__bf16)a, (__bf16)b, (__bf16)c, (__bf16)d};
  *reinterpret_cast<bf16x4*>(p) = x;
}

// Writes the chunk summaries of the wave's 32 (row, head) slots, for the lanes
// with `ok`: (m, l) and the normalized output z / l in bf16.  Every summary
// written has l >= 1: the key that set the reference maximum contributes 2^0.
// The output rows go through the wave's part of the key tiles (free here: every
// key loop ends with a barrier, and the next item's gathers start after
// another) and out as whole rows, 16 bytes a lane, where 8-byte stores spread
// over each row would leave the L2 with partly written lines.  Called by every
// lane of the wave.
template <int D>
__device__ __forceinline__ void write_summary(Lds<D>& s, const BmWs& w, int64_t p, bool ok,
                                              const WaveState<D>& st, int lane, int wave) {
  const int half = lane >> 5;
  if (ok && half == 0) w.part_ml[p] = make_float2(st.m, st.l);
  const float inv = ok ? 1.f / st.l : 0.f;
  constexpr int kRowB = 2 * D + 16;  // staged row pitch in bytes (padded)
  constexpr int kUnits = D / 8;      // 16-byte units of a row
  static_assert(kWaves * kQW * kRowB <= (int)sizeof(s.k), "staging fits in the key tiles");
  char* stg = reinterpret_cast<char*>(&s.k[0][0]) + wave * kQW * kRowB;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const bf16x4 x = {(__bf16)(st.o[dt][4 * jj] * inv), (__bf16)(st.o[dt][4 * jj + 1] * inv),
                        (__bf16)(st.o[dt][4 * jj + 2] * inv), (__bf16)(st.o[dt][4 * jj + 3] * inv)};
      *reinterpret_cast<bf16x4*>(stg + (lane & 31) * kRowB + (dt * 32 + 8 * jj + 4 * half) * 2) = x;
    }
#pragma unroll
  for (int e0 = 0; e0 < kQW * kUnits; e0 += kWave) {
    const int r = (e0 + lane) / kUnits, un = (e0 + lane) % kUnits;
    const int64_t pr = __shfl(p, r, kWave);
    const int okr = __shfl((int)ok, r, kWave);
    if (okr)
      *reinterpret_cast<uint4*>(w.part_o + pr * D + un * 8) =
          *reinterpret_cast<const uint4*>(stg + r * kRowB + un * 16);
  }
}

template <int D>
__device__ __forceinline__ void reset(WaveState<D>& st) {
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) st.o[dt] = f32x16{};
  st.m = -INFINITY;
  st.l = 0.f;
}

// List tile: up to kTM gathered (row, head) slots of one list against the
// list's full key block; one summary per slot.
template <int D>
__device__ __forceinline__ void list_item(Lds<D>& s, const AttnKernelArgs& a, const BmWs& w,
                                          int n_blocks, int t) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int half = lane >> 5;
  const int hq = a.q.h;
  const int W = a.idx_width;
  const int4 tl = w.tiles[t];
  const int list = tl.x;
  const int g = list / n_blocks;
  const int blk = list % n_blocks;
  const int cnt = tl.z;
  const int32_t* ent = w.entries + tl.y;
  const int n = wave * kQW + (lane & 31);
  const bool valid = n < cnt;
  const int p = ent[valid ? n : 0];
  const int row = p / (hq * W);
  const int head = (p / W) % hq;
  bf16x8 qf[D / 16];
  load_q<D>(a.q, row, head, qf);
  WaveState<D> st;
  reset(st);
  const int2 b = w.bt.blocks[blk];
  run_keys<D, false>(s, a.k, a.v, g, b.x, b.y, wave * kQW < cnt, qf, a.scale_log2, st, 0, 0);
  write_summary<D>(s, w, p, valid, st, lane, wave);
}

// Diagonal tile: TR = kTM / G consecutive rows x the G query heads of one key
// head against their own blocks, with the causal mask at each row's global
// position.  Rows of a tile whose own blocks differ (sequence or zigzag-chunk
// boundaries) are handled run by run: each lane only takes keys in the pass of
// its own row's block.  The summary goes to the (row, head)'s first own-block
// slot; rows that did not select their own block write nothing.
// Lowest set bit at or above `from` of the 128-bit mask (m1:m0), or n if none is below n.
__device__ inline int next_set(uint64_t m0, uint64_t m1, int from, int n) {
  if (from < 64) {
    const uint64_t x = m0 & (~0ull << from);
    if (x) return min(n, __builtin_ctzll(x));
    from = 64;
  }
  if (from < 128) {
    const uint64_t x = m1 & (~0ull << (from - 64));
    if (x) return min(n, 64 + __builtin_ctzll(x));
  }
  return n;
}

// Diagonal tile: TR = kTM / G consecutive rows x the G query heads of one key
// head against their own blocks, with the causal mask at each row's global
// position.  Rows of a tile whose own blocks differ (sequence or zigzag-chunk
// boundaries) are handled run by run: each lane only takes keys in the pass of
// its own row's block.  The summary goes to the (row, head)'s first own-block
// slot; rows that did not select their own block write nothing.  The runs are
// found in parallel (one bit per row starting a run); positions normally rise
// along a run, so its last row holds its largest position.
template <int D>
__device__ __forceinline__ void diag_item(Lds<D>& s, int* s_own, int* s_pos, int* s_ostart,
                                          uint64_t* s_mask, const AttnKernelArgs& a,
                                          const BmWs& w, int item) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int half = lane >> 5;
  const int hkv = a.k.h;
  const int hq = a.q.h;
  const int G = hq / hkv;
  const int TR = kTM / G;
  const int tile = item / hkv;
  const int g = item % hkv;
  const int r0 = tile * TR;
  const int nrows = min(TR, a.L.n_q - r0);
  const int n = wave * kQW + (lane & 31);
  const int rl = n % TR;
  const int head = g * G + n / TR;
  const bool valid = rl < nrows;
  const int rowc = r0 + (valid ? rl : 0);
  const int pair = rowc * hq + head;
  const int own_slot = w.pinfo[pair].w;  // the load overlaps the key loop
  bf16x8 qf[D / 16];
  load_q<D>(a.q, rowc, head, qf);
  if (threadIdx.x < kTM) {  // waves 0 and 1: one row each
    const int t = threadIdx.x;
    bool start = false, bad = false;
    if (t < nrows) {
      const int4 ri = w.rowinfo[r0 + t];
      const int4 rp = w.rowinfo[r0 + max(t - 1, 0)];
      start = t == 0 || rp.x != ri.x;
      bad = !start && rp.y >= ri.y;
      s_own[t] = ri.x;
      s_pos[t] = ri.y;
      s_ostart[t] = ri.z;
    }
    const uint64_t sm = __builtin_amdgcn_ballot_w64(start);
    const uint64_t bm = __builtin_amdgcn_ballot_w64(bad);
    if (lane == 0) {
      s_mask[wave] = sm;
      s_mask[2 + wave] = bm;
    }
  }
  __syncthreads();
  const int my_pos = valid ? s_pos[rl] : -1;
  const uint64_t m0 = s_mask[0], m1 = s_mask[1];
  const bool rising = (s_mask[2] | s_mask[3]) == 0;

  WaveState<D> st;
  reset(st);
  bool has_keys = false;
  for (int start = 0; start < nrows;) {
    const int end = next_set(m0, m1, start + 1, nrows);
    const int ob = s_own[start];
    if (ob >= 0) {
      int maxpos = s_pos[end - 1];
      if (!rising)
        for (int t = start; t < end; ++t) maxpos = max(maxpos, s_pos[t]);
      // a lane joins only the run that holds its row: two runs may share a
      // block when rows without keys sit between them
      const bool mine = valid && rl >= start && rl < end;
      has_keys |= mine;
      const int qpos = mine ? my_pos : -1;
      int wmax = qpos;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) wmax = max(wmax, __shfl_xor(wmax, off, kWave));
      const int own_start = s_ostart[start];
      run_keys<D, true>(s, a.k, a.v, g, own_start, maxpos - own_start + 1, wmax >= own_start,
                        qf, a.scale_log2, st, qpos, wmax);
    }
    start = end;
  }
  write_summary<D>(s, w, (int64_t)pair * a.idx_width + own_slot, has_keys && own_slot >= 0, st,
                   lane, wave);
}

// One persistent kernel for both kinds of chunk: workgroup b runs on XCD
// b % 8 and takes items from that XCD's queue, which holds a contiguous eighth
// of the list tiles (so the tiles of one key block share one L2) followed by
// an eighth of the diagonal tiles (smaller, uneven items that fill the tail).
// A queue's first items go one to each of its workgroups without an atomic
// (b / 8 is the workgroup's index among them); the counter hands out the rest.
// Device-scope atomics take microseconds here, and all workgroups asking at
// once made the first one the slowest.  The workgroup that takes a queue's
// last item knows that nothing is left and ends without asking again.
template <int D>
__global__ __launch_bounds__(kThreads, 2) void k_bm_attn(AttnKernelArgs a, BmWs w,
                                                         int n_blocks) {
  __shared__ Lds<D> s;
  __shared__ int s_own[kTM];
  __shared__ int s_pos[kTM];
  __shared__ int s_ostart[kTM];
  __shared__ uint64_t s_mask[4];
  __shared__ int s_item;
  const int n_lt = w.totals[0];
  const int G = a.q.h / a.k.h;
  const int n_dt = (a.L.n_q + kTM / G - 1) / (kTM / G) * a.k.h;
  const int x = blockIdx.x % kXcds;
  const int lper = (n_lt + kXcds - 1) / kXcds, dper = (n_dt + kXcds - 1) / kXcds;
  const int lb = min(n_lt, x * lper), ln = min(n_lt, lb + lper) - lb;
  const int db = min(n_dt, x * dper), dn = min(n_dt, db + dper) - db;
  const int nper = (gridDim.x - x + kXcds - 1) / kXcds;  // workgroups serving this queue
  int q = blockIdx.x / kXcds;
  while (q < ln + dn) {
    if (q < ln)
      list_item<D>(s, a, w, n_blocks, lb + q);
    else
      diag_item<D>(s, s_own, s_pos, s_ostart, s_mask, a, w, db + q - ln);
    if (q == ln + dn - 1) break;  // the counter hands out items in order: none is left
    // s_item and the diagonal tile's row tables are rewritten by the next item
    __syncthreads();
    if (threadIdx.x == 0) s_item = nper + atomicAdd(&w.totals[kQueue0 + x], 1);
    __syncthreads();
    q = s_item;
  }
}

__device__ inline float4 load4(const __bf16* p) {
  const bf16x4 x = *reinterpret_cast<const bf16x4*>(p);
  return make_float4((float)x[0], (float)x[1], (float)x[2], (float)x[3]);
}

// Merge of each (row, head)'s chunk summaries ("Context parallel attention:
// exchange keys and merge softmax globally", merge step): the own block
// counted with its multiplicity first, then the full-block slots in slot
// order, each by rescaling to the larger maximum; then the output z / l and
// the log-sum-exp.  A (row, head) with no summary gets the neutral summary:
// zero output, lse = -inf.  kLanes lanes per (row, head), 8 values each.
template <int D, typename TO>
__global__ __launch_bounds__(kHistThreads) void k_bm_merge(AttnKernelArgs a, BmWs w) {
  constexpr int kLanes = D / 8;
  const int64_t pair = (int64_t)blockIdx.x * (kHistThreads / kLanes) + threadIdx.x / kLanes;
  if (pair >= (int64_t)a.L.n_q * a.q.h) return;
  const int c8 = (threadIdx.x % kLanes) * 8;
  const int W = a.idx_width;
  const int4 info = w.pinfo[pair];
  float m = -INFINITY, l = 0.f, z[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) z[e] = 0.f;
  auto take = [&](int64_t p, float mult) {
    const float2 ml = w.part_ml[p];
    const uint4 raw = *reinterpret_cast<const uint4*>(w.part_o + p * D + c8);
    const float mn = fmaxf(m, ml.x);
    const float al = (m == -INFINITY) ? 0.f : exp2f(m - mn);
    const float be = exp2f(ml.x - mn) * ml.y * mult;
    l = l * al + be;
    m = mn;
    const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float o = __uint_as_float(e & 1 ? wd[e / 2] & 0xffff0000u : wd[e / 2] << 16);
      z[e] = z[e] * al + o * be;
    }
  };
  const int64_t pb = pair * W;
  if (info.x > 0 && info.w >= 0) take(pb + info.w, (float)info.x);
  uint64_t full = (uint64_t)(uint32_t)info.y | ((uint64_t)(uint32_t)info.z << 32);
  while (full) {
    take(pb + __builtin_ctzll(full), 1.f);
    full &= full - 1;
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  TO* out = reinterpret_cast<TO*>(a.out) + pair * D + c8;
  store4(out, z[0] * inv, z[1] * inv, z[2] * inv, z[3] * inv);
  store4(out + 4, z[4] * inv, z[5] * inv, z[6] * inv, z[7] * inv);
  if (a.lse && c8 == 0) a.lse[pair] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
}

template <int D>
hipError_t launch_d(const AttnKernelArgs& a, int n_blocks, void* ws, hipStream_t stream) {
  BmWs w;
  const int n_seq = a.L.n_seq;
  const int hq = a.q.h, hkv = a.k.h;
  carve_bm<true>(ws, a.L.n_q, n_seq, n_blocks, hq, hkv, D, a.idx_width, &w);
  const int n_lists = hkv * n_blocks;
  const int n_hist = hist_wgs((int64_t)a.L.n_q * hq, n_lists);
  // the LDS of a bucketing workgroup holds the list bins and, if local, the offsets
  const bool local = n_seq <= kLocalSeqs && (int64_t)(2 * n_lists + n_seq + 1) * 4 <= 65536;
  hipError_t e;
  if (!local) {
    // also zeroes the list-tile total and the work-queue counters
    e = launch_block_table(a.L.cu, n_seq, a.block_size, n_blocks, w.bt, w.totals, 16, stream);
    if (e != hipSuccess) return e;
  }
  const size_t bins = (size_t)(n_lists + (local ? n_seq + 1 : 0)) * sizeof(int);
  if (local)
    hipLaunchKernelGGL(k_bm_hist<true>, dim3(n_hist), dim3(kHistThreads), bins, stream, a, w.bt,
                       n_blocks, n_lists, w.hist, w.pinfo, w.rowinfo, w.totals);
  else
    hipLaunchKernelGGL(k_bm_hist<false>, dim3(n_hist), dim3(kHistThreads), bins, stream, a,
                       w.bt, n_blocks, n_lists, w.hist, w.pinfo, w.rowinfo, w.totals);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const bool fused = (int64_t)n_lists * n_hist <= kFillScanCells && n_lists <= kFillScanLists;
  if (!fused) {
    const int lists_per_wg = kHistThreads / kWave;
    hipLaunchKernelGGL(k_bm_colscan, dim3((n_lists + lists_per_wg - 1) / lists_per_wg),
                       dim3(kHistThreads), 0, stream, n_lists, n_hist, w.hist, w.counts);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(k_bm_scan, dim3(1), dim3(kScanThreads), 0, stream, n_lists, w.counts,
                       w.list_off, w.tiles, w.totals);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const size_t fbins = bins + (fused ? (size_t)n_lists * sizeof(int) : 0);
#define CSA_FILL(L_, S_)                                                                      \
  hipLaunchKernelGGL((k_bm_fill<L_, S_>), dim3(n_hist), dim3(kHistThreads), fbins, stream, a, \
                     w.bt, n_blocks, n_lists, w.list_off, w.hist, w.entries, w.counts, w.tiles, \
                     w.totals)
  if (local && fused) CSA_FILL(true, true);
  else if (local) CSA_FILL(true, false);
  else if (fused) CSA_FILL(false, true);
  else CSA_FILL(false, false);
#undef CSA_FILL
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int grid = 2 * device_cus();
  int slot;
  trace_begin(stream, "k_bm_attn", &slot);
  hipLaunchKernelGGL((k_bm_attn<D>), dim3(grid), dim3(kThreads), 0, stream, a, w, n_blocks);
  trace_end(stream, slot);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t pairs = (int64_t)a.L.n_q * hq;
  const int per_wg = kHistThreads / (D / 8);
  const dim3 mgrid((unsigned)((pairs + per_wg - 1) / per_wg));
  trace_begin(stream, "k_bm_merge", &slot);
  if (a.out_dtype == CSA_BF16)
    hipLaunchKernelGGL((k_bm_merge<D, __bf16>), mgrid, dim3(kHistThreads), 0, stream, a, w);
  else
    hipLaunchKernelGGL((k_bm_merge<D, float>), mgrid, dim3(kHistThreads), 0, stream, a, w);
  trace_end(stream, slot);
  return hipGetLastError();
}

}  // namespace

size_t attn_block_mfma_ws_bytes(int n_q, int n_seq, int n_blocks, int hq, int hkv, int dv,
                                int idx_width) {
  return carve_bm<false>(nullptr, n_q, n_seq, n_blocks, hq, hkv, dv, idx_width, nullptr);
}

bool attn_block_mfma_supported(const AttnKernelArgs& a, int n_blocks) {
  const int G = a.q.h / a.k.h;
  const int D = a.q.d;
  return a.mode == CSA_SEL_BLOCK && a.dtype == CSA_BF16 && (D == 64 || D == 128) &&
         a.idx_width <= 64 &&
         (int64_t)a.k.h * n_blocks <= kMaxLists &&
         a.v.d == D && a.block_size % kTN == 0 && G >= 1 && G <= kTM && (G & (G - 1)) == 0 &&
         a.scale_log2 > 0.f;
}

hipError_t launch_attn_block_mfma(const AttnKernelArgs& a, int n_blocks, void* ws,
                                  hipStream_t stream) {
  if (a.L.n_q == 0) return hipSuccess;
  if (a.q.d == 64) return launch_d<64>(a, n_blocks, ws, stream);
  return launch_d<128>(a, n_blocks, ws, stream);
}

}  // namespace csa
