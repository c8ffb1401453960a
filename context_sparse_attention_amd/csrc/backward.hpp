// Internal interface of the backward kernels (the gradients of the sparse shard
// attention with the selection held fixed).
#pragma once

#include "common.hpp"

namespace csa {

// Block-mode backward on the matrix cores, over the per-(key head, block) lists
// of flat slot ids that launch_attn_backward builds: bf16, D = Dqk = Dv in
// {64, 128}, one index row per query head.
struct BwEntryInfo {  // one list entry, as the dK/dV kernel reads it (32 bytes)
  int64_t qoff;        // element offset of the query row (i, h)
  int64_t goff;        // element offset of its bf16 dO row
  float lse2;          // lse * log2(e)
  float dl;            // D = dO . O
  int32_t pos;         // q_pos[i]
  int32_t pad;
};
struct BwMfmaArgs {
  View q, k, v, dout;
  int dout_dtype;
  View g16;                 // dO in bf16: dout itself, or a rounded copy
  BwEntryInfo* info;        // [entries + 128]
  DevLayout L;
  const int32_t* idx;
  int idx_width, block_size, n_blocks, n_lists, n_sub;
  BlockTable bt;
  const int32_t* list_off;  // [n_lists + 1]
  const int32_t* entries;   // flat slot ids, list by list, ascending
  const float* lse;
  const float* delta;       // dO . O per (row, head)
  float scale, scale_log2;
  float *dq, *dk, *dv;
  float* dq_part;           // [n_q * Hq * idx_width, D]: one dQ partial per slot
  int2* tiles;              // [max_tiles] (list, first entry) of 128-entry chunks
  int32_t* n_tiles;
  int64_t max_tiles;
  int64_t max_entries;      // n_q * Hq * idx_width (bounds the lists' total)
  __bf16* dout16;           // [n_q, Hq, D]: room for the rounded dO
};
int attn_bwd_block_mfma_subtiles(int block_size);
int64_t attn_bwd_block_mfma_max_tiles(int64_t n_entries, int64_t n_lists);
bool attn_bwd_block_mfma_supported(int mode, int dtype, int dqk, int dv, int hq, int idx_heads,
                                   int block_size, int64_t n_lists, int64_t n_entries);
hipError_t launch_attn_bwd_block_mfma(const BwMfmaArgs& a, hipStream_t stream);

// Token-mode backward on the matrix cores (one selection per token, bf16,
// Dqk = 576, Dv = 512, Hq / Hkv in {32, 64, 128}, index width at most 4096).
struct BwTokArgs {
  View q, k, v, dout;
  int dout_dtype;
  View g16;                 // dO in bf16: dout itself, or a rounded copy
  DevLayout L;
  const int32_t* idx;       // [n_q, idx_width]
  int idx_width;
  const float* lse;         // [n_q, Hq]
  const float* delta;       // [n_q, Hq]
  float scale, scale_log2;
  float *dq, *dk, *dv;
  __bf16* dout16;           // [n_q, Hq, 512]: room for the rounded dO
  __bf16 *ds, *pb;          // [n_q, Hq, wpad]: dS' and P per slot
  int wpad;                 // idx_width rounded up to 128
  __bf16 *ck, *cv;          // [n_q * idx_width, Hkv, 576 / 512]: per-slot contributions
  const int32_t* list_off;  // [n_kv + 1]: each key's slots (flat slot ids, ascending)
  const int32_t* entries;
};
bool attn_bwd_token_mfma_supported(int mode, int dtype, int dqk, int dv, int hq, int hkv,
                                   int idx_heads, int idx_width);
int attn_bwd_token_wpad(int idx_width);
// dK, dV and dQ
hipError_t launch_attn_bwd_token(const BwTokArgs& a, hipStream_t stream);

}  // namespace csa
