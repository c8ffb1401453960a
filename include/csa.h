/*
 * csa.h - C ABI of the context-parallel sparse-attention shard library (libcsa.so)
 * for AMD Instinct MI355X (gfx950).
 *
 * One call computes one step of the attention forward of one context-parallel
 * rank's shard: local queries at their global token positions attend to the
 * full gathered key/value stream, over key chunks picked per query either by
 * MoBA-style block gating or by a DSA-style token indexer, and per-chunk
 * softmax summaries (m, l, z) are merged by rescaling to the larger maximum.
 *
 * Sources (pages, by title and section):
 *  [MoBA#34]  MoBA issue #34 "Question on Implementing Context Parallelism with
 *             MoBA Efficient Attention", opening question: top-k key blocks per
 *             query from gating scores Q x K^T, local Q against gathered K.
 *  [CPA]      "Context parallel attention: exchange keys and merge softmax
 *             globally": global positions decide masks; packed sequences keep
 *             their boundaries; chunk summary (m, l, z) and its rescaled merge;
 *             neutral summary for all-masked chunks; explicit convention for a
 *             query with no permitted key; zigzag layouts keep global positions.
 *  [MLM#4878] Megatron-LM issue #4878 "[Feature-request] Context Parallel
 *             support for DSAttention", "Strategy: allgather CP mode": local Q
 *             against gathered K/V with the causal diagonal shifted by the
 *             rank's offset; top-k indices in global-sequence coordinates; a
 *             sparse kernel that iterates only over the top-k indices.
 *  [MLM#3674] Megatron-LM PR #3674 "[1/2] Enable DSA CP, THD with absorbed
 *             MLA", Description and sequence diagram: an indexer picks the
 *             top-k key tokens of each query; packed THD masking from sequence
 *             metadata; absorbed MLA (value = latent part of the key).
 *
 * Conventions shared by every entry point
 *  - Every pointer is DEVICE memory owned by the caller unless marked (host).
 *    The library allocates nothing, keeps no pointer after return, and never
 *    writes an input.  Work is enqueued on `stream` (a hipStream_t; NULL is the
 *    default stream) and the call returns without synchronising.
 *  - All argument checks run on the host before anything is enqueued.  A
 *    failed check returns a non-OK status, enqueues nothing and sets the text
 *    returned by csa_last_error() (per thread).  A failed HIP launch returns
 *    CSA_ERR_HIP.  No C++ exception crosses this interface.
 *  - Row i of the shard has global position q_pos[i] inside packed sequence
 *    q_seq[i] = [cu_seqlens[s], cu_seqlens[s+1]).  It may attend to the keys
 *    [lo_i, pos_i] with lo_i = cu_seqlens[q_seq[i]] [CPA, MLM#4878].  A row
 *    whose sequence id is out of range or whose position lies outside its
 *    sequence has no permitted key: it selects nothing, its output is 0 and
 *    its log-sum-exp is -inf [CPA].  Such rows are not an error.
 *  - Index values are int32 global key positions [MLM#4878], ascending within
 *    a row, padded with -1 at the end.  An index slot whose chunk has no
 *    permitted key of the row (including -1) is neutral; it is never read.
 *  - Query head h reads key/value head h / (Hq / Hkv) (grouped-query
 *    attention); Hq must be a multiple of Hkv.
 *  - Results are bitwise reproducible run to run (no floating-point atomics).
 *  - Tensors: element (t, h, e) lives at data + t*stride_n + h*stride_h + e
 *    (strides in elements).  The last dimension is contiguous, `data` is
 *    16-byte aligned and both strides are multiples of 16 bytes.
 */
#ifndef CSA_H
#define CSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CSA_OK = 0,
  CSA_ERR_INVALID_ARG = 1, /* a shape, dtype, stride, pointer or range check failed */
  CSA_ERR_UNSUPPORTED = 2, /* a valid request outside what the kernels implement   */
  CSA_ERR_WORKSPACE = 3,   /* workspace pointer missing, misaligned or too small  */
  CSA_ERR_HIP = 4          /* the HIP runtime rejected a launch                    */
} csa_status;

typedef enum { CSA_F32 = 0, CSA_BF16 = 1 } csa_dtype;

typedef enum {
  CSA_SEL_BLOCK = 0, /* index slots are block starts (MoBA) */
  CSA_SEL_TOKEN = 1  /* index slots are key tokens (DSA)    */
} csa_sel_mode;

/* A [n, h, d] tensor view.  `data` is device memory; the struct itself is host memory. */
typedef struct {
  const void* data;
  int32_t dtype; /* csa_dtype */
  int64_t n;
  int32_t h;
  int32_t d;
  int64_t stride_n; /* elements */
  int64_t stride_h; /* elements */
} csa_tensor3;

/* Shard layout.  The struct is host memory. */
typedef struct {
  int32_t n_q;                    /* local query rows                                  */
  int32_t n_kv;                   /* tokens in the gathered key/value stream           */
  const int32_t* q_pos;           /* [n_q] global position of each row (device)        */
  const int32_t* q_seq;           /* [n_q] packed-sequence id of each row (device)     */
  int32_t n_seq;                  /* packed sequences (1 for an unpacked stream)       */
  const int32_t* cu_seqlens;      /* [n_seq+1] sequence starts, last = n_kv (device)   */
  const int32_t* cu_seqlens_host; /* (host) the same values; used to size and check    */
} csa_layout;

/* ---------------------------------------------------------------------------------
 * moba_gate_topk - MoBA block gating and top-k block selection [MoBA#34].
 *
 * Blocks are cut per packed sequence from its first token, block_size tokens
 * each (the last block of a sequence may be shorter) [CPA: packed boundaries].
 * The score of block b for row i, query head h is q[i,h] . mean(k[t, kv(h)] for
 * t in b), in fp32 from an fp32 block mean.  Candidates of row i are the blocks
 * of its sequence that end at or before the start of the row's own block (the
 * block holding pos_i).  Each (row, head) keeps the min(topk, #candidates)
 * best candidates (score descending, ties to the lower block) and then its own
 * block.
 *
 *  q   [n_q, Hq, D]  bf16 or f32;  k [n_kv, Hkv, D] same dtype;  D <= 256.
 *  idx [n_q, Hq, topk+1] int32 out (contiguous): global start position of each
 *      selected block, ascending (so the own block is last), -1 padded.
 *  score [n_q, Hq, topk+1] f32 out, nullable: the gate score of each selected
 *      block; +inf for the own block, -inf for padding.
 *  topk in [0, 32].  ws: at least moba_gate_topk_workspace_size() bytes,
 *  256-byte aligned.
 * ------------------------------------------------------------------------------- */
size_t moba_gate_topk_workspace_size(const csa_layout* L, int32_t hkv, int32_t d,
                                     int32_t block_size);
csa_status moba_gate_topk(const csa_tensor3* q, const csa_tensor3* k, const csa_layout* L,
                          int32_t block_size, int32_t topk, int32_t* idx, float* score,
                          void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------
 * moba_gate_topk_noalloc - moba_gate_topk without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, serving loops
 * that forbid allocation, harnesses without an allocator).
 *
 * Same arguments, results and errors as moba_gate_topk, minus ws / ws_bytes.  The
 * scratch it needs lives in a fixed device array of CSA_GATE_SCRATCH_BYTES per GPU,
 * inside the library, held from the first call on that GPU until the process ends;
 * this call allocates nothing.  A request whose workspace would exceed that size
 * (moba_gate_topk_workspace_size() > CSA_GATE_SCRATCH_BYTES) returns
 * CSA_ERR_UNSUPPORTED and enqueues nothing.  All calls on one GPU share its scratch:
 * calls that may overlap on one GPU (different streams, or host threads) race and
 * must be ordered by the caller.  The first call on a GPU looks up that GPU's copy
 * (hipGetSymbolAddress) with the GPU current; a failure there returns CSA_ERR_HIP.
 * ------------------------------------------------------------------------------- */
#define CSA_GATE_SCRATCH_BYTES (16 * 1024 * 1024)
csa_status moba_gate_topk_noalloc(const csa_tensor3* q, const csa_tensor3* k,
                                  const csa_layout* L, int32_t block_size, int32_t topk,
                                  int32_t* idx, float* score, void* stream);

/* ---------------------------------------------------------------------------------
 * dsa_indexer_topk - DSA-style token indexer and top-k token selection
 * [MLM#3674 Description, MLM#4878 Strategy].
 *
 * Logit of key j for row i: L[i,j] = sum_h w[i,h] * max(0, iq[i,h] . ik[j]),
 * products and sums in fp32, over the permitted keys j in [lo_i, pos_i].
 * Each row keeps the min(topk, pos_i - lo_i + 1) largest logits, ties to the
 * lower key index.
 *
 *  iq [n_q, H_I, D_I] bf16 or f32;  ik [n_kv, 1, D_I] same dtype;  D_I <= 128,
 *     a multiple of 8.
 *  w  [n_q, H_I] f32 (row stride w_stride_n elements, H_I contiguous).
 *  idx [n_q, topk] int32 out (contiguous): selected global key positions,
 *     ascending, -1 padded.
 *  score [n_q, topk] f32 out, nullable: the logit of each selected key, -inf
 *     for padding.
 *  topk >= 1.  ws: at least dsa_indexer_topk_workspace_size() bytes (it holds
 *  the fp32 logits of the permitted keys), 256-byte aligned.
 * ------------------------------------------------------------------------------- */
size_t dsa_indexer_topk_workspace_size(const csa_layout* L, int32_t topk);
csa_status dsa_indexer_topk(const csa_tensor3* iq, const csa_tensor3* ik, const float* w,
                            int64_t w_stride_n, const csa_layout* L, int32_t topk,
                            int32_t* idx, float* score, void* ws, size_t ws_bytes,
                            void* stream);

/* ---------------------------------------------------------------------------------
 * sparse_attn_fwd_shard - attention of the shard's rows over their selected
 * key chunks [MLM#4878 "iterate only over topk indices", CPA summary merge].
 *
 * For row i, query head h, the selected keys are the multiset union over the
 * slots of idx row (i, h) (or (i, 0) when idx_heads == 1) of each slot's
 * permitted keys:
 *   CSA_SEL_TOKEN: slot j selects key j when lo_i <= j <= pos_i;
 *   CSA_SEL_BLOCK: slot s selects the block of the row's sequence starting at
 *     s when lo_i <= s <= pos_i and (s - lo_i) is a multiple of block_size;
 *     its keys are [s, min(s + block_size, sequence end)) cut to [lo_i, pos_i].
 * Slots are expected to be distinct; a repeated slot counts its keys again.
 * With logits x = softmax_scale * q . k, the output is
 *   out[i,h] = sum_j exp(x_j - M) v_j / sum_j exp(x_j - M),  lse = M + ln(sum),
 * computed as a merge of per-chunk (m, l, z) summaries in fp32 with bf16
 * products for bf16 inputs.  No selected key: out = 0, lse = -inf [CPA].
 *
 *  q [n_q, Hq, Dqk], k [n_kv, Hkv, Dqk], v [n_kv, Hkv, Dv]: same dtype.  v may
 *     alias k (absorbed MLA: v.data = k.data, v.d = 512 < k.d = 576).
 *     Dqk <= 576, Dv <= 512.
 *  idx [n_q, idx_heads, idx_width] int32 (contiguous); idx_heads is 1 or Hq.
 *  out [n_q, Hq, Dv] (contiguous) in out_dtype (CSA_F32 or CSA_BF16, rounded
 *     to nearest even); lse [n_q, Hq] f32, nullable (natural-log units).
 *  ws: at least sparse_attn_fwd_shard_workspace_size() bytes, 256-byte aligned.
 * ------------------------------------------------------------------------------- */
size_t sparse_attn_fwd_shard_workspace_size(const csa_layout* L, int32_t mode, int32_t hq,
                                            int32_t hkv, int32_t dv, int32_t idx_width,
                                            int32_t block_size);
csa_status sparse_attn_fwd_shard(const csa_tensor3* q, const csa_tensor3* k,
                                 const csa_tensor3* v, const csa_layout* L, int32_t mode,
                                 const int32_t* idx, int32_t idx_heads, int32_t idx_width,
                                 int32_t block_size, float softmax_scale, void* out,
                                 int32_t out_dtype, float* lse, void* ws, size_t ws_bytes,
                                 void* stream);

/* ---------------------------------------------------------------------------------
 * sparse_attn_fwd_shard_kernel - which kernel family sparse_attn_fwd_shard runs for
 * these arguments (the data pointers are not read; only shapes, dtypes and the
 * layout's host sequence starts are):
 *   "block_mfma"  block mode on the matrix cores: bf16, D = Dqk = Dv in {64, 128},
 *                 block_size a multiple of 64, a power-of-two group Hq/Hkv <= 128,
 *                 idx_width <= 64, at most 16384 (key head, block) lists;
 *   "token_mfma"  token mode on the matrix cores: bf16, one index row per token,
 *                 (Dqk, Dv) in {(576, 512), (128, 128), (64, 64)}, Hq/Hkv in
 *                 {32, 64, 128};
 *   "generic"     everything else: one wavefront per (row, head), fp32 arithmetic.
 * A positive softmax_scale is required by both MFMA families.  Returns a static
 * string, or NULL (with csa_last_error set) when the arguments would be rejected.
 * ------------------------------------------------------------------------------- */
const char* sparse_attn_fwd_shard_kernel(const csa_tensor3* q, const csa_tensor3* k,
                                         const csa_tensor3* v, const csa_layout* L,
                                         int32_t mode, int32_t idx_heads, int32_t idx_width,
                                         int32_t block_size, float softmax_scale,
                                         int32_t out_dtype);

/* ---------------------------------------------------------------------------------
 * sparse_attn_bwd_shard - gradients of sparse_attn_fwd_shard with the selection held
 * fixed [CPA, paragraph on positions and masks: the backward returns key and value
 * gradients to their owners; MLM#4878 "Strategy: allgather CP mode", backward step:
 * the gathered keys' and values' gradients are computed per rank, then
 * reduce-scattered (that reduction is the caller's)].
 *
 * With dO = dout, the forward's lse, P_j = exp(softmax_scale * q . k_j - lse) and
 * D = dO . out over each (row, head)'s selected keys (the same multiset as the
 * forward):
 *   dq[i,h]   = scale * sum_j P_j (dO . v_j - D) k_j
 *   dk[j,g]  += scale * P_j (dO . v_j - D) q[i,h]
 *   dv[j,g]  += P_j dO[i,h]
 * summed over every (row, head) whose selection holds key j, with g = h / (Hq/Hkv).
 * Each key's sums run over its selecting (row, head) pairs in ascending order and
 * each dq over its slots in order: bitwise reproducible, no floating-point atomics.
 * bf16 block mode with D = Dqk = Dv in {64, 128} and idx_heads = Hq runs on the
 * matrix cores ("block_mfma": P and dS rounded to bf16 as operands, as P is in
 * the forward; fp32 accumulation).  bf16 token mode with one selection per row
 * (idx_heads = 1), idx_width <= 4096, Dqk = 576, Dv = 512 (the absorbed-MLA
 * shape) and Hq / Hkv in {32, 64, 128} runs on the matrix cores too
 * ("token_mfma": P and dS as bf16 operands; each slot's dK and dV
 * contributions, summed over the group's heads in fp32, are stored in bf16 and
 * then summed per key in fp32).  Every other case runs fp32 arithmetic on the
 * vector ALUs ("generic").
 *
 *  q, k, v, idx, idx_heads, idx_width, block_size, softmax_scale, L, mode: as in
 *     sparse_attn_fwd_shard (the forward's arguments).  When v aliases k (absorbed
 *     MLA) dk and dv are still separate outputs; the gradient of the shared tensor
 *     is dk plus dv on its first Dv columns.
 *  out, dout [n_q, Hq, Dv] (f32 or bf16 each): the forward's output and the loss's
 *     gradient with respect to it.  lse [n_q, Hq] f32: the forward's log-sum-exp
 *     (natural log; -inf for a (row, head) without keys, which gets dq = 0).
 *  dq [n_q, Hq, Dqk], dk [n_kv, Hkv, Dqk], dv [n_kv, Hkv, Dv]: f32, contiguous,
 *     every element written (0 where nothing contributes).
 *  ws: at least sparse_attn_bwd_shard_workspace_size() bytes, 256-byte aligned (it
 *     holds D, the block table and the key lists: about 4 bytes per index slot; on
 *     the "block_mfma" path also one fp32 dq partial per slot, 4 * Dqk bytes; on the
 *     "token_mfma" path also dS and P per (row, head, slot), 4 bytes, and the
 *     per-slot contributions, 2 * Hkv * (Dqk + Dv) bytes per (row, slot): about
 *     22.5 GB for 4096 rows of 2048 slots, 128 heads, one latent head).
 *  n_q * Hq and n_q * idx_heads * idx_width must stay below 2^31.
 * ------------------------------------------------------------------------------- */
/* The workspace of a call with q [n_q, hq, dqk] and v [n_kv, hkv, dv] of dtype
 * `dtype` (CSA_F32 or CSA_BF16) and the other arguments as in the call; 0 when
 * they are malformed. */
size_t sparse_attn_bwd_shard_workspace_size(const csa_layout* L, int32_t mode, int32_t dtype,
                                            int32_t hq, int32_t hkv, int32_t dqk, int32_t dv,
                                            int32_t idx_heads, int32_t idx_width,
                                            int32_t block_size);
/* "block_mfma", "token_mfma" or "generic": the kernel family such a call runs; NULL (with
 * csa_last_error set) when the arguments are malformed. */
const char* sparse_attn_bwd_shard_kernel(const csa_layout* L, int32_t mode, int32_t dtype,
                                         int32_t hq, int32_t hkv, int32_t dqk, int32_t dv,
                                         int32_t idx_heads, int32_t idx_width,
                                         int32_t block_size);
csa_status sparse_attn_bwd_shard(const csa_tensor3* q, const csa_tensor3* k,
                                 const csa_tensor3* v, const csa_layout* L, int32_t mode,
                                 const int32_t* idx, int32_t idx_heads, int32_t idx_width,
                                 int32_t block_size, float softmax_scale,
                                 const csa_tensor3* out, const csa_tensor3* dout,
                                 const float* lse, float* dq, float* dk, float* dv, void* ws,
                                 size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------
 * summary_merge - merge P chunk summaries per row [CPA, summary paragraph].
 *
 * Part p of row r is (m[p,r], l[p,r], z[p,r,:]) with m in natural-log units.
 * Parts merge in ascending p: m = max(m_a, m_b); each side is scaled by
 * exp(m_side - m), a side with m = -inf by 0.  The neutral summary is
 * (-inf, 0, 0); merging two neutral summaries gives the neutral summary
 * without NaN [CPA, neutral-summary paragraph].
 *
 *  m, l [n_parts, n_rows] f32;  z [n_parts, n_rows, dv] f32 (all contiguous).
 *  m_out, l_out [n_rows], z_out [n_rows, dv]: merged summary, f32 (nullable
 *     together).
 *  o_out [n_rows, dv] in o_dtype and lse_out [n_rows] f32: finalized output
 *     o = z / l and lse = m + ln l; o = 0 and lse = -inf when l = 0 (nullable
 *     together).
 * ------------------------------------------------------------------------------- */
csa_status summary_merge(int32_t n_parts, int64_t n_rows, int32_t dv, const float* m,
                         const float* l, const float* z, float* m_out, float* l_out,
                         float* z_out, void* o_out, int32_t o_dtype, float* lse_out,
                         void* stream);

/* ---------------------------------------------------------------------------------
 * mla_v_up_proj - absorbed-MLA value up-projection after the sparse attention
 * [MLM#3674, the earlier PR description quoted on that page: with matrix
 * absorption the value up-projection is applied after sparse attention; the
 * review summary's sequence diagram: an einsum with up_v_weight after the
 * sparse attention gives [sq, b, np, v_channels]].
 *
 *   out[i, h, d] = sum_c o[i, h, c] * w[h, d, c]
 *
 *  o    [n_q, Hq, Dl] bf16: the latent attention output (sparse_attn_fwd_shard's
 *       out with the latent part of the key as the value).  Dl a multiple of 64,
 *       at most 8192; 128 rows span less than 4 GiB.
 *  w    bf16, head h's up-projection as a linear layer's weight: row d holds
 *       the Dl latent weights of output channel d.  Passed as a csa_tensor3
 *       with n = Hq, h = Dv, d = Dl.  Dv is 32, 64, 96 or 128.
 *  out  [n_q, Hq, Dv] in out_dtype (CSA_BF16 or CSA_F32), contiguous, 16-byte
 *       aligned, written.
 *  fp32 accumulation of exact bf16 products; deterministic.  No workspace.
 * ------------------------------------------------------------------------------- */
csa_status mla_v_up_proj(const csa_tensor3* o, const csa_tensor3* w, void* out,
                         int32_t out_dtype, void* stream);

/* ---------------------------------------------------------------------------------
 * Tracing (host-side, for profiling; not needed for computing).
 *
 * csa_trace_begin(n) allocates n HIP event pairs and turns tracing on
 * (n <= 0 turns it off and frees them).  While on, each call records one pair
 * on its stream around its dominant kernel until the n pairs are used.
 * csa_trace_collect waits for the recorded pairs, writes up to `max` elapsed
 * times (ms) and kernel names (static strings; either array nullable), returns
 * how many it wrote and rewinds the ring.  Returns CSA_ERR_HIP if event
 * creation fails.
 * ------------------------------------------------------------------------------- */
int csa_trace_begin(int max_records);
int csa_trace_collect(float* ms, const char** kernels, int max);

/* Text of the last non-OK status on the calling thread ("" if none). */
const char* csa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* CSA_H */
