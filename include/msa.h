/*
 * msa.h -- block-sparse attention over a paged KV cache, for AMD Instinct
 * MI355X (gfx950).  C ABI of libmsa.so.
 *
 * The method (sglang page minimax_sparse_backend.py, MiniMaxSparseAttnBackend:
 * per-token block selection with block_size_q = 1, block_size_k = 128, init,
 * local and top-k block counts; vLLM page sparse_attention_msa.py,
 * MiniMaxM3SparseMSAImpl.forward: causal attention over the selected 128-token
 * blocks of a paged cache, decode by split-K):
 *
 *   1. score  -- for query position p and index head h, block j < nb(p) =
 *                p/128 + 1 scores max over its tokens t <= p of
 *                q_idx[h] . k_idx[t, h]  (blocks >= nb(p) score -inf);
 *   2. select -- S = {init blocks 0..init-1} U {local blocks nb-local..nb-1}
 *                U top-k of the remaining blocks by (score desc, block asc),
 *                listed ascending, |S| = min(nb, |F| + topk) (or, with
 *                forced_in_budget, top-max(topk - |F|, 0) of the others);
 *   3. attend -- exact softmax attention of each q head over the tokens
 *                t <= p of the blocks in S of its index head, split along the
 *                selected-block axis and merged with a log-sum-exp combine.
 *
 * Layouts (all row-major, contiguous, caller-owned device memory):
 *   q          [T, Hq, D]           q_dtype
 *   idx_q      [T, Hidx, Di]        idx_dtype
 *   k_pool     [P, Hkv, 128, D]     kv_dtype  (per page, per head: 128 tokens)
 *   v_pool     [P, Hkv, 128, D]     kv_dtype
 *   idx_k_pool [P, Hidx, 128, Di]   idx_dtype
 *   block_table[B, max_blocks] int32: logical block j of sequence b lives in
 *              physical page block_table[b*max_blocks + j]; entries past a
 *              sequence's last block are ignored (-1 by convention)
 *   seq_lens   [B] int32: tokens of sequence b, including the query token(s)
 *   cu_seqlens_q [B+1] int32 (prefill only): query tokens of sequence b are
 *              rows cu[b]..cu[b+1]-1 and are the sequence's LAST tokens, at
 *              positions seq_lens[b] - n_b + i
 *   scores     [T, Hidx, max_blocks] float32
 *   idx_v_pool [P, Hidx, 128, Di]   idx_dtype (index-value branch only)
 *   sel_blocks [T, Hidx, Kmax] int32, Kmax = topk + init + local, ascending,
 *              -1 padded;  sel_count [T, Hidx] int32
 *   out        [T, Hq, D] q_dtype;  lse [T, Hq] float32 (natural log, of the
 *              scaled logits; -inf and out = 0 for a query with no tokens)
 *   idx_out    [T, Hidx, Di] q_dtype (index-value branch): per index head,
 *              softmax attention of the index query over the index keys and
 *              index values of every token t <= p, logits q_idx . k_idx /
 *              sqrt(Di); zeros for a query with no tokens.  The sglang page
 *              returns such an index output (idx_o, num_idx_heads *
 *              sparse_index_dim per token) beside the attention output; what
 *              its ops compute is not on the page, this is the reading taken.
 *
 * Head maps: q head hq reads kv head g = hq / (Hq/Hkv); kv head g uses index
 * head h = g / (Hkv/Hidx).
 *
 * Conventions:
 *  - The caller owns every buffer.  The library allocates nothing, frees
 *    nothing, copies nothing between host and device and never synchronises:
 *    every call only enqueues kernels on `stream` (a hipStream_t; NULL is the
 *    null stream), so calls can be captured into a HIP graph.  Host integers
 *    (num_seqs, max_blocks, num_q_tokens, num_pages) are shapes or upper
 *    bounds; per-step data (seq_lens, tables) is read on the device.
 *  - Arguments are validated before anything is enqueued; on any error the
 *    call returns a non-zero status and enqueues nothing.  Block-table
 *    entries outside [0, num_pages) are never dereferenced (such a block
 *    reads as empty); faults in the caller's memory surface at the caller's
 *    next synchronisation, as usual in HIP.
 *  - A sequence with seq_len 0 yields out = 0, lse = -inf, sel_count = 0.
 *  - Workspaces are plain device memory of msa_*_workspace_size() bytes,
 *    256-byte aligned; their contents on entry do not matter.  Calls that
 *    share a workspace must be ordered on one stream.
 *  - MSA_LOG=1 in the environment: every call prints the launch configuration
 *    it chose (grids, blocks per split, prefill path) on stderr.
 */
#ifndef MSA_H
#define MSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MSA_OK = 0,
  MSA_ERR_INVALID_ARG = 1, /* null pointer, bad shape or range            */
  MSA_ERR_UNSUPPORTED = 2, /* outside the supported parameter set         */
  MSA_ERR_WORKSPACE = 3,   /* workspace missing, too small or misaligned  */
  MSA_ERR_HIP = 4          /* a HIP launch failed; see msa_last_error()   */
} msa_status_t;

typedef enum {
  MSA_BF16 = 0,
  MSA_F32 = 1,
  MSA_FP8_E4M3 = 2, /* OCP e4m3 ("e4m3fn"): bias 7, no inf, S.1111.111 = NaN */
  MSA_FP8_E5M2 = 3, /* OCP e5m2: bias 15, S.11111.00 = inf, other S.11111.xx NaN
                       (the sglang page keeps fp8 main caches of either format
                       on its sparse path that dequantises on load) */
  MSA_MXFP4 = 4,    /* OCP MX-fp4 K/V pools: E2M1 codes (s.ee.m, bias 1: 0, 0.5,
                       1, 1.5, 2, 3, 4, 6) with an E8M0 scale 2^(e - 127) (0xFF
                       NaN) per 32 elements; per (page, head) the 128 x 64 code
                       bytes (element 2i of a row in the low nibble of byte i)
                       then the 128 x 4 scale bytes: pools [P, Hkv, 8704] bytes
                       at head_dim 128.  The gfx950 counterpart of the vLLM
                       page's 4-bit K/V caches with block scales in per-head
                       slots (MiniMaxM3SparseMSANvfp4Backend). */
  MSA_MXFP6 = 5     /* OCP MX-fp6 K/V pools: E2M3 codes (s.ee.mmm, bias 1:
                       k / 8 below 2, then steps of 1/4 and 1/2 up to 7.5)
                       with the same E8M0 scale per 32 elements; per (page,
                       head) the 128 x 96 code bytes (a 32-element group in 24
                       bytes, element i at bits 6i .. 6i + 5 of their
                       little-endian value) then the 128 x 4 scale bytes:
                       pools [P, Hkv, 12800] bytes at head_dim 128.  The other
                       block-scaled width gfx950 converts in hardware; a finer
                       grid than E2M1 at 25/32 byte per element. */
} msa_dtype_t;

/*
 * Model parameters (sglang page, MiniMaxSparseAttnBackend.__init__: sparse
 * index dim, block size, init / local / top-k block counts; vLLM page: k/v
 * scales of an fp8 cache).  Supported set:
 *   block_size == 128 (page size == block size), head_dim == 128,
 *   idx_dim in {64, 128}, topk in {4, 8, 16, 32}, 0 <= init, local <= 64,
 *   Hq % Hkv == 0 with Hq/Hkv in {1, 2, 4, 8, 16}, Hkv % Hidx == 0,
 *   (q_dtype, kv_dtype) in {(bf16, bf16), (bf16, fp8_e4m3), (bf16, fp8_e5m2),
 *   (bf16, mxfp4), (bf16, mxfp6), (f32, f32)},
 *   idx_dtype in {bf16, f32} (idx_q and idx_k share it).
 */
typedef struct {
  int32_t num_q_heads;   /* Hq   */
  int32_t num_kv_heads;  /* Hkv  */
  int32_t num_idx_heads; /* Hidx */
  int32_t head_dim;      /* D    */
  int32_t idx_dim;       /* Di   */
  int32_t block_size;    /* tokens per block == tokens per page           */
  int32_t topk;          /* top-k blocks chosen among non-forced blocks   */
  int32_t init_blocks;   /* leading blocks always kept (attention sink)   */
  int32_t local_blocks;  /* trailing blocks always kept, incl. own block  */
  float softmax_scale;   /* 0 => 1/sqrt(head_dim)                         */
  int32_t q_dtype;       /* msa_dtype_t */
  int32_t kv_dtype;      /* msa_dtype_t */
  int32_t idx_dtype;     /* msa_dtype_t */
  float k_scale;         /* fp8 and MX only: k = stored value * k_scale */
  float v_scale;         /* fp8 and MX only: v = stored value * v_scale */
  int32_t forced_in_budget; /* 0: S = F U top-k of the rest (|S| = min(nb,
                            |F| + topk)); 1: the forced blocks count inside
                            the budget, S = F U top-max(topk - |F|, 0) of the
                            rest (|S| = min(nb, max(topk, |F|))), the reading
                            under which the sglang page sizes its dense
                            fallback for topk_blocks * block_size_k tokens */
  int32_t index_value;   /* 1: the index-value branch is on: decode and
                            prefill also take the index-value pool and write
                            idx_out, the append stores index values; 0: off
                            (the sglang page's disable_index_value), those
                            pointers must be NULL */
  int32_t score_type;    /* block score of step 1 (the sglang page reads a
                            score type from the model config without printing
                            its values): 0 max (the default above), 1 the mean
                            of q_idx . k_idx over the block's tokens t <= p,
                            2 log sum exp(q_idx . k_idx / sqrt(Di)) over them;
                            1 and 2 are this library's definitions */
} msa_params_t;

/* Library version, (major << 16) | minor. */
int32_t msa_version(void);
const char* msa_status_string(msa_status_t status);
/* Detail of the last error returned on the calling thread ("" if none). */
const char* msa_last_error(void);

/*
 * Workspace sizes in bytes for msa_sparse_decode / msa_sparse_attend
 * (decode: num_q_tokens == num_seqs) and msa_sparse_prefill.  Returns 0 for
 * an invalid or unsupported parameter set (see msa_last_error()).
 */
size_t msa_decode_workspace_size(const msa_params_t* params, int32_t num_seqs,
                                 int32_t max_blocks);
size_t msa_prefill_workspace_size(const msa_params_t* params, int32_t num_seqs,
                                  int32_t num_q_tokens, int32_t max_blocks);

/*
 * Step 1 (score).  Defined by the sglang page minimax_sparse_backend.py:
 * MiniMaxSparseAttnBackend.__init__ reads the sparse index dim, block_size_k
 * (128) and the score type, and forward_decode hands the index query idx_q
 * and the index-key cache to minimax_sparse_decode, which scores every key
 * block for each query; the score of a block is the maximum over its tokens
 * up to the query of q_idx . k_idx (the page leaves the score type open; this
 * is the reading taken).
 * Writes scores[T, Hidx, max_blocks] (float32; -inf for
 * blocks past each query).  cu_seqlens_q == NULL: decode, T = num_seqs, one
 * query per sequence at position seq_len - 1.  Otherwise T = num_q_tokens
 * query tokens laid out by cu_seqlens_q.  Accumulation is float32.
 */
msa_status_t msa_block_score(const msa_params_t* params, const void* idx_q,
                             const void* idx_k_pool, int64_t num_pages,
                             const int32_t* block_table, int32_t max_blocks,
                             const int32_t* seq_lens,
                             const int32_t* cu_seqlens_q, int32_t num_seqs,
                             int32_t num_q_tokens, float* scores,
                             void* stream);

/*
 * Step 2 (select).  Defined by the sglang page minimax_sparse_backend.py,
 * MiniMaxSparseAttnBackend.__init__: one selection per query token
 * (block_size_q = 1) of the init, local and top-k key blocks, which
 * forward_decode / forward_extend pass to the sparse ops; the vLLM page
 * sparse_attention_msa.py (MiniMaxM3SparseMSAImpl.forward) consumes such a
 * selection as a token-major [total_q, H, MK] index buffer.
 * From scores[T, Hidx, max_blocks] writes
 * sel_blocks[T, Hidx, Kmax] and sel_count[T, Hidx].  Only the first nb(p)
 * scores of each row affect the result (the rest of the row may hold
 * anything).  Deterministic: equal scores (+0 and -0 are equal) go to the
 * lower block index.  With cu_seqlens_q given and num_seqs == 0 there is
 * nothing to select: returns MSA_OK and enqueues nothing.
 */
msa_status_t msa_select_blocks(const msa_params_t* params,
                               const float* scores, int32_t max_blocks,
                               const int32_t* seq_lens,
                               const int32_t* cu_seqlens_q, int32_t num_seqs,
                               int32_t num_q_tokens, int32_t* sel_blocks,
                               int32_t* sel_count, void* stream);

/*
 * Steps 1-3 for decode.  Defined by the sglang page minimax_sparse_backend.py,
 * forward_decode (the minimax_sparse_decode call: one query per sequence over
 * the paged cache, block table and seq_lens), attending as the vLLM page's
 * module docstring describes its decode: split-K over the selected blocks.
 * One query per sequence: score, select, split-K
 * attention over the selected blocks and log-sum-exp combine.  out [B, Hq, D]
 * in q_dtype.  lse_out, sel_blocks_out and sel_count_out may be NULL; when
 * given they receive the per-head lse and the selection.  With
 * params->index_value, the index scan also reads idx_v_pool and the
 * index-value output goes to idx_out [B, Hidx, Di] (one pass over the index
 * keys serves both); otherwise both must be NULL.  ws: a workspace of
 * msa_decode_workspace_size() bytes.
 */
msa_status_t msa_sparse_decode(const msa_params_t* params, const void* q,
                               const void* idx_q, const void* k_pool,
                               const void* v_pool, const void* idx_k_pool,
                               const void* idx_v_pool, int64_t num_pages,
                               const int32_t* block_table, int32_t max_blocks,
                               const int32_t* seq_lens, int32_t num_seqs,
                               void* out, void* idx_out, float* lse_out,
                               int32_t* sel_blocks_out,
                               int32_t* sel_count_out, void* ws,
                               size_t ws_bytes, void* stream);

/*
 * msa_sparse_decode without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, serving loops that
 * must not call the allocator, harnesses that forbid it.  Same arguments,
 * results and kernels as msa_sparse_decode; the workspace is a scratch area
 * the library keeps in each GPU's memory (16 MiB per GPU, held until the
 * process ends; its address is looked up once per device, on the first call
 * with that device current).  The stream must belong to the current device.
 * Calls whose decode workspace (msa_decode_workspace_size()) exceeds 16 MiB
 * return MSA_ERR_UNSUPPORTED and enqueue nothing.  No call allocates or frees
 * memory.  Every call on one GPU shares that GPU's scratch: calls that may
 * overlap on one GPU (different streams without ordering) race and must not
 * be issued; each call clears what it needs cleared inside its own kernels.
 */
msa_status_t msa_sparse_decode_noalloc(const msa_params_t* params, const void* q,
                                       const void* idx_q, const void* k_pool,
                                       const void* v_pool, const void* idx_k_pool,
                                       const void* idx_v_pool, int64_t num_pages,
                                       const int32_t* block_table, int32_t max_blocks,
                                       const int32_t* seq_lens, int32_t num_seqs,
                                       void* out, void* idx_out, float* lse_out,
                                       int32_t* sel_blocks_out, int32_t* sel_count_out,
                                       void* stream);

/*
 * Step 3 alone (decode).  Defined by the vLLM page sparse_attention_msa.py,
 * MiniMaxM3SparseMSAImpl.forward, decode part: split-K attention of the
 * decode queries over the blocks an indexer selected, through the block
 * table and seq_lens, with the fp8 k_scale / v_scale.
 * Attention over a given selection sel_blocks
 * [B, Hidx, Kmax] / sel_count [B, Hidx] (ascending block ids < nb).  Same
 * outputs and workspace as msa_sparse_decode.
 */
msa_status_t msa_sparse_attend(const msa_params_t* params, const void* q,
                               const void* k_pool, const void* v_pool,
                               int64_t num_pages, const int32_t* block_table,
                               int32_t max_blocks, const int32_t* seq_lens,
                               int32_t num_seqs, const int32_t* sel_blocks,
                               const int32_t* sel_count, void* out,
                               float* lse_out, void* ws, size_t ws_bytes,
                               void* stream);

/*
 * Steps 1-3 for chunked prefill.  Defined by the vLLM page
 * sparse_attention_msa.py, MiniMaxM3SparseMSAImpl.forward, prefill part
 * (per-block query lists from build_k2q_csr, then causal attention over the
 * selected 128-token blocks, causal=True, blk_kv = 128) and the sglang page's
 * forward_extend (cu_seqlens from the extend lengths, prefix lengths beside
 * seq_lens).
 * num_q_tokens new tokens laid out by
 * cu_seqlens_q [B+1], each attending causally to its sequence's tokens
 * t <= p through its own selection.  Outputs as for decode, per token.
 * Short chunks (num_q_tokens <= 8 * num_seqs, e.g. multi-token decode for
 * speculative verification) are scored by a page scan over several queries
 * per pass and attend per token with split-K; longer chunks take the causal
 * index GEMM and key-major tiles over per-block token lists.  The choice
 * follows from the shapes alone, like the workspace size.
 * Needs bf16 index keys and num_q_tokens < 2^23 (MSA_ERR_UNSUPPORTED
 * otherwise).  With params->index_value, idx_out [T, Hidx, Di] receives the
 * index-value branch (causal attention over the index keys and values, split
 * over runs of key blocks as the index scoring is, on the matrix cores);
 * otherwise idx_v_pool and idx_out must be NULL.
 * ws: msa_prefill_workspace_size() bytes.
 */
msa_status_t msa_sparse_prefill(const msa_params_t* params, const void* q,
                                const void* idx_q, const void* k_pool,
                                const void* v_pool, const void* idx_k_pool,
                                const void* idx_v_pool, int64_t num_pages,
                                const int32_t* block_table, int32_t max_blocks,
                                const int32_t* seq_lens,
                                const int32_t* cu_seqlens_q, int32_t num_seqs,
                                int32_t num_q_tokens, void* out, void* idx_out,
                                float* lse_out, int32_t* sel_blocks_out,
                                int32_t* sel_count_out, void* ws,
                                size_t ws_bytes, void* stream);

/*
 * Paged append, the step before the path: the sglang page's backend writes
 * the new tokens' K, V and index keys into its pool at out_cache_loc before
 * it attends (minimax_sparse_backend.py, forward_decode / forward_extend).
 * Token t's rows go to slot slot_mapping[t]: page s / 128, offset s % 128, of
 * every head.  Slots outside [0, num_pages * 128) (e.g. -1 padding) are
 * skipped; slots must be distinct (with a repeated slot, which token lands
 * there is unspecified).
 *   k_new, v_new [T, Hkv, D]: bf16 for bf16 and fp8 pools, f32 for f32 pools
 *                (q_dtype); idx_k_new [T, Hidx, Di] in idx_dtype.
 *   fp8 pools store e4m3fn(RNE(clamp(x / k_scale, +-448))) (v_scale for V;
 *   the division in float32); e5m2 pools the same with +-57344.  MX-fp4
 *   pools store y = x / k_scale (float32) per group of 32: the E8M0 scale
 *   2^(floor(log2 max|y|) - 2) clamped to the code range (an all-zero group
 *   takes code 0, a group with a NaN the NaN code and zero codes) and each
 *   element's E2M1 code nearest to y / 2^(code - 127), ties to the even code,
 *   clamped at 6 (the OCP Microscaling rule).  MX-fp6 pools the same with
 *   E2M3 codes, clamped at 7.5.
 *   With params->index_value, idx_v_new [T, Hidx, Di] (idx_dtype) goes to
 *   idx_v_pool beside the index keys (the page stores idx_v unless the layer
 *   disables the value branch); otherwise both must be NULL.
 * Nothing else is read or written.
 */
msa_status_t msa_append_kv(const msa_params_t* params, const void* k_new,
                           const void* v_new, const void* idx_k_new,
                           const void* idx_v_new, const int64_t* slot_mapping,
                           int32_t num_tokens, void* k_pool, void* v_pool,
                           void* idx_k_pool, void* idx_v_pool, int64_t num_pages,
                           void* stream);

/*
 * fp8-e4m3 dequantisation exactly as the attention loaders do it (sglang
 * page: the sparse path dequantises an fp8 main KV cache on load):
 * out[i] = value(in[i]) * scale for n codes.
 */
msa_status_t msa_fp8_e4m3_dequant(const uint8_t* in, float* out, int64_t n,
                                  float scale, void* stream);

/*
 * The same for either fp8 format of the K/V pools (dtype MSA_FP8_E4M3 or
 * MSA_FP8_E5M2; e5m2 infinities stay infinite, NaN codes give NaN):
 * out[i] = value(in[i]) * scale, through the loaders' bf16 conversion.
 * MSA_MXFP4: in holds n / 2 code bytes then n / 32 scale bytes (n a
 * multiple of 32, the order of one pool run) and out[i] = code value times
 * its group's scale, through the loaders' conversion, times scale.
 * MSA_MXFP6: the same with 3 n / 4 code bytes then n / 32 scale bytes.
 * MSA_ERR_UNSUPPORTED for any other dtype.
 */
msa_status_t msa_fp8_dequant(const uint8_t* in, float* out, int64_t n, float scale,
                             int32_t dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MSA_H */
