// Internal launch interface between the C-ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

// Decode block scoring.
struct ScoreArgs {
  const void* idx_q;         // [B, Hidx, Di]
  const void* idx_k;         // [P, Hidx, 128, Di]
  int64_t num_pages;
  const int32_t* block_table;
  int32_t max_blocks;
  const int32_t* seq_lens;
  int32_t num_seqs;
  int32_t hidx;
  int32_t pages_per_item;    // blocks scored by one workgroup
  int32_t chunks_per_pair;   // ceil(max_blocks / pages_per_item)
  float* scores;             // [B, Hidx, max_blocks]
  int32_t fill_tail;         // write -inf past each row's last block
  // words zeroed by workgroup 0 (hand-off counters of a later kernel), or nullptr
  uint32_t* zero_words;
  int32_t zero_count;
  // short chunks (several queries per sequence): query rows of sequence b are
  // cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1; nullptr for decode
  const int32_t* cu_seqlens_q;
  // index-value branch (decode): index values [P, Hidx, 128, Di] and, per
  // (pair, chunk), the chunk's partial: Di sums of p v, then the base-2 max
  // m and the sum l of p = 2^(scaled logit - m); nullptr when off
  const void* idx_v;
  float* iv_part;            // [B * Hidx * chunks_per_pair, Di + 2]
  float iv_scale_log2;       // log2(e) / sqrt(Di)
  float st_scale_log2;       // log-sum-exp block scores: log2(e) / sqrt(Di)
};

// Prefill index scoring (causal GEMM with a block-max epilogue).
struct PrefillScoreArgs {
  const void* idx_q;         // [T, Hidx, Di] bf16
  const void* idx_k;         // [P, Hidx, 128, Di] bf16
  int64_t num_pages;
  const int32_t* block_table;
  int32_t max_blocks;
  const int32_t* seq_lens;
  const int32_t* cu_seqlens_q;
  int32_t num_seqs;
  int32_t hidx;
  int32_t max_tiles;         // 256-row query tiles of the longest possible sequence
  int32_t blocks_per_chunk;  // key blocks per workgroup (kPrefillBlocksPerChunk)
  int32_t kchunks;           // ceil(max_blocks / blocks_per_chunk)
  float* scores;             // [T, Hidx, max_blocks]
  float st_scale_log2;       // log-sum-exp block scores: log2(e) / sqrt(Di)
};

// Standalone selection over precomputed score rows.
struct SelectArgs {
  const float* scores;       // [T, Hidx, max_blocks]
  int32_t max_blocks;
  const int32_t* seq_lens;
  const int32_t* cu_seqlens_q;  // nullptr: decode
  int32_t num_seqs;
  int32_t num_tokens;
  int32_t hidx;
  int32_t topk, init, local, kmax;
  int32_t forced_in_budget;  // forced blocks count inside topk
  int32_t* sel;
  int32_t* cnt;
  // words the launch clears for the kernels after it (the prefill's k2q list
  // counts or split tickets), nullptr for none
  uint32_t* zero_words;
  int64_t zero_count;
};

// Decode split-K attention with a fused log-sum-exp combine.
struct AttendArgs {
  const void* q;             // [B, Hq, D]
  const void* k_pool;        // [P, Hkv, 128, D]
  const void* v_pool;
  int64_t num_pages;
  const int32_t* block_table;
  int32_t max_blocks;
  const int32_t* seq_lens;
  const int32_t* cu_seqlens_q;  // nullptr: decode (query t is sequence t)
  int32_t num_seqs;
  int32_t num_tokens;        // query tokens (decode: num_seqs)
  const int32_t* sel;        // [T, Hidx, kmax]
  const int32_t* cnt;        // [B, Hidx]
  // Selection inside the kernel (decode): when `scores` is set, every workgroup
  // selects its (sequence, index head) row itself and sel/cnt/sel_pages are
  // ignored; split 0 of the first kv head of each index head writes the
  // selection to sel_out/cnt_out when they are set.
  const float* scores;       // [B, Hidx, max_blocks] or nullptr
  int32_t topk, init, local;
  int32_t forced_in_budget;  // forced blocks count inside topk
  int32_t* sel_out;          // [B, Hidx, kmax] or nullptr
  int32_t* cnt_out;          // [B, Hidx] or nullptr
  int32_t kmax;
  int32_t hkv, hidx;
  int32_t bps;               // selected blocks per split
  int32_t nsplit_max;        // ceil(kmax / bps)
  float qk_scale_log2;       // softmax_scale * k_scale * log2(e)
  float v_scale;
  void* out;                 // [B, Hq, D] in the query dtype
  float* lse_out;            // [B, Hq] or nullptr
  float* part_o;             // [B, Hkv, nsplit_max, G, D]
  float* part_lse;           // [B, Hkv, nsplit_max, G]
  uint32_t* tickets;         // [B * Hkv], zero on entry
  // index-value branch (decode): the scan's per-chunk partials, merged by
  // split 0 of the first kv head of each index head into idx_out [B, Hidx, Di]
  const float* iv_part;      // [B * Hidx * iv_chunks, Di + 2] or nullptr
  void* idx_out;             // q dtype
  int32_t iv_chunks;         // chunks per (sequence, index head) of the scan
  int32_t iv_pages;          // pages per scan chunk
  int32_t idx_dim;
};

// Paged append of new tokens (k_new/v_new [T, Hkv, D], idx_k_new [T, Hidx, Di]).
struct AppendArgs {
  const void* k_new;
  const void* v_new;
  const void* idx_k_new;
  const int64_t* slots;      // [T] token slots; outside [0, num_pages * 128): skipped
  int32_t num_tokens;
  void* k_pool;              // [P, Hkv, 128, D]
  void* v_pool;
  void* idx_k_pool;          // [P, Hidx, 128, Di]
  const void* idx_v_new;     // [T, Hidx, Di] or nullptr (index-value branch off)
  void* idx_v_pool;          // [P, Hidx, 128, Di] or nullptr
  int64_t num_pages;
  int32_t hkv, hidx, head_dim, idx_dim;
  float k_scale, v_scale;    // fp8 pools only
};

// One prefill attention tile: up to kPrefillTileRows query rows of one k2q
// list against its key block, with page and bounds resolved by the kernel
// that fills the lists.
struct Tile {
  int32_t c0;      // first list entry of the tile
  int32_t ntok;    // tokens in the tile
  int32_t j;       // key block
  int32_t nvalid;  // keys of the block before the sequence end (0: no page)
  int32_t p0;      // position of token t is p0 + t
  int32_t g0;      // first kv head of the list's index head
  int64_t head0;   // element offset of (page, kv head g0) in the K/V pools
};

// Prefill index-value branch: causal softmax attention of every new token's
// index query over the index keys and values of its sequence, split over
// chunks of key blocks (the scoring grid), then merged per token.
struct PrefillValueArgs {
  const void* idx_q;         // [T, Hidx, Di] bf16
  const void* idx_k;         // [P, Hidx, 128, Di] bf16
  const void* idx_v;         // [P, Hidx, 128, Di] bf16
  int64_t num_pages;
  const int32_t* block_table;
  int32_t max_blocks;
  const int32_t* seq_lens;
  const int32_t* cu_seqlens_q;
  int32_t num_seqs;
  int32_t num_tokens;
  int32_t hidx;
  int32_t max_tiles;         // 256-row query tiles of the longest possible sequence
  int32_t blocks_per_chunk;  // key blocks per workgroup (kPrefillBlocksPerChunk)
  int32_t kchunks;           // ceil(max_blocks / blocks_per_chunk)
  float scale_log2;          // log2(e) / sqrt(Di)
  float* part_o;             // [T, Hidx, kchunks, Di] normalised partial outputs
  float* part_lse;           // [T, Hidx, kchunks] natural log
  void* idx_out;             // [T, Hidx, Di] in the query dtype (bf16 or f32)
  int32_t out_f32;           // 1: idx_out is float32
};

// Key-major prefill attention over the k2q lists (bf16 q; bf16 or fp8 K/V).
constexpr int kMaxSelect = 160;        // topk + init + local, at most
constexpr int kPrefillTileRows = 256;  // query rows (token x GQA head) per tile
// Blocks of keys per prefill scoring (and index-value) workgroup.
constexpr int kPrefillBlocksPerChunk = 16;
constexpr int kForcedRows = 128;       // query rows (token x GQA head) per forced-block group
struct PrefillAttnArgs {
  const void* q;             // [T, Hq, D] bf16
  const void* k_pool;        // [P, Hkv, 128, D]
  const void* v_pool;
  int64_t num_pages;
  const int32_t* block_table;
  int32_t max_blocks;
  const int32_t* seq_lens;
  const int32_t* cu_seqlens_q;
  int32_t num_seqs;
  int32_t num_tokens;
  const int32_t* sel;        // [T, Hidx, kmax]
  const int32_t* cnt;        // [T, Hidx]
  int32_t kmax;
  int32_t hkv, hidx;
  int32_t tq;                // tokens per tile: kPrefillTileRows / G
  // forced_split: the forced blocks (the first `init` and the last `local`
  // visible ones of every token) run in the query-major forced kernel, which
  // writes one partial per (token, kv head) into the token's first forced
  // slot; the lists leave them out and the combine reads only that slot of
  // them
  int32_t init, local;
  int32_t forced_split;
  int32_t* forced_off;       // [B + 1] forced-block token groups before each sequence
  int32_t tqf;               // tokens per forced-block group: kForcedRows / G
  // k2q lists, per (b, index head, block j): counts and cursor zero on entry
  int32_t* counts;           // [B * Hidx * max_blocks]
  int32_t* cursor;           // [B * Hidx * max_blocks]
  int32_t* tok_off;          // [B * Hidx * max_blocks] list offsets
  int32_t* tile_off;         // [B * Hidx * max_blocks] first work tile of each list
  int32_t* csr;              // [T * Hidx * kmax] entries token << 8 | slot
  struct Tile* items;        // [max_items] resolved work tiles
  int32_t* n_items;          // [1]
  int32_t max_items;         // upper bound of the tile count
  float qk_scale_log2;       // softmax_scale * k_scale * log2(e)
  float v_scale;
  uint16_t* part_o;          // [T, Hkv, kmax, G, D] normalised partial outputs, bf16
  float* part_lse;           // [T, Hkv, kmax, G]
  // write-only sink of the rows past a tile's last token (G * D bf16, then
  // G floats), so that every row stores unconditionally
  uint16_t* sink_o;
  float* sink_lse;
  void* out;                 // [T, Hq, D] bf16
  float* lse_out;            // [T, Hq] or nullptr
};

hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t value, hipStream_t s);
hipError_t launch_decode_score(const ScoreArgs& a, int idx_dtype, int idx_dim, int score_type,
                               hipStream_t s);
hipError_t launch_multi_score(const ScoreArgs& a, int idx_dim, int score_type, hipStream_t s);
hipError_t launch_select(const SelectArgs& a, hipStream_t s);
hipError_t launch_prefill_score(const PrefillScoreArgs& a, int idx_dim, int score_type,
                                hipStream_t s);
bool select_wave_fits(int max_blocks);
hipError_t launch_select_wave(const SelectArgs& a, hipStream_t s);
// Grid-stride clear of a.zero_words (every workgroup of a selection launch
// calls it first).
__device__ __forceinline__ void clear_words(const SelectArgs& a) {
  const int64_t n = a.zero_count;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    a.zero_words[i] = 0u;
}
hipError_t launch_fill_f32(float* p, int64_t n, float value, hipStream_t s);
hipError_t launch_decode_attend(const AttendArgs& a, int q_dtype, int kv_dtype,
                                int group, hipStream_t s);
hipError_t launch_prefill_k2q(const PrefillAttnArgs& a, hipStream_t s);
hipError_t launch_prefill_attend(const PrefillAttnArgs& a, int kv_dtype, int group,
                                 hipStream_t s);

hipError_t launch_append(const AppendArgs& a, int kv_dtype, int idx_dtype, hipStream_t s);
hipError_t launch_prefill_value(const PrefillValueArgs& a, int idx_dim, hipStream_t s);
hipError_t launch_fp8_dequant(const uint8_t* in, float* out, int64_t n, float scale, int dtype,
                              hipStream_t s);

}  // namespace msa
