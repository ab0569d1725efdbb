// C ABI of libmsa: argument validation, workspace layout and kernel launches.
// Every entry point validates everything it can on the host before it
// enqueues anything; it never allocates, copies or synchronises.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "msa.h"
#include "msa_internal.h"

namespace {

using msa::kPrefillBlocksPerChunk;

thread_local char g_err[512] = "";

msa_status_t fail(msa_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

msa_status_t ok() {
  g_err[0] = '\0';
  return MSA_OK;
}

// MSA_LOG=1 in the environment: one line per entry-point call on stderr with
// the launch configuration it chose (the variable is read once).
bool log_on() {
  static const bool on = [] {
    const char* v = std::getenv("MSA_LOG");
    return v != nullptr && v[0] == '1';
  }();
  return on;
}

void log_line(const char* fmt, ...) {
  if (!log_on()) return;
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  std::fprintf(stderr, "[msa] %s\n", buf);
}

constexpr int kMaxBlocksLimit = 8192;  // 1M tokens per sequence
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int kmax_of(const msa_params_t& p) { return p.topk + p.init_blocks + p.local_blocks; }
int group_of(const msa_params_t& p) { return p.num_q_heads / p.num_kv_heads; }

bool is_fp8(int dtype) { return dtype == MSA_FP8_E4M3 || dtype == MSA_FP8_E5M2; }
// K/V formats whose per-tensor k_scale / v_scale apply (fp8 codes, MX-fp4,
// MX-fp6)
bool is_mx(int dtype) { return dtype == MSA_MXFP4 || dtype == MSA_MXFP6; }
bool scaled_kv(int dtype) { return is_fp8(dtype) || is_mx(dtype); }

msa_status_t check_params(const msa_params_t* p) {
  if (p == nullptr) return fail(MSA_ERR_INVALID_ARG, "params is NULL");
  if (p->num_q_heads <= 0 || p->num_kv_heads <= 0 || p->num_idx_heads <= 0)
    return fail(MSA_ERR_INVALID_ARG, "head counts must be positive (Hq=%d Hkv=%d Hidx=%d)",
                p->num_q_heads, p->num_kv_heads, p->num_idx_heads);
  if (p->num_q_heads % p->num_kv_heads != 0)
    return fail(MSA_ERR_INVALID_ARG, "Hq=%d is not a multiple of Hkv=%d", p->num_q_heads,
                p->num_kv_heads);
  const int G = p->num_q_heads / p->num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16)
    return fail(MSA_ERR_UNSUPPORTED, "Hq/Hkv=%d not in {1,2,4,8,16}", G);
  if (p->num_kv_heads % p->num_idx_heads != 0)
    return fail(MSA_ERR_UNSUPPORTED, "Hkv=%d is not a multiple of Hidx=%d", p->num_kv_heads,
                p->num_idx_heads);
  if (p->block_size != 128)
    return fail(MSA_ERR_UNSUPPORTED, "block_size=%d (only 128, equal to the page size)",
                p->block_size);
  if (p->head_dim != 128)
    return fail(MSA_ERR_UNSUPPORTED, "head_dim=%d (only 128)", p->head_dim);
  if (p->idx_dim != 64 && p->idx_dim != 128)
    return fail(MSA_ERR_UNSUPPORTED, "idx_dim=%d (only 64 or 128)", p->idx_dim);
  if (p->topk != 4 && p->topk != 8 && p->topk != 16 && p->topk != 32)
    return fail(MSA_ERR_UNSUPPORTED, "topk=%d not in {4,8,16,32}", p->topk);
  if (p->init_blocks < 0 || p->local_blocks < 0)
    return fail(MSA_ERR_INVALID_ARG, "negative init/local block count");
  if (p->forced_in_budget != 0 && p->forced_in_budget != 1)
    return fail(MSA_ERR_INVALID_ARG, "forced_in_budget=%d (0 or 1)", p->forced_in_budget);
  if (p->index_value != 0 && p->index_value != 1)
    return fail(MSA_ERR_INVALID_ARG, "index_value=%d (0 or 1)", p->index_value);
  if (p->score_type < 0 || p->score_type > 2)
    return fail(MSA_ERR_INVALID_ARG, "score_type=%d (0 max, 1 mean, 2 lse)", p->score_type);
  if (p->init_blocks > 64 || p->local_blocks > 64)
    return fail(MSA_ERR_UNSUPPORTED, "init/local block counts above 64");
  if (!std::isfinite(p->softmax_scale) || p->softmax_scale < 0.f)
    return fail(MSA_ERR_INVALID_ARG, "softmax_scale must be finite and >= 0");
  const bool qkv_ok = (p->q_dtype == MSA_BF16 && p->kv_dtype == MSA_BF16) ||
                      (p->q_dtype == MSA_BF16 && p->kv_dtype == MSA_FP8_E4M3) ||
                      (p->q_dtype == MSA_BF16 && p->kv_dtype == MSA_FP8_E5M2) ||
                      (p->q_dtype == MSA_BF16 && p->kv_dtype == MSA_MXFP4) ||
                      (p->q_dtype == MSA_BF16 && p->kv_dtype == MSA_MXFP6) ||
                      (p->q_dtype == MSA_F32 && p->kv_dtype == MSA_F32);
  if (!qkv_ok)
    return fail(MSA_ERR_UNSUPPORTED, "(q_dtype=%d, kv_dtype=%d) not supported", p->q_dtype,
                p->kv_dtype);
  if (p->idx_dtype != MSA_BF16 && p->idx_dtype != MSA_F32)
    return fail(MSA_ERR_UNSUPPORTED, "idx_dtype=%d not supported", p->idx_dtype);
  if (scaled_kv(p->kv_dtype) &&
      (!std::isfinite(p->k_scale) || !std::isfinite(p->v_scale) || p->k_scale <= 0.f ||
       p->v_scale <= 0.f))
    return fail(MSA_ERR_INVALID_ARG, "fp8 k_scale/v_scale must be finite and > 0");
  return MSA_OK;
}

msa_status_t check_shape(int32_t num_seqs, int32_t max_blocks) {
  if (num_seqs < 0) return fail(MSA_ERR_INVALID_ARG, "num_seqs=%d < 0", num_seqs);
  if (max_blocks < 1) return fail(MSA_ERR_INVALID_ARG, "max_blocks=%d < 1", max_blocks);
  if (max_blocks > kMaxBlocksLimit)
    return fail(MSA_ERR_UNSUPPORTED, "max_blocks=%d above %d", max_blocks, kMaxBlocksLimit);
  return MSA_OK;
}

float softmax_scale_of(const msa_params_t& p) {
  return p.softmax_scale > 0.f ? p.softmax_scale : 1.0f / std::sqrt(float(p.head_dim));
}

// Selected blocks handled by one split-K workgroup.  The attention kernel is
// bound by how many blocks the busiest CU streams, so the batch is cut into
// about one workgroup per CU (256 on MI355X, floor, so that no CU gets two
// while others idle): a unit (query, kv head) gets 256 / units splits.
constexpr int kAttendWgTarget = 256;
constexpr int kMaxBlocksPerSplit = 32;  // the attention kernel's limit
int blocks_per_split(const msa_params_t& p, int32_t num_units) {
  const int kmax = kmax_of(p);
  const int units = num_units * p.num_kv_heads > 0 ? num_units * p.num_kv_heads : 1;
  const int splits = kAttendWgTarget / units > 1 ? kAttendWgTarget / units : 1;
  const int bps = (kmax + splits - 1) / splits;
  return bps > kMaxBlocksPerSplit ? kMaxBlocksPerSplit : bps;
}

// Pages scored by one workgroup in the decode scan (two per wave): small
// items spread sequences of very different lengths evenly over the CUs
// (B = 64 with L from 4K to 128K: 361 -> 342 us for the scan), at no cost
// for equal lengths.
constexpr int kPagesPerItem = 8;
// Prefill list entries pack a token index above an 8-bit selection slot.
constexpr int kMaxPrefillTokens = 1 << 23;

// Decode workspace: block scores, split partials and the split tickets (and,
// with the index-value branch, the scan's per-chunk value partials).
struct DecodeLayout {
  size_t scores, part_o, part_lse, tickets, iv_part, total;
  int bps, nsplit_max;
};

DecodeLayout decode_layout(const msa_params_t& p, int32_t B, int32_t MB) {
  DecodeLayout l{};
  const int kmax = kmax_of(p);
  const int G = group_of(p);
  l.bps = blocks_per_split(p, B);
  l.nsplit_max = (kmax + l.bps - 1) / l.bps;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align_up(bytes);
    return at;
  };
  l.scores = take(sizeof(float) * size_t(B) * p.num_idx_heads * MB);
  l.part_o = take(sizeof(float) * size_t(B) * p.num_kv_heads * l.nsplit_max * G * p.head_dim);
  l.part_lse = take(sizeof(float) * size_t(B) * p.num_kv_heads * l.nsplit_max * G);
  l.tickets = take(sizeof(uint32_t) * size_t(B) * p.num_kv_heads);
  if (p.index_value)
    l.iv_part = take(sizeof(float) * size_t(B) * p.num_idx_heads *
                     ((MB + kPagesPerItem - 1) / kPagesPerItem) * (p.idx_dim + 2));
  l.total = off;
  return l;
}

// Prefill workspace: scores, selection, split partials and tickets per token.
// Key-major prefill attention (k2q lists) serves bf16 queries over bf16 or
// fp8 pools; f32 runs the per-token split-K attention.
// Short chunks (multi-token decode, e.g. speculative verification: at most
// kShortChunk new tokens per sequence on average) are scored by the page scan
// with several queries per pass and attend per token with split-K; the
// key-major lists and tiles pay off only for long chunks.  The choice depends
// on shapes only, so workspace sizes stay a function of them.
constexpr int kShortChunk = 8;
bool short_chunks(int32_t B, int32_t T) { return int64_t(T) <= int64_t(kShortChunk) * B; }

bool prefill_key_major(const msa_params_t& p, int32_t B, int32_t T) {
  return !short_chunks(B, T) && p.q_dtype == MSA_BF16 &&
         (p.kv_dtype == MSA_BF16 || scaled_kv(p.kv_dtype));
}

// log2(e) / sqrt(Di): the log-sum-exp block score accumulates in base 2.
float score_scale_log2(const msa_params_t& p) {
  return 1.4426950408889634f / std::sqrt(float(p.idx_dim));
}

// Index scan of the short-chunk path (all queries of a sequence per pass).
msa::ScoreArgs multi_score_args(const msa_params_t& p, const void* idx_q, const void* idx_k_pool,
                                int64_t num_pages, const int32_t* block_table,
                                int32_t max_blocks, const int32_t* seq_lens,
                                const int32_t* cu_seqlens_q, int32_t num_seqs, float* scores) {
  msa::ScoreArgs a{};
  a.idx_q = idx_q;
  a.idx_k = idx_k_pool;
  a.num_pages = num_pages;
  a.block_table = block_table;
  a.max_blocks = max_blocks;
  a.seq_lens = seq_lens;
  a.cu_seqlens_q = cu_seqlens_q;
  a.num_seqs = num_seqs;
  a.hidx = p.num_idx_heads;
  a.pages_per_item = kPagesPerItem;
  a.chunks_per_pair = (max_blocks + kPagesPerItem - 1) / kPagesPerItem;
  a.scores = scores;
  a.fill_tail = 0;
  a.st_scale_log2 = score_scale_log2(p);
  return a;
}

struct PrefillLayout {
  size_t scores, sel, cnt, part_o, part_lse, tickets;
  size_t iv_o, iv_lse;  // index-value branch: partials per (token, index head, key run)
  size_t counts, cursor, tok_off, tile_off, csr, items, n_items, sink;  // key-major only
  size_t forced_off;  // key-major: forced-block token groups before each sequence [B + 1]
  size_t total;
  int bps, nsplit_max;
  int tq, max_items;  // key-major only
};

PrefillLayout prefill_layout(const msa_params_t& p, int32_t B, int32_t T, int32_t MB) {
  PrefillLayout l{};
  const int kmax = kmax_of(p);
  const int G = group_of(p);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align_up(bytes);
    return at;
  };
  l.scores = take(sizeof(float) * size_t(T) * p.num_idx_heads * MB);
  l.sel = take(sizeof(int32_t) * size_t(T) * p.num_idx_heads * kmax);
  l.cnt = take(sizeof(int32_t) * size_t(T) * p.num_idx_heads);
  if (prefill_key_major(p, B, T)) {
    const size_t lists = size_t(B) * p.num_idx_heads * MB;
    const size_t entries = size_t(T) * p.num_idx_heads * kmax;
    l.tq = msa::kPrefillTileRows / G;
    l.max_items = int(entries / l.tq + std::min(lists, entries));
    l.counts = take(sizeof(int32_t) * 2 * lists);  // counts, then cursor
    l.cursor = l.counts + sizeof(int32_t) * lists;
    l.tok_off = take(sizeof(int32_t) * lists);
    l.tile_off = take(sizeof(int32_t) * lists);
    l.csr = take(sizeof(int32_t) * entries);
    l.items = take(sizeof(msa::Tile) * size_t(l.max_items));
    l.n_items = take(sizeof(int32_t));
    l.forced_off = take(sizeof(int32_t) * (size_t(B) + 1));
    const size_t parts = size_t(T) * p.num_kv_heads * kmax * G;
    l.part_o = take(sizeof(uint16_t) * parts * p.head_dim);  // bf16
    l.part_lse = take(sizeof(float) * parts);
    l.sink = take(sizeof(uint16_t) * G * p.head_dim + sizeof(float) * G);
  } else {
    l.bps = blocks_per_split(p, T);
    l.nsplit_max = (kmax + l.bps - 1) / l.bps;
    const size_t parts = l.nsplit_max > 1 ? size_t(T) * p.num_kv_heads * l.nsplit_max * G : 0;
    l.part_o = take(sizeof(float) * parts * p.head_dim);
    l.part_lse = take(sizeof(float) * parts);
    l.tickets = take(sizeof(uint32_t) * size_t(T) * p.num_kv_heads);
  }
  if (p.index_value) {
    const size_t runs = size_t(T) * p.num_idx_heads *
                        ((MB + kPrefillBlocksPerChunk - 1) / kPrefillBlocksPerChunk);
    l.iv_o = take(sizeof(float) * runs * p.idx_dim);
    l.iv_lse = take(sizeof(float) * runs);
  }
  l.total = off;
  return l;
}

msa::PrefillScoreArgs prefill_score_args(const msa_params_t& p, const void* idx_q,
                                         const void* idx_k_pool, int64_t num_pages,
                                         const int32_t* block_table, int32_t max_blocks,
                                         const int32_t* seq_lens, const int32_t* cu_seqlens_q,
                                         int32_t num_seqs, int32_t T, float* scores) {
  msa::PrefillScoreArgs a{};
  a.idx_q = idx_q;
  a.idx_k = idx_k_pool;
  a.num_pages = num_pages;
  a.block_table = block_table;
  a.max_blocks = max_blocks;
  a.seq_lens = seq_lens;
  a.cu_seqlens_q = cu_seqlens_q;
  a.num_seqs = num_seqs;
  a.hidx = p.num_idx_heads;
  a.max_tiles = (T + 255) / 256;
  a.blocks_per_chunk = kPrefillBlocksPerChunk;
  a.kchunks = (max_blocks + kPrefillBlocksPerChunk - 1) / kPrefillBlocksPerChunk;
  a.scores = scores;
  a.st_scale_log2 = score_scale_log2(p);
  return a;
}

msa::SelectArgs select_args(const msa_params_t& p, const float* scores, int32_t max_blocks,
                            const int32_t* seq_lens, const int32_t* cu_seqlens_q,
                            int32_t num_seqs, int32_t T, int32_t* sel, int32_t* cnt) {
  msa::SelectArgs a{};
  a.scores = scores;
  a.max_blocks = max_blocks;
  a.seq_lens = seq_lens;
  a.cu_seqlens_q = cu_seqlens_q;
  a.num_seqs = num_seqs;
  a.num_tokens = T;
  a.hidx = p.num_idx_heads;
  a.topk = p.topk;
  a.init = p.init_blocks;
  a.local = p.local_blocks;
  a.kmax = kmax_of(p);
  a.forced_in_budget = p.forced_in_budget;
  a.sel = sel;
  a.cnt = cnt;
  return a;
}

hipError_t launch_selection(const msa::SelectArgs& a, hipStream_t s) {
  return msa::select_wave_fits(a.max_blocks) ? msa::launch_select_wave(a, s)
                                             : msa::launch_select(a, s);
}

msa_status_t check_ws(const void* ws, size_t ws_bytes, size_t need) {
  if (ws == nullptr) return fail(MSA_ERR_WORKSPACE, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(ws) % kAlign != 0)
    return fail(MSA_ERR_WORKSPACE, "workspace not %zu-byte aligned", kAlign);
  if (ws_bytes < need)
    return fail(MSA_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, need);
  return MSA_OK;
}

// The index-value pointers go with params->index_value: all given when it is
// on, none when it is off.
msa_status_t check_iv(const msa_params_t& p, const void* a, const void* b, const char* names) {
  if (p.index_value && (a == nullptr || b == nullptr))
    return fail(MSA_ERR_INVALID_ARG, "index_value=1 needs %s", names);
  if (!p.index_value && (a != nullptr || b != nullptr))
    return fail(MSA_ERR_INVALID_ARG, "%s given with index_value=0", names);
  return MSA_OK;
}

msa_status_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return MSA_OK;
  return fail(MSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Launch-size limits, checked before a call enqueues anything: a dispatch
// holds each grid dimension as a 32-bit count of work-items, and the
// launchers count workgroups in int.
msa_status_t check_grid(int64_t workgroups, int threads, const char* what) {
  if (workgroups > 0x7fffffffLL || workgroups * threads > 0xffffffffLL)
    return fail(MSA_ERR_UNSUPPORTED,
                "%s: %lld workgroups of %d threads exceed a grid's 32-bit work-item count",
                what, (long long)workgroups, threads);
  return MSA_OK;
}

constexpr int kScanThreads = 256;     // decode and short-chunk scans, selection, combine
constexpr int kAttendThreads = 512;   // decode attention: eight waves
// Prefill scoring grid: (sequence, index head, 16-block run) triples rounded
// up to a multiple of 8, times the 256-row tiles of the longest possible
// sequence (launch_prefill_score).
int64_t prefill_score_workgroups(int32_t B, int hidx, int32_t MB, int32_t T) {
  const int64_t runs = int64_t(B) * hidx * ((MB + kPrefillBlocksPerChunk - 1) / kPrefillBlocksPerChunk);
  return (runs + 7) / 8 * 8 * ((int64_t(T) + 255) / 256);
}

int64_t scan_workgroups(int32_t B, int hidx, int32_t MB) {
  return int64_t(B) * hidx * ((MB + kPagesPerItem - 1) / kPagesPerItem);
}
// the attention grid holds every (token, kv head, split) unit, rounded up to
// one run per XCD
int64_t attend_workgroups(int nsplit, int hkv, int32_t T) {
  return (int64_t(nsplit) * hkv * T + 7) / 8 * 8;
}
int64_t select_workgroups(int32_t T, int hidx, int32_t MB) {
  const int64_t rows = int64_t(T) * hidx;
  return msa::select_wave_fits(MB) ? (rows + 3) / 4 : rows;
}

// Arguments of the split-K attention (decode).
msa::AttendArgs attend_args(const msa_params_t& p, const void* q, const void* k_pool,
                            const void* v_pool, int64_t num_pages, const int32_t* block_table,
                            int32_t max_blocks, const int32_t* seq_lens, int32_t num_seqs,
                            const int32_t* sel, const int32_t* cnt, void* out,
                            float* lse_out, void* ws, const DecodeLayout& l) {
  char* w = static_cast<char*>(ws);
  msa::AttendArgs a{};
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.num_pages = num_pages;
  a.block_table = block_table;
  a.max_blocks = max_blocks;
  a.seq_lens = seq_lens;
  a.cu_seqlens_q = nullptr;
  a.num_seqs = num_seqs;
  a.num_tokens = num_seqs;
  a.sel = sel;
  a.cnt = cnt;
  a.kmax = kmax_of(p);
  a.forced_in_budget = p.forced_in_budget;
  a.hkv = p.num_kv_heads;
  a.hidx = p.num_idx_heads;
  a.bps = l.bps;
  a.nsplit_max = l.nsplit_max;
  const float ks = scaled_kv(p.kv_dtype) ? p.k_scale : 1.f;
  a.qk_scale_log2 = softmax_scale_of(p) * ks * 1.4426950408889634f;
  a.v_scale = scaled_kv(p.kv_dtype) ? p.v_scale : 1.f;
  a.out = out;
  a.lse_out = lse_out;
  a.part_o = reinterpret_cast<float*>(w + l.part_o);
  a.part_lse = reinterpret_cast<float*>(w + l.part_lse);
  a.tickets = reinterpret_cast<uint32_t*>(w + l.tickets);
  return a;
}

// Scratch of msa_sparse_decode_noalloc: the decode workspace of callers that
// cannot allocate.  One copy per GPU, held until the process ends.  Host code
// never uses the array's name as an address: each device's address comes from
// hipGetSymbolAddress, taken once per device with that device current.
constexpr size_t kScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

msa_status_t scratch_of_current_device(void** out) {
  int dev = -1;
  msa_status_t st = hip_status(hipGetDevice(&dev), "hipGetDevice");
  if (st != MSA_OK) return st;
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MSA_ERR_UNSUPPORTED, "device %d: scratch is kept for devices 0..%d", dev,
                kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    st = hip_status(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "hipGetSymbolAddress");
    if (st != MSA_OK) return st;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MSA_OK;
}

// Decode with the caller's workspace, or (use_scratch) with this device's
// scratch.  Everything is validated before the first launch.
msa_status_t sparse_decode_impl(const msa_params_t* params, const void* q, const void* idx_q,
                                const void* k_pool, const void* v_pool, const void* idx_k_pool,
                                const void* idx_v_pool, int64_t num_pages,
                                const int32_t* block_table, int32_t max_blocks,
                                const int32_t* seq_lens, int32_t num_seqs, void* out,
                                void* idx_out, float* lse_out, int32_t* sel_blocks_out,
                                int32_t* sel_count_out, void* ws, size_t ws_bytes,
                                bool use_scratch, void* stream) {
  msa_status_t st = check_params(params);
  if (st != MSA_OK) return st;
  if ((st = check_shape(num_seqs, max_blocks)) != MSA_OK) return st;
  if (!q || !idx_q || !k_pool || !v_pool || !idx_k_pool || !block_table || !seq_lens || !out)
    return fail(MSA_ERR_INVALID_ARG, "NULL tensor pointer");
  if ((sel_blocks_out == nullptr) != (sel_count_out == nullptr))
    return fail(MSA_ERR_INVALID_ARG, "sel_blocks_out and sel_count_out go together");
  if (num_pages < 1) return fail(MSA_ERR_INVALID_ARG, "num_pages=%lld < 1", (long long)num_pages);
  if ((st = check_iv(*params, idx_v_pool, idx_out, "idx_v_pool and idx_out")) != MSA_OK) return st;
  const msa_params_t& p = *params;
  const DecodeLayout l = decode_layout(p, num_seqs, max_blocks);
  if ((st = check_grid(scan_workgroups(num_seqs, p.num_idx_heads, max_blocks), kScanThreads,
                       "index scan")) != MSA_OK ||
      (st = check_grid(attend_workgroups(l.nsplit_max, p.num_kv_heads, num_seqs),
                       kAttendThreads, "decode attention")) != MSA_OK)
    return st;
  if (use_scratch) {
    if (l.total > kScratchBytes)
      return fail(MSA_ERR_UNSUPPORTED,
                  "B=%d with max_blocks=%d needs %zu bytes of decode scratch; the library holds "
                  "%zu (use msa_sparse_decode with a workspace)",
                  num_seqs, max_blocks, l.total, kScratchBytes);
    if ((st = scratch_of_current_device(&ws)) != MSA_OK) return st;
    ws_bytes = kScratchBytes;
  }
  if ((st = check_ws(ws, ws_bytes, l.total)) != MSA_OK) return st;
  log_line("msa_sparse_decode%s: B=%d max_blocks=%d scan grid %d (%d pages per item), attention "
           "grid %d x %d x %d (%d blocks per split), G=%d", use_scratch ? "_noalloc" : "",
           num_seqs, max_blocks,
           num_seqs * p.num_idx_heads * ((max_blocks + kPagesPerItem - 1) / kPagesPerItem),
           kPagesPerItem, l.nsplit_max, p.num_kv_heads, num_seqs, l.bps, group_of(p));
  if (num_seqs == 0) return ok();
  const hipStream_t s = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);

  // 1. scores of every visible block; workgroup 0 also zeroes the split
  //    tickets of step 2
  msa::ScoreArgs a{};
  a.idx_q = idx_q;
  a.idx_k = idx_k_pool;
  a.num_pages = num_pages;
  a.block_table = block_table;
  a.max_blocks = max_blocks;
  a.seq_lens = seq_lens;
  a.num_seqs = num_seqs;
  a.hidx = p.num_idx_heads;
  a.pages_per_item = kPagesPerItem;
  a.chunks_per_pair = (max_blocks + kPagesPerItem - 1) / kPagesPerItem;
  a.scores = reinterpret_cast<float*>(w + l.scores);
  a.fill_tail = 0;
  a.zero_words = reinterpret_cast<uint32_t*>(w + l.tickets);
  a.zero_count = num_seqs * p.num_kv_heads;
  a.st_scale_log2 = score_scale_log2(p);
  if (p.index_value) {
    a.idx_v = idx_v_pool;
    a.iv_part = reinterpret_cast<float*>(w + l.iv_part);
    a.iv_scale_log2 = 1.4426950408889634f / std::sqrt(float(p.idx_dim));
  }
  st = hip_status(msa::launch_decode_score(a, p.idx_dtype, p.idx_dim, p.score_type, s),
                  "score launch");
  if (st != MSA_OK) return st;
  // 2. selection inside each attention workgroup, split-K attention, combine
  msa::AttendArgs aa = attend_args(p, q, k_pool, v_pool, num_pages, block_table, max_blocks,
                                   seq_lens, num_seqs, nullptr, nullptr, out, lse_out, ws, l);
  aa.scores = a.scores;
  aa.topk = p.topk;
  aa.init = p.init_blocks;
  aa.local = p.local_blocks;
  aa.sel_out = sel_blocks_out;
  aa.cnt_out = sel_count_out;
  if (p.index_value) {
    aa.iv_part = a.iv_part;
    aa.idx_out = idx_out;
    aa.iv_chunks = a.chunks_per_pair;
    aa.iv_pages = kPagesPerItem;
    aa.idx_dim = p.idx_dim;
  }
  st = hip_status(msa::launch_decode_attend(aa, p.q_dtype, p.kv_dtype, group_of(p), s),
                  "attention launch");
  return st == MSA_OK ? ok() : st;
}

}  // namespace

extern "C" {

int32_t msa_version(void) { return (1 << 16) | 0; }

const char* msa_status_string(msa_status_t st) {
  switch (st) {
    case MSA_OK: return "ok";
    case MSA_ERR_INVALID_ARG: return "invalid argument";
    case MSA_ERR_UNSUPPORTED: return "unsupported";
    case MSA_ERR_WORKSPACE: return "workspace too small or misaligned";
    case MSA_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* msa_last_error(void) { return g_err; }

size_t msa_decode_workspace_size(const msa_params_t* params, int32_t num_seqs,
                                 int32_t max_blocks) {
  if (check_params(params) != MSA_OK) return 0;
  if (check_shape(num_seqs, max_blocks) != MSA_OK) return 0;
  return decode_layout(*params, num_seqs, max_blocks).total;
}

size_t msa_prefill_workspace_size(const msa_params_t* params, int32_t num_seqs,
                                  int32_t num_q_tokens, int32_t max_blocks) {
  if (check_params(params) != MSA_OK) return 0;
  if (check_shape(num_seqs, max_blocks) != MSA_OK) return 0;
  if (num_q_tokens < 0) {
    fail(MSA_ERR_INVALID_ARG, "num_q_tokens=%d < 0", num_q_tokens);
    return 0;
  }
  if (num_q_tokens >= kMaxPrefillTokens) {
    fail(MSA_ERR_UNSUPPORTED, "num_q_tokens=%d above %d", num_q_tokens, kMaxPrefillTokens - 1);
    return 0;
  }
  return prefill_layout(*params, num_seqs, num_q_tokens, max_blocks).total;
}

msa_status_t msa_block_score(const msa_params_t* params, const void* idx_q,
                             const void* idx_k_pool, int64_t num_pages,
                             const int32_t* block_table, int32_t max_blocks,
                             const int32_t* seq_lens, const int32_t* cu_seqlens_q,
                             int32_t num_seqs, int32_t num_q_tokens, float* scores,
                             void* stream) {
  msa_status_t st = check_params(params);
  if (st != MSA_OK) return st;
  if ((st = check_shape(num_seqs, max_blocks)) != MSA_OK) return st;
  if (!idx_q || !idx_k_pool || !block_table || !seq_lens || !scores)
    return fail(MSA_ERR_INVALID_ARG, "NULL tensor pointer");
  if (num_pages < 1) return fail(MSA_ERR_INVALID_ARG, "num_pages=%lld < 1", (long long)num_pages);
  if (num_seqs == 0) return ok();
  if (cu_seqlens_q != nullptr) {
    if (num_q_tokens < 0) return fail(MSA_ERR_INVALID_ARG, "num_q_tokens=%d < 0", num_q_tokens);
    if (params->idx_dtype != MSA_BF16)
      return fail(MSA_ERR_UNSUPPORTED, "prefill scoring needs bf16 index keys");
    if (num_q_tokens == 0) return ok();
    if (short_chunks(num_seqs, num_q_tokens)) {
      st = check_grid(scan_workgroups(num_seqs, params->num_idx_heads, max_blocks), kScanThreads,
                      "chunk scan");
    } else {
      st = check_grid(prefill_score_workgroups(num_seqs, params->num_idx_heads, max_blocks,
                                               num_q_tokens),
                      kScanThreads, "prefill scoring");
    }
    if (st != MSA_OK) return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    st = hip_status(msa::launch_fill_f32(scores, int64_t(num_q_tokens) * params->num_idx_heads *
                                                     max_blocks, -INFINITY, s),
                    "score fill launch");
    if (st != MSA_OK) return st;
    if (short_chunks(num_seqs, num_q_tokens)) {
      const msa::ScoreArgs ma =
          multi_score_args(*params, idx_q, idx_k_pool, num_pages, block_table, max_blocks,
                           seq_lens, cu_seqlens_q, num_seqs, scores);
      st = hip_status(msa::launch_multi_score(ma, params->idx_dim, params->score_type, s),
                      "chunk scan launch");
      return st == MSA_OK ? ok() : st;
    }
    const msa::PrefillScoreArgs pa =
        prefill_score_args(*params, idx_q, idx_k_pool, num_pages, block_table, max_blocks,
                           seq_lens, cu_seqlens_q, num_seqs, num_q_tokens, scores);
    st = hip_status(msa::launch_prefill_score(pa, params->idx_dim, params->score_type, s),
                    "prefill score launch");
    return st == MSA_OK ? ok() : st;
  }
  if ((st = check_grid(scan_workgroups(num_seqs, params->num_idx_heads, max_blocks),
                       kScanThreads, "index scan")) != MSA_OK)
    return st;
  msa::ScoreArgs a{};
  a.idx_q = idx_q;
  a.idx_k = idx_k_pool;
  a.num_pages = num_pages;
  a.block_table = block_table;
  a.max_blocks = max_blocks;
  a.seq_lens = seq_lens;
  a.num_seqs = num_seqs;
  a.hidx = params->num_idx_heads;
  a.pages_per_item = kPagesPerItem;
  a.chunks_per_pair = (max_blocks + kPagesPerItem - 1) / kPagesPerItem;
  a.scores = scores;
  a.fill_tail = 1;
  a.st_scale_log2 = score_scale_log2(*params);
  st = hip_status(msa::launch_decode_score(a, params->idx_dtype, params->idx_dim,
                                           params->score_type, static_cast<hipStream_t>(stream)),
                  "block score launch");
  return st == MSA_OK ? ok() : st;
}

msa_status_t msa_select_blocks(const msa_params_t* params, const float* scores,
                               int32_t max_blocks, const int32_t* seq_lens,
                               const int32_t* cu_seqlens_q, int32_t num_seqs,
                               int32_t num_q_tokens, int32_t* sel_blocks,
                               int32_t* sel_count, void* stream) {
  msa_status_t st = check_params(params);
  if (st != MSA_OK) return st;
  if ((st = check_shape(num_seqs, max_blocks)) != MSA_OK) return st;
  if (!scores || !seq_lens || !sel_blocks || !sel_count)
    return fail(MSA_ERR_INVALID_ARG, "NULL tensor pointer");
  const int32_t T = cu_seqlens_q == nullptr ? num_seqs : num_q_tokens;
  if (T < 0) return fail(MSA_ERR_INVALID_ARG, "num_q_tokens=%d < 0", T);
  // (no sequences: nothing to select, as in msa_sparse_prefill; the kernel
  // reads at least one sequence's offsets)
  if (T == 0 || num_seqs == 0) return ok();
  if ((st = check_grid(select_workgroups(T, params->num_idx_heads, max_blocks), kScanThreads,
                       "selection")) != MSA_OK)
    return st;
  const msa::SelectArgs a = select_args(*params, scores, max_blocks, seq_lens, cu_seqlens_q,
                                        num_seqs, T, sel_blocks, sel_count);
  st = hip_status(launch_selection(a, static_cast<hipStream_t>(stream)), "select launch");
  return st == MSA_OK ? ok() : st;
}

msa_status_t msa_sparse_decode(const msa_params_t* params, const void* q, const void* idx_q,
                               const void* k_pool, const void* v_pool,
                               const void* idx_k_pool, const void* idx_v_pool,
                               int64_t num_pages, const int32_t* block_table,
                               int32_t max_blocks, const int32_t* seq_lens, int32_t num_seqs,
                               void* out, void* idx_out, float* lse_out,
                               int32_t* sel_blocks_out, int32_t* sel_count_out, void* ws,
                               size_t ws_bytes, void* stream) {
  return sparse_decode_impl(params, q, idx_q, k_pool, v_pool, idx_k_pool, idx_v_pool, num_pages,
                            block_table, max_blocks, seq_lens, num_seqs, out, idx_out, lse_out,
                            sel_blocks_out, sel_count_out, ws, ws_bytes, false, stream);
}

msa_status_t msa_sparse_decode_noalloc(const msa_params_t* params, const void* q,
                                       const void* idx_q, const void* k_pool,
                                       const void* v_pool, const void* idx_k_pool,
                                       const void* idx_v_pool, int64_t num_pages,
                                       const int32_t* block_table, int32_t max_blocks,
                                       const int32_t* seq_lens, int32_t num_seqs, void* out,
                                       void* idx_out, float* lse_out, int32_t* sel_blocks_out,
                                       int32_t* sel_count_out, void* stream) {
  return sparse_decode_impl(params, q, idx_q, k_pool, v_pool, idx_k_pool, idx_v_pool, num_pages,
                            block_table, max_blocks, seq_lens, num_seqs, out, idx_out, lse_out,
                            sel_blocks_out, sel_count_out, nullptr, 0, true, stream);
}

msa_status_t msa_sparse_attend(const msa_params_t* params, const void* q, const void* k_pool,
                               const void* v_pool, int64_t num_pages,
                               const int32_t* block_table, int32_t max_blocks,
                               const int32_t* seq_lens, int32_t num_seqs,
                               const int32_t* sel_blocks, const int32_t* sel_count, void* out,
                               float* lse_out, void* ws, size_t ws_bytes, void* stream) {
  msa_status_t st = check_params(params);
  if (st != MSA_OK) return st;
  if ((st = check_shape(num_seqs, max_blocks)) != MSA_OK) return st;
  if (!q || !k_pool || !v_pool || !block_table || !seq_lens || !sel_blocks || !sel_count || !out)
    return fail(MSA_ERR_INVALID_ARG, "NULL tensor pointer");
  if (num_pages < 1) return fail(MSA_ERR_INVALID_ARG, "num_pages=%lld < 1", (long long)num_pages);
  const DecodeLayout l = decode_layout(*params, num_seqs, max_blocks);
  if ((st = check_grid(attend_workgroups(l.nsplit_max, params->num_kv_heads, num_seqs),
                       kAttendThreads, "decode attention")) != MSA_OK)
    return st;
  if ((st = check_ws(ws, ws_bytes, l.total)) != MSA_OK) return st;
  log_line("msa_sparse_attend: B=%d attention grid %d x %d x %d (%d blocks per split)", num_seqs,
           l.nsplit_max, params->num_kv_heads, num_seqs, l.bps);
  if (num_seqs == 0) return ok();
  const hipStream_t s = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  st = hip_status(msa::launch_fill_u32(reinterpret_cast<uint32_t*>(w + l.tickets),
                                       int64_t(params->num_kv_heads) * num_seqs, 0u, s),
                  "ticket reset launch");
  if (st != MSA_OK) return st;
  const msa::AttendArgs aa =
      attend_args(*params, q, k_pool, v_pool, num_pages, block_table, max_blocks, seq_lens,
                  num_seqs, sel_blocks, sel_count, out, lse_out, ws, l);
  st = hip_status(msa::launch_decode_attend(aa, params->q_dtype, params->kv_dtype,
                                            group_of(*params), s),
                  "decode attend launch");
  return st == MSA_OK ? ok() : st;
}

msa_status_t msa_append_kv(const msa_params_t* params, const void* k_new, const void* v_new,
                           const void* idx_k_new, const void* idx_v_new,
                           const int64_t* slot_mapping, int32_t num_tokens, void* k_pool,
                           void* v_pool, void* idx_k_pool, void* idx_v_pool, int64_t num_pages,
                           void* stream) {
  msa_status_t st = check_params(params);
  if (st != MSA_OK) return st;
  if (!k_new || !v_new || !idx_k_new || !slot_mapping || !k_pool || !v_pool || !idx_k_pool)
    return fail(MSA_ERR_INVALID_ARG, "NULL tensor pointer");
  if ((st = check_iv(*params, idx_v_new, idx_v_pool, "idx_v_new and idx_v_pool")) != MSA_OK)
    return st;
  if (num_tokens < 0) return fail(MSA_ERR_INVALID_ARG, "num_tokens=%d < 0", num_tokens);
  if (num_pages < 1) return fail(MSA_ERR_INVALID_ARG, "num_pages=%lld < 1", (long long)num_pages);
  {
    const int64_t per_token = 2 * int64_t(params->num_kv_heads) * (params->head_dim / 8) +
                              (params->index_value ? 2 : 1) * int64_t(params->num_idx_heads) *
                                  (params->idx_dim / 8);
    if ((st = check_grid((int64_t(num_tokens) * per_token + 255) / 256, 256, "append")) !=
        MSA_OK)
      return st;
  }
  log_line("msa_append_kv: T=%d into %lld pages (kv dtype %d)", num_tokens,
           (long long)num_pages, params->kv_dtype);
  if (num_tokens == 0) return ok();
  msa::AppendArgs a{};
  a.k_new = k_new;
  a.v_new = v_new;
  a.idx_k_new = idx_k_new;
  a.slots = slot_mapping;
  a.num_tokens = num_tokens;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.idx_k_pool = idx_k_pool;
  a.idx_v_new = idx_v_new;
  a.idx_v_pool = idx_v_pool;
  a.num_pages = num_pages;
  a.hkv = params->num_kv_heads;
  a.hidx = params->num_idx_heads;
  a.head_dim = params->head_dim;
  a.idx_dim = params->idx_dim;
  a.k_scale = scaled_kv(params->kv_dtype) ? params->k_scale : 1.f;
  a.v_scale = scaled_kv(params->kv_dtype) ? params->v_scale : 1.f;
  st = hip_status(msa::launch_append(a, params->kv_dtype, params->idx_dtype,
                                     static_cast<hipStream_t>(stream)),
                  "append launch");
  return st == MSA_OK ? ok() : st;
}

msa_status_t msa_sparse_prefill(const msa_params_t* params, const void* q, const void* idx_q,
                                const void* k_pool, const void* v_pool,
                                const void* idx_k_pool, const void* idx_v_pool,
                                int64_t num_pages, const int32_t* block_table,
                                int32_t max_blocks, const int32_t* seq_lens,
                                const int32_t* cu_seqlens_q, int32_t num_seqs,
                                int32_t num_q_tokens, void* out, void* idx_out, float* lse_out,
                                int32_t* sel_blocks_out, int32_t* sel_count_out, void* ws,
                                size_t ws_bytes, void* stream) {
  msa_status_t st = check_params(params);
  if (st != MSA_OK) return st;
  if ((st = check_shape(num_seqs, max_blocks)) != MSA_OK) return st;
  if (!q || !idx_q || !k_pool || !v_pool || !idx_k_pool || !block_table || !seq_lens ||
      !cu_seqlens_q || !out)
    return fail(MSA_ERR_INVALID_ARG, "NULL tensor pointer");
  if ((sel_blocks_out == nullptr) != (sel_count_out == nullptr))
    return fail(MSA_ERR_INVALID_ARG, "sel_blocks_out and sel_count_out go together");
  if (num_pages < 1) return fail(MSA_ERR_INVALID_ARG, "num_pages=%lld < 1", (long long)num_pages);
  if (num_q_tokens < 0) return fail(MSA_ERR_INVALID_ARG, "num_q_tokens=%d < 0", num_q_tokens);
  if ((st = check_iv(*params, idx_v_pool, idx_out, "idx_v_pool and idx_out")) != MSA_OK) return st;
  const msa_params_t& p = *params;
  if (p.idx_dtype != MSA_BF16)
    return fail(MSA_ERR_UNSUPPORTED, "prefill scoring needs bf16 index keys");
  if (num_q_tokens >= kMaxPrefillTokens)
    return fail(MSA_ERR_UNSUPPORTED, "num_q_tokens=%d above %d", num_q_tokens,
                kMaxPrefillTokens - 1);
  const PrefillLayout l = prefill_layout(p, num_seqs, num_q_tokens, max_blocks);
  if (short_chunks(num_seqs, num_q_tokens)) {
    st = check_grid(scan_workgroups(num_seqs, p.num_idx_heads, max_blocks), kScanThreads,
                    "chunk scan");
  } else {
    st = check_grid(prefill_score_workgroups(num_seqs, p.num_idx_heads, max_blocks, num_q_tokens),
                    kScanThreads, "prefill scoring");
  }
  if (st != MSA_OK) return st;
  if ((st = check_grid(select_workgroups(num_q_tokens, p.num_idx_heads, max_blocks),
                       kScanThreads, "selection")) != MSA_OK)
    return st;
  if (prefill_key_major(p, num_seqs, num_q_tokens)) {
    // list kernels: one grid row per sequence; combine: 16 / G units per workgroup
    if (num_seqs > 65535)
      return fail(MSA_ERR_UNSUPPORTED, "num_seqs=%d above 65535 for a long prefill chunk",
                  num_seqs);
    const int per = 16 / group_of(p);
    if ((st = check_grid((int64_t(num_q_tokens) * p.num_kv_heads + per - 1) / per,
                         kScanThreads, "prefill combine")) != MSA_OK)
      return st;
  } else if ((st = check_grid(attend_workgroups(l.nsplit_max, p.num_kv_heads, num_q_tokens),
                              kAttendThreads, "per-token attention")) != MSA_OK) {
    return st;
  }
  if (p.index_value) {
    const int64_t tiles = (int64_t(num_q_tokens) + 255) / 256;
    if ((st = check_grid(int64_t(num_seqs) * tiles * p.num_idx_heads *
                             ((max_blocks + kPrefillBlocksPerChunk - 1) / kPrefillBlocksPerChunk),
                         kAttendThreads, "index-value attention")) != MSA_OK)
      return st;
  }
  if ((st = check_ws(ws, ws_bytes, l.total)) != MSA_OK) return st;
  if (short_chunks(num_seqs, num_q_tokens))
    log_line("msa_sparse_prefill: B=%d T=%d short chunks: scan with four queries per pass, "
             "per-token split-K (%d blocks per split)", num_seqs, num_q_tokens, l.bps);
  else if (prefill_key_major(p, num_seqs, num_q_tokens))
    log_line("msa_sparse_prefill: B=%d T=%d key-major: %d tokens per tile, at most %d tiles",
             num_seqs, num_q_tokens, l.tq, l.max_items);
  else
    log_line("msa_sparse_prefill: B=%d T=%d per-token split-K (%d blocks per split)", num_seqs,
             num_q_tokens, l.bps);
  if (num_seqs == 0 || num_q_tokens == 0) return ok();
  const hipStream_t s = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  int32_t* sel = sel_blocks_out ? sel_blocks_out : reinterpret_cast<int32_t*>(w + l.sel);
  int32_t* cnt = sel_count_out ? sel_count_out : reinterpret_cast<int32_t*>(w + l.cnt);
  float* scores = reinterpret_cast<float*>(w + l.scores);

  // index-value branch: its own kernels, independent of the selection
  if (p.index_value) {
    msa::PrefillValueArgs va{};
    va.idx_q = idx_q;
    va.idx_k = idx_k_pool;
    va.idx_v = idx_v_pool;
    va.num_pages = num_pages;
    va.block_table = block_table;
    va.max_blocks = max_blocks;
    va.seq_lens = seq_lens;
    va.cu_seqlens_q = cu_seqlens_q;
    va.num_seqs = num_seqs;
    va.num_tokens = num_q_tokens;
    va.hidx = p.num_idx_heads;
    va.max_tiles = (num_q_tokens + 255) / 256;
    va.blocks_per_chunk = kPrefillBlocksPerChunk;
    va.kchunks = (max_blocks + kPrefillBlocksPerChunk - 1) / kPrefillBlocksPerChunk;
    va.scale_log2 = 1.4426950408889634f / std::sqrt(float(p.idx_dim));
    va.part_o = reinterpret_cast<float*>(w + l.iv_o);
    va.part_lse = reinterpret_cast<float*>(w + l.iv_lse);
    va.idx_out = idx_out;
    va.out_f32 = p.q_dtype == MSA_F32;
    st = hip_status(msa::launch_prefill_value(va, p.idx_dim, s), "index-value launch");
    if (st != MSA_OK) return st;
  }

  const bool key_major = prefill_key_major(p, num_seqs, num_q_tokens);
  // 1. scores (short chunks: page scan, several queries per pass; long
  //    chunks: causal GEMM with a block-max epilogue)
  if (short_chunks(num_seqs, num_q_tokens)) {
    const msa::ScoreArgs ma = multi_score_args(p, idx_q, idx_k_pool, num_pages, block_table,
                                               max_blocks, seq_lens, cu_seqlens_q, num_seqs,
                                               scores);
    st = hip_status(msa::launch_multi_score(ma, p.idx_dim, p.score_type, s), "chunk scan launch");
  } else {
    const msa::PrefillScoreArgs pa =
        prefill_score_args(p, idx_q, idx_k_pool, num_pages, block_table, max_blocks, seq_lens,
                           cu_seqlens_q, num_seqs, num_q_tokens, scores);
    st = hip_status(msa::launch_prefill_score(pa, p.idx_dim, p.score_type, s),
                    "prefill score launch");
  }
  if (st != MSA_OK) return st;
  // 2. per-token selection; its workgroups also clear the k2q list counts
  //    (key-major attention) or the split tickets (per-token attention)
  msa::SelectArgs sa = select_args(p, scores, max_blocks, seq_lens, cu_seqlens_q, num_seqs,
                                   num_q_tokens, sel, cnt);
  if (key_major) {
    sa.zero_words = reinterpret_cast<uint32_t*>(w + l.counts);
    sa.zero_count = 2 * int64_t(num_seqs) * p.num_idx_heads * max_blocks;
  } else if (l.nsplit_max > 1) {
    sa.zero_words = reinterpret_cast<uint32_t*>(w + l.tickets);
    sa.zero_count = int64_t(num_q_tokens) * p.num_kv_heads;
  }
  st = hip_status(launch_selection(sa, s), "prefill select launch");
  if (st != MSA_OK) return st;
  // 3. attention over each token's selection
  if (key_major) {
    msa::PrefillAttnArgs ka{};
    ka.q = q;
    ka.k_pool = k_pool;
    ka.v_pool = v_pool;
    ka.num_pages = num_pages;
    ka.block_table = block_table;
    ka.max_blocks = max_blocks;
    ka.seq_lens = seq_lens;
    ka.cu_seqlens_q = cu_seqlens_q;
    ka.num_seqs = num_seqs;
    ka.num_tokens = num_q_tokens;
    ka.sel = sel;
    ka.cnt = cnt;
    ka.kmax = kmax_of(p);
    ka.hkv = p.num_kv_heads;
    ka.hidx = p.num_idx_heads;
    ka.tq = l.tq;
    ka.init = p.init_blocks;
    ka.local = p.local_blocks;
    ka.forced_split = p.init_blocks + p.local_blocks > 0 ? 1 : 0;
    ka.counts = reinterpret_cast<int32_t*>(w + l.counts);
    ka.cursor = reinterpret_cast<int32_t*>(w + l.cursor);
    ka.tok_off = reinterpret_cast<int32_t*>(w + l.tok_off);
    ka.tile_off = reinterpret_cast<int32_t*>(w + l.tile_off);
    ka.csr = reinterpret_cast<int32_t*>(w + l.csr);
    ka.items = reinterpret_cast<msa::Tile*>(w + l.items);
    ka.n_items = reinterpret_cast<int32_t*>(w + l.n_items);
    ka.forced_off = reinterpret_cast<int32_t*>(w + l.forced_off);
    ka.tqf = msa::kForcedRows / group_of(p);
    ka.max_items = l.max_items;
    const float ks = scaled_kv(p.kv_dtype) ? p.k_scale : 1.f;
    ka.qk_scale_log2 = softmax_scale_of(p) * ks * 1.4426950408889634f;
    ka.v_scale = scaled_kv(p.kv_dtype) ? p.v_scale : 1.f;
    ka.part_o = reinterpret_cast<uint16_t*>(w + l.part_o);
    ka.part_lse = reinterpret_cast<float*>(w + l.part_lse);
    ka.sink_o = reinterpret_cast<uint16_t*>(w + l.sink);
    ka.sink_lse = reinterpret_cast<float*>(w + l.sink + sizeof(uint16_t) * group_of(p) * p.head_dim);
    ka.out = out;
    ka.lse_out = lse_out;
    st = hip_status(msa::launch_prefill_k2q(ka, s), "prefill k2q launch");
    if (st != MSA_OK) return st;
    st = hip_status(msa::launch_prefill_attend(ka, p.kv_dtype, group_of(p), s),
                    "prefill attention launch");
    return st == MSA_OK ? ok() : st;
  }
  msa::AttendArgs aa{};
  aa.q = q;
  aa.k_pool = k_pool;
  aa.v_pool = v_pool;
  aa.num_pages = num_pages;
  aa.block_table = block_table;
  aa.max_blocks = max_blocks;
  aa.seq_lens = seq_lens;
  aa.cu_seqlens_q = cu_seqlens_q;
  aa.num_seqs = num_seqs;
  aa.num_tokens = num_q_tokens;
  aa.sel = sel;
  aa.cnt = cnt;
  aa.kmax = kmax_of(p);
  aa.forced_in_budget = p.forced_in_budget;
  aa.hkv = p.num_kv_heads;
  aa.hidx = p.num_idx_heads;
  aa.bps = l.bps;
  aa.nsplit_max = l.nsplit_max;
  const float ks = scaled_kv(p.kv_dtype) ? p.k_scale : 1.f;
  aa.qk_scale_log2 = softmax_scale_of(p) * ks * 1.4426950408889634f;
  aa.v_scale = scaled_kv(p.kv_dtype) ? p.v_scale : 1.f;
  aa.out = out;
  aa.lse_out = lse_out;
  aa.part_o = reinterpret_cast<float*>(w + l.part_o);
  aa.part_lse = reinterpret_cast<float*>(w + l.part_lse);
  aa.tickets = reinterpret_cast<uint32_t*>(w + l.tickets);
  st = hip_status(msa::launch_decode_attend(aa, p.q_dtype, p.kv_dtype, group_of(p), s),
                  "prefill attend launch");
  return st == MSA_OK ? ok() : st;
}

msa_status_t msa_fp8_dequant(const uint8_t* in, float* out, int64_t n, float scale,
                             int32_t dtype, void* stream) {
  if (n < 0) return fail(MSA_ERR_INVALID_ARG, "n=%lld < 0", (long long)n);
  if (n > 0 && (!in || !out)) return fail(MSA_ERR_INVALID_ARG, "NULL tensor pointer");
  if (!std::isfinite(scale)) return fail(MSA_ERR_INVALID_ARG, "scale must be finite");
  if (!scaled_kv(dtype))
    return fail(MSA_ERR_UNSUPPORTED, "dtype=%d is not an fp8 or MX format", dtype);
  if (is_mx(dtype) && n % 32 != 0)
    return fail(MSA_ERR_INVALID_ARG, "MX format: n=%lld is not a multiple of 32", (long long)n);
  msa_status_t st = check_grid((n / 8 + 1 + 255) / 256, 256, "fp8 dequant");
  if (st != MSA_OK) return st;
  st = hip_status(
      msa::launch_fp8_dequant(in, out, n, scale, dtype, static_cast<hipStream_t>(stream)),
      "fp8 dequant launch");
  return st == MSA_OK ? ok() : st;
}

msa_status_t msa_fp8_e4m3_dequant(const uint8_t* in, float* out, int64_t n, float scale,
                                  void* stream) {
  return msa_fp8_dequant(in, out, n, scale, MSA_FP8_E4M3, stream);
}

}  // extern "C"
