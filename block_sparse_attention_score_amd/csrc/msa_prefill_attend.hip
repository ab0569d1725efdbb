// Chunked-prefill attention, key-major.
//
// Selection is per query token (sglang page minimax_sparse_backend.py,
// MiniMaxSparseAttnBackend.__init__: one query per selection block), so in a
// prefill chunk every key block j of a sequence is attended by the tokens
// that selected it.  The vLLM page sparse_attention_msa.py (its module
// docstring, and the prefill part of MiniMaxM3SparseMSAImpl.forward:
// build_k2q_csr, then sparse_atten_func) builds, per (sequence, head, key
// block), the list of those tokens and runs key-major attention tiles over it;
// this file does the same on gfx950:
//   1. k2q CSR: count the selecting tokens of every (b, index head, j), scan
//      the counts into list offsets and 256-row work tiles, fill the lists;
//   2. per tile: up to 256 query rows (tokens x GQA heads of one kv head,
//      eight waves of 32 rows) against block j, staged once in LDS (K as
//      [key][dim], V as [dim][key] with the dims permuted so that each lane
//      ends up holding 8-dim runs of its output row); S^T = K Q^T and
//      O^T = V^T P^T on bf16 MFMA, causal mask per row; a normalised partial
//      (o in bf16, lse in f32) per (token, kv head, slot);
//   3. the forced blocks (the first `init` and the last `local` visible blocks
//      of every token) query-major: consecutive tokens share them, so one
//      workgroup runs a group of tokens over their union with an online
//      softmax and writes one partial per (token, kv head); the lists of
//      step 1 hold only the top-k entries;
//   4. per (token, kv head), the log-sum-exp combine of its partials.
#include "msa_device.h"
#include "msa_internal.h"

namespace msa {

namespace {

constexpr int kPfWaves = 8;                 // waves of a tile workgroup
constexpr int kPfThreads = kPfWaves * kWave;
constexpr int kRows = kPrefillTileRows;     // query rows (token x head) per tile
static_assert(kRows == 32 * kPfWaves, "each wave owns 32 query rows");
// LDS row strides in bf16 elements, chosen by the bank conflicts measured on
// gfx950 (rocprofv3 SQ_LDS_BANK_CONFLICT over each access pattern): the
// 16-byte K fragment reads of 16 rows are conflict-free at a 288-byte row
// (272 bytes cost a fifth more cycles), the 8-byte V^T fragment reads at 264
// bytes (272: a fifth more), and the transposing 8-byte V^T stores conflict
// half as often at 264 as at 272 bytes.
constexpr int kStrideK = 144;
constexpr int kStrideV = 132;
constexpr float kLn2f = 0.69314718055994531f;

struct PfStage {
  alignas(16) uint16_t k[kBlock * kStrideK];   // K   [key][dim]
  alignas(16) uint16_t vt[kBlock * kStrideV];  // V^T [dim][key]
  int tok[kRows];                 // token of each token slot of the tile (-1: none)
  int slot[kRows];                // its slot in the token's selection
  int pos[kRows];                 // its position in the sequence
};
// Two stages: tile i is computed from one while tile i+1 is written to the
// other.
struct PfLds {
  PfStage st[2];
};

// LDS fragments through 16- and 8-byte vector types (single ds_read_b128 /
// ds_read_b64; every address below is aligned to the type).
__device__ __forceinline__ bf16x8_t lds_b128(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8_t*>(p);
}
__device__ __forceinline__ u32x2_t lds_b64(const uint16_t* p) {
  return *reinterpret_cast<const u32x2_t*>(p);
}

// Sum and max over the four 16-lane rows (lanes l, l^16, l^32, l^48) with
// the gfx950 row-swap moves instead of LDS permutes; every lane gets the
// same result.
__device__ __forceinline__ float rows_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = max_nan(__uint_as_float(r[0]), __uint_as_float(r[1]));
  const auto r2 = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return max_nan(__uint_as_float(r2[0]), __uint_as_float(r2[1]));
}
__device__ __forceinline__ float rows_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  const auto r2 = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __uint_as_float(r2[0]) + __uint_as_float(r2[1]);
}

// Eight consecutive bf16 elements through the caches (a query row is
// gathered by every tile that holds one of its token's slots).
__device__ __forceinline__ bf16x8_t load8_cached(const BF16*, const void* base, int64_t idx) {
  bf16x8_t r;
  __builtin_memcpy(&r, reinterpret_cast<const uint16_t*>(base) + idx, 16);
  return r;
}
// Buffer descriptor of one (page, head) run of a pool: base = pool + byte
// offset, raw 32-bit words, 64 KB of records (bounds beyond read as 0).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t run_rsrc(const void* pool, int64_t byte_off) {
  return __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(reinterpret_cast<const char*>(pool) + byte_off), 0, kBlock * 128 * 4,
      0x00020000);
}
template <class T>
struct RawOf;
template <>
struct RawOf<BF16> {
  typedef uint16_t elem;
};
template <>
struct RawOf<FP8> {
  typedef uint8_t elem;
};
template <>
struct RawOf<BF8> {
  typedef uint8_t elem;
};
template <>
struct RawOf<FP4> {
  typedef uint8_t elem;  // (unused: MX-fp4 runs are addressed in bytes below)
};
template <>
struct RawOf<FP6> {
  typedef uint8_t elem;  // (unused: MX-fp6 runs are addressed in bytes below)
};
// Eight E2M3 codes (dims d0 .. d0 + 7, d0 a multiple of 8, of a key row) from
// an MX-fp6 run, times their group's scale: the 6 code bytes start at row * 96
// + 3 d0 / 4, 4-byte aligned when d0 / 8 is even and 2 bytes past that
// otherwise, so one dword-aligned 8-byte load covers them; the codes are
// shifted down to bit 0 and converted by the 32-code instruction (its upper
// 24 codes zero and unused).
__device__ __forceinline__ bf16x8_t fp6x8_load(__amdgpu_buffer_rsrc_t r, uint32_t row_byte,
                                               int d0, uint32_t soff, uint32_t scale_off) {
  const uint32_t b = static_cast<uint32_t>(3 * d0 / 4);
  const auto raw = __builtin_amdgcn_raw_buffer_load_b64(r, row_byte + (b & ~3u), soff, 0);
  const uint64_t v = (static_cast<uint64_t>(raw[1]) << 32 | raw[0]) >> (8 * (b & 3u));
  const uint32_t e = __builtin_amdgcn_raw_buffer_load_b8(r, scale_off, 0, 0);
  const uint32_t w[6] = {static_cast<uint32_t>(v), static_cast<uint32_t>(v >> 32) & 0xffffu,
                         0u, 0u, 0u, 0u};
  return bf16x32_part(fp6x32_to_bf16x32(w, e8m0_to_f32(e)), 0);
}
// Eight elements at byte offset voff + soff of a run, as bf16.
__device__ __forceinline__ bf16x8_t load8_buf(const BF16*, __amdgpu_buffer_rsrc_t r, uint32_t voff,
                                              uint32_t soff) {
  return __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ bf16x8_t load8_buf(const FP8*, __amdgpu_buffer_rsrc_t r, uint32_t voff,
                                              uint32_t soff) {
  const auto raw = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
  return fp8x8_to_bf16x8(raw[0], raw[1]);
}
__device__ __forceinline__ bf16x8_t load8_buf(const BF8*, __amdgpu_buffer_rsrc_t r, uint32_t voff,
                                              uint32_t soff) {
  const auto raw = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
  return bf8x8_to_bf16x8(raw[0], raw[1]);
}

// V^T rows are staged in a permuted dim order: MFMA result row 16 dt + 4 q4
// + r of O^T holds dim 32 (dt / 2) + 8 q4 + 4 (dt % 2) + r, so lane q4 of a
// query row holds dims 32 k + 8 q4 .. + 8 (from dt = 2k, 2k + 1) and the
// four lanes of the row store 64 contiguous bytes per instruction.  The LDS
// row of dim D is the inverse map.
__device__ __forceinline__ int vt_row_of_dim(int D) {
  return 16 * (2 * (D >> 5) + ((D >> 2) & 1)) + 4 * ((D >> 3) & 3) + (D & 3);
}

// Clears v unless keep, without a branch.
__device__ __forceinline__ void mask_bf16x8(bf16x8_t& v, bool keep) {
  uint32_t u[4];
  __builtin_memcpy(u, &v, 16);
  const uint32_t m = keep ? 0xffffffffu : 0u;
#pragma unroll
  for (int i = 0; i < 4; ++i) u[i] &= m;
  __builtin_memcpy(&v, u, 16);
}

// 2^x on the hardware instruction: 2^-inf = 0, results below 2^-126 flush
// to zero (probabilities that small do not change a bf16 P or an f32 sum).
__device__ __forceinline__ float exp2_raw(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint32_t pack2_rne(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v;
  v[0] = static_cast<__bf16>(lo);
  v[1] = static_cast<__bf16>(hi);
  uint32_t u;
  __builtin_memcpy(&u, &v, 4);
  return u;
}

typedef const __attribute__((address_space(4))) Tile ConstTile;
__device__ __forceinline__ Tile read_tile(const ConstTile* p) {
  Tile m;
  m.c0 = p->c0;
  m.ntok = p->ntok;
  m.j = p->j;
  m.nvalid = p->nvalid;
  m.p0 = p->p0;
  m.g0 = p->g0;
  m.head0 = p->head0;
  return m;
}

}  // namespace

// The forced blocks of the token at position p (a selection row of nb = p /
// 128 + 1 visible blocks, clipped to the table): [0, init') and [lo, nb), as
// the selection forces them, and the token's first forced selection slot,
// where its forced partial goes.  All empty when the forced blocks are not
// split off.
struct ForcedRange {
  int init_end;  // init' = min(init, nb)
  int lo;        // first local block, max(0, nb - local) (nb when local = 0)
  int nb;
  __device__ bool has(int j) const { return j < init_end || (j >= lo && j < nb); }
  __device__ int count() const { return init_end + (nb - lo) - max(0, init_end - lo); }
  // the selection lists the forced blocks first (init) and last (local), in
  // ascending order: the first forced slot is 0, or cnt - (forced count) when
  // init' = 0
  __device__ int first_slot(int cnt) const { return init_end > 0 ? 0 : cnt - count(); }
};
__device__ __forceinline__ ForcedRange forced_range(const PrefillAttnArgs& a, int p) {
  ForcedRange r;
  r.nb = (a.forced_split && p >= 0) ? min(p / kBlock + 1, a.max_blocks) : 0;
  r.init_end = min(a.init, r.nb);
  r.lo = a.local > 0 ? max(0, r.nb - a.local) : r.nb;
  return r;
}

// ---------------------------------------------------------------- k2q CSR

// Workgroup (chunk c, sequence b, index head h): the 256 tokens
// cu[b] + 256 c + tid count their selected blocks in an LDS histogram of the
// sequence's max_blocks bins, then add the non-zero bins to the lists' counts
// (blocks many tokens select cost one global atomic per bin).  With the
// forced blocks split off, a token's init and local entries are left out.
__global__ __launch_bounds__(kWgThreads) void k2q_count_kernel(PrefillAttnArgs a) {
  extern __shared__ int hist[];
  const int b = blockIdx.y;
  const int h = blockIdx.z;
  const int tid = threadIdx.x;
  const int cu0 = a.cu_seqlens_q[b];
  const int n_b = a.cu_seqlens_q[b + 1] - cu0;
  if (static_cast<int>(blockIdx.x) * kWgThreads >= n_b) return;
  for (int i = tid; i < a.max_blocks; i += kWgThreads) hist[i] = 0;
  __syncthreads();
  const int i_tok = blockIdx.x * kWgThreads + tid;
  if (i_tok < n_b) {
    const int row = (cu0 + i_tok) * a.hidx + h;
    const int n = min(max(a.cnt[row], 0), a.kmax);
    const ForcedRange fr = forced_range(a, a.seq_lens[b] - n_b + i_tok);
    for (int s = 0; s < n; ++s) {
      const int j = a.sel[static_cast<int64_t>(row) * a.kmax + s];
      if (j >= 0 && j < a.max_blocks && !fr.has(j)) atomicAdd(&hist[j], 1);
    }
  }
  __syncthreads();
  int32_t* c = a.counts + (static_cast<int64_t>(b) * a.hidx + h) * a.max_blocks;
  for (int i = tid; i < a.max_blocks; i += kWgThreads)
    if (hist[i] > 0) atomicAdd(c + i, hist[i]);
}

// One workgroup: exclusive scans of the counts (list offsets) and of the
// tiles per list (work-tile offsets), lists in rounds of 1024, one per
// thread; the fill kernel writes the tiles themselves.
__global__ __launch_bounds__(1024) void k2q_scan_kernel(PrefillAttnArgs a, int n) {
  __shared__ int wsum[16];
  __shared__ int carry[2];
  const int tid = threadIdx.x;
  if (tid == 0) carry[0] = carry[1] = 0;
  __syncthreads();
  for (int base = 0; base < n; base += 1024) {
    const int i = base + tid;
    const int c = i < n ? a.counts[i] : 0;
    const int nt = (c + a.tq - 1) / a.tq;
    const int c0 = carry[0], t0 = carry[1];
    const int incl_c = block_incl_scan(c, wsum);
    const int incl_t = block_incl_scan(nt, wsum);
    if (i < n) {
      a.tok_off[i] = c0 + incl_c - c;
      a.tile_off[i] = t0 + incl_t - nt;
    }
    if (tid == 1023) {  // (every thread read the carry before the scans' barriers)
      carry[0] = c0 + incl_c;
      carry[1] = t0 + incl_t;
    }
    __syncthreads();
  }
  if (tid == 0) *a.n_items = min(carry[1], a.max_items);
  // forced-block token groups of each sequence, exclusive prefix (the forced
  // kernel's units, sequence by sequence)
  if (a.forced_split) {
    __syncthreads();
    if (tid == 0) carry[0] = 0;
    __syncthreads();
    for (int base = 0; base < a.num_seqs; base += 1024) {
      const int i = base + tid;
      const int ng = i < a.num_seqs
                         ? (a.cu_seqlens_q[i + 1] - a.cu_seqlens_q[i] + a.tqf - 1) / a.tqf
                         : 0;
      const int c0 = carry[0];
      const int incl = block_incl_scan(ng, wsum);
      if (i < a.num_seqs) a.forced_off[i] = c0 + incl - ng;
      if (tid == 1023) carry[0] = c0 + incl;
      __syncthreads();
    }
    if (tid == 0) a.forced_off[a.num_seqs] = carry[0];
  }
}

// Same workgroups as the count: append (token, slot) to the list of every
// selected block.  Each non-zero bin reserves its range of the list with one
// global atomic; LDS atomics hand out the places inside it.  The order inside
// a list is arbitrary; every query row of a tile is computed on its own, so
// results do not depend on it.
__global__ __launch_bounds__(kWgThreads) void k2q_fill_kernel(PrefillAttnArgs a) {
  extern __shared__ int hist[];
  const int b = blockIdx.y;
  const int h = blockIdx.z;
  const int tid = threadIdx.x;
  const int cu0 = a.cu_seqlens_q[b];
  const int n_b = a.cu_seqlens_q[b + 1] - cu0;
  if (static_cast<int>(blockIdx.x) * kWgThreads >= n_b) return;
  for (int i = tid; i < a.max_blocks; i += kWgThreads) hist[i] = 0;
  __syncthreads();
  const int i_tok = blockIdx.x * kWgThreads + tid;
  const int t = cu0 + i_tok;
  const int row = t * a.hidx + h;
  const int n = i_tok < n_b ? min(max(a.cnt[row], 0), a.kmax) : 0;
  const ForcedRange fr = forced_range(a, a.seq_lens[b] - n_b + i_tok);
  for (int s = 0; s < n; ++s) {
    const int j = a.sel[static_cast<int64_t>(row) * a.kmax + s];
    if (j >= 0 && j < a.max_blocks && !fr.has(j)) atomicAdd(&hist[j], 1);
  }
  __syncthreads();
  const int64_t bh0 = (static_cast<int64_t>(b) * a.hidx + h) * a.max_blocks;
  for (int i = tid; i < a.max_blocks; i += kWgThreads)
    if (hist[i] > 0) hist[i] = a.tok_off[bh0 + i] + atomicAdd(a.cursor + bh0 + i, hist[i]);
  __syncthreads();
  for (int s = 0; s < n; ++s) {
    const int j = a.sel[static_cast<int64_t>(row) * a.kmax + s];
    if (j < 0 || j >= a.max_blocks || fr.has(j)) continue;
    a.csr[atomicAdd(&hist[j], 1)] = (t << 8) | s;
  }

  // The work tiles of the lists j = blockIdx.x, blockIdx.x + nact, ... of
  // (b, h), nact being the sequence's active chunks, dealt to the waves; one
  // tile per lane, with the page, the sequence bounds and the pool offset
  // resolved, so that consecutive lanes store consecutive records.
  constexpr int kWaves = kWgThreads / kWave;
  const int nact = (n_b + kWgThreads - 1) / kWgThreads;
  const int lane = tid & (kWave - 1);
  const int L = a.seq_lens[b];
  const int p0 = L - n_b - cu0;
  const int g0 = h * (a.hkv / a.hidx);
  for (int j = blockIdx.x + nact * (tid / kWave); j < a.max_blocks; j += nact * kWaves) {
    const int c = a.counts[bh0 + j];
    if (c == 0) continue;
    const int et = a.tile_off[bh0 + j];
    const int ec = a.tok_off[bh0 + j];
    const int nt = (c + a.tq - 1) / a.tq;
    const int page = a.block_table[static_cast<int64_t>(b) * a.max_blocks + j];
    const bool page_ok = page >= 0 && page < a.num_pages;
    for (int k = lane; k < nt && et + k < a.max_items; k += kWave) {
      Tile m;
      m.c0 = ec + k * a.tq;
      m.ntok = min(a.tq, c - k * a.tq);
      m.j = j;
      // keys at or past the sequence end hold stale bytes: staged as zeros
      m.nvalid = page_ok ? max(0, min(kBlock, L - j * kBlock)) : 0;
      m.p0 = p0;
      m.g0 = g0;
      m.head0 = (static_cast<int64_t>(page_ok ? page : 0) * a.hkv + g0) * kBlock * 128;
      a.items[et + k] = m;
    }
  }
}

// ------------------------------------------------------------ attention tile

// Persistent: the workgroups of one XCD (x, x + 8, ...) walk a contiguous
// range of tiles, so the tiles of a key block run on one XCD and its L2 serves
// the block to all of them.  Software pipeline over a workgroup's tiles
// i, i+1, i+2, i+3: while tile i is computed, the key block of tile i+1 and,
// after S^T, its query rows are in flight; the list entries of tile i+2 and
// the record of tile i+3 are being fetched.
template <class KT, int G>
__global__ __launch_bounds__(kPfThreads, 1) void prefill_attend_kernel(PrefillAttnArgs a) {
  __shared__ PfLds S;
  constexpr int TQ = kRows / G;  // tokens per tile
  const KT* ktag = nullptr;
  const BF16* qtag = nullptr;
  const int total = *a.n_items;
  const int per = (total + 7) / 8;
  const int stride = gridDim.x / 8;  // workgroups per XCD (grid is a multiple of 8)
  const int hi = min((blockIdx.x % 8 + 1) * per, total);
  int item = (blockIdx.x % 8) * per + blockIdx.x / 8;
  if (item >= hi) return;
  const int kv = blockIdx.y;                         // kv head within the index head's group
  const int64_t kv_off = static_cast<int64_t>(kv) * kBlock * 128;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int w = tid / kWave;
  const int l16 = lane & 15;
  const int q4 = lane >> 4;
  const int kr = tid >> 4;           // staging: K key 32 i + kr, V keys 4 kr .. + 4
  const int dc = (tid & 15) * 8;     // staging dims dc .. dc + 8
  const int hq_stride = a.hkv * G;

  // Query row r = 32 w + 16 nt + l16 of a tile is token slot r / G, head r % G.
  int qhh[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) qhh[nt] = (32 * w + 16 * nt + l16) % G;

  bf16x8_t qf[2][4];
  bf16x8_t kraw[4], vraw[4];
  // list entry of token slot tid (tid < TQ) and of this lane's two query rows
  // (t: a copy of the thread index).  Clamped loads, no branch; whether an
  // entry exists (slot < ntok) is decided where it is used, so nothing here
  // waits for the loads.
  auto load_entries = [&](const Tile& m, int t, int& et, int (&eq)[2]) {
    const int* lst = a.csr + m.c0;
    et = lst[min(t, m.ntok - 1)];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
      eq[nt] = lst[min((32 * (t / kWave) + 16 * nt + (t & 15)) / G, m.ntok - 1)];
  };
  // Every row of the (page, head) run is loaded (a missing page reads page
  // 0, rows past the sequence end hold stale bytes) and cleared afterwards
  // by a select, so the loads carry no branch.  Buffer loads: the run's base
  // in a descriptor, one loop-invariant lane offset and a scalar offset per
  // load, so the addressing costs no VGPR pairs.
  constexpr int kEb = sizeof(typename RawOf<KT>::elem);  // bytes per element
  const uint32_t k_lane = static_cast<uint32_t>(kr * 128 + dc) * kEb;
  const uint32_t v_lane = static_cast<uint32_t>(4 * kr * 128 + dc) * kEb;
  auto load_block = [&](const Tile& m) {
    const int64_t h0 = m.head0 + kv_off;
    if constexpr (__is_same(KT, FP4)) {
      // an MX-fp4 run per (page, head): per key row 64 code bytes, and its
      // four scale bytes after all codes; 8 dims = 4 code bytes + 1 scale
      const int64_t rb = (h0 >> 14) * kFp4Run;
      const auto ks = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<char*>(reinterpret_cast<const char*>(a.k_pool)) + rb, 0, kFp4Run, 0x00020000);
      const auto vs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<char*>(reinterpret_cast<const char*>(a.v_pool)) + rb, 0, kFp4Run, 0x00020000);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t w = __builtin_amdgcn_raw_buffer_load_b32(ks, kr * 64 + dc / 2, 32 * i * 64, 0);
        const uint32_t e = __builtin_amdgcn_raw_buffer_load_b8(ks, kFp4Codes + kr * 4 + dc / 32,
                                                               32 * i * 4, 0);
        kraw[i] = fp4x8_to_bf16x8(w, e8m0_to_f32(e));
      }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const uint32_t w = __builtin_amdgcn_raw_buffer_load_b32(vs, 4 * kr * 64 + dc / 2, kk * 64, 0);
        const uint32_t e = __builtin_amdgcn_raw_buffer_load_b8(vs, kFp4Codes + 4 * kr * 4 + dc / 32,
                                                               kk * 4, 0);
        vraw[kk] = fp4x8_to_bf16x8(w, e8m0_to_f32(e));
      }
    } else if constexpr (__is_same(KT, FP6)) {
      // an MX-fp6 run per (page, head): per key row 96 code bytes, and its
      // four scale bytes after all codes
      const int64_t rb = (h0 >> 14) * kFp6Run;
      const auto ks = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<char*>(reinterpret_cast<const char*>(a.k_pool)) + rb, 0, kFp6Run, 0x00020000);
      const auto vs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<char*>(reinterpret_cast<const char*>(a.v_pool)) + rb, 0, kFp6Run, 0x00020000);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        kraw[i] = fp6x8_load(ks, kr * 96, dc, 32 * i * 96, kFp6Codes + (32 * i + kr) * 4 + dc / 32);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        vraw[kk] = fp6x8_load(vs, (4 * kr + kk) * 96, dc, 0, kFp6Codes + (4 * kr + kk) * 4 + dc / 32);
    } else {
      const auto kr_src = run_rsrc(a.k_pool, h0 * kEb);
      const auto vr_src = run_rsrc(a.v_pool, h0 * kEb);
#pragma unroll
      for (int i = 0; i < 4; ++i) kraw[i] = load8_buf(ktag, kr_src, k_lane, 32 * i * 128 * kEb);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) vraw[kk] = load8_buf(ktag, vr_src, v_lane, kk * 128 * kEb);
    }
  };
  // V rows at or past the sequence end (stale bytes, possibly NaN) are
  // cleared: their probabilities are 0, but 0 * NaN would reach the MFMA
  // sums.  Stale K rows need nothing: their scores are replaced by -inf (a
  // block with such rows always takes the masked softmax path).
  auto clear_stale = [&](const Tile& m, int krow) {
    if (m.nvalid < kBlock) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) mask_bf16x8(vraw[kk], 4 * krow + kk < m.nvalid);
    }
  };
  // (rows past the tile's last token gather the clamped entry's real, finite
  // query row; their position -1 masks every key, so they produce zeros,
  // stored into the sink)
  auto q_rows = [&](const Tile& m, const int (&eq)[2], int64_t (&qo)[2]) {
    const int gg = m.g0 + kv;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
      qo[nt] = (static_cast<int64_t>(eq[nt] >> 8) * hq_stride + gg * G + qhh[nt]) * 128 + 8 * q4;
  };
  auto load_q = [&](const int64_t (&qo)[2]) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) qf[nt][ks] = load8_cached(qtag, a.q, qo[nt] + 32 * ks);
  };

  // Writes tile m (block in kraw/vraw, entry et of token slot tid) to stage
  // buffer B.  The LDS addresses come from a fresh copy of the thread index
  // each time rather than being kept live across the loop.
  auto stage = [&](PfStage& B, const Tile& m, int et) {
    int tl = tid;
    asm volatile("" : "+v"(tl));
    const int krl = tl >> 4;
    const int dcl = (tl & 15) * 8;
    clear_stale(m, krl);
    if (tl < TQ) {
      const bool ok = tl < m.ntok;
      B.tok[tl] = ok ? et >> 8 : -1;
      B.slot[tl] = ok ? et & 255 : 0;
      B.pos[tl] = ok ? m.p0 + (et >> 8) : -1;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<bf16x8_t*>(&B.k[(32 * i + krl) * kStrideK + dcl]) = kraw[i];
    uint16_t v[4][8];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) __builtin_memcpy(&v[kk][0], &vraw[kk], 16);
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const uint32_t w0 = static_cast<uint32_t>(v[0][d]) | (static_cast<uint32_t>(v[1][d]) << 16);
      const uint32_t w1 = static_cast<uint32_t>(v[2][d]) | (static_cast<uint32_t>(v[3][d]) << 16);
      const u32x2_t pr = {w0, w1};
      *reinterpret_cast<u32x2_t*>(&B.vt[vt_row_of_dim(dcl + d) * kStrideV + 4 * krl]) = pr;
    }
  };

  // Pipeline state: tiles i (m0, staged), i+1 (m1: block in flight), i+2
  // (m2).  One register set each for the block, the list entries and the
  // query rows, each reloaded right after its last use, so nothing loaded is
  // copied between registers at the loop edge.  Every load is issued
  // unconditionally (past the last tile, the clamped record re-reads tile i)
  // and every iteration issues the same memory operations in the same order;
  // the prologue issues the same sequence, ending with stores into the sink,
  // so the waits the compiler derives at the loop head hold on both edges and
  // never drain the previous tile's partial stores.
  // (read through the constant address space: the records are not written by
  // this kernel, and scalar loads keep them off the vector memory counter,
  // whose in-order waits would otherwise drain the previous tile's stores)
  const ConstTile* tiles = (const ConstTile*)(reinterpret_cast<uintptr_t>(a.items));
  Tile m0 = read_tile(tiles + item);
  bool has1 = item + stride < hi;
  bool has2 = item + 2 * stride < hi;
  Tile m1 = read_tile(tiles + (has1 ? item + stride : item));
  Tile m2 = read_tile(tiles + (has2 ? item + 2 * stride : item));
  int e_tok, e_q[2];
  int64_t q_off[2];
  load_entries(m0, tid, e_tok, e_q);
  load_block(m0);
  stage(S.st[0], m0, e_tok);
  q_rows(m0, e_q, q_off);
  load_entries(m1, tid, e_tok, e_q);
  load_block(m1);
  load_q(q_off);
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    uint16_t* po = a.sink_o + qhh[nt] * 128 + 8 * q4;
#pragma unroll
    for (int k = 0; k < 4; ++k) *reinterpret_cast<u32x4_t*>(po + 32 * k) = u32x4_t{0u, 0u, 0u, 0u};
    a.sink_lse[qhh[nt]] = 0.f;
  }
  __syncthreads();
  int buf = 0;

  while (true) {
    // ---- tile i+1 into the other stage (its block and entries are in
    // registers); then the record of tile i+3, the entries and the block of
    // tile i+2 go out
    if (has1) stage(S.st[buf ^ 1], m1, e_tok);
    q_rows(m1, e_q, q_off);
    const bool has3 = item + 3 * stride < hi;
    const Tile m3 = read_tile(tiles + (has3 ? item + 3 * stride : item));
    load_entries(m2, tid, e_tok, e_q);
    load_block(m2);
    const PfStage& B = S.st[buf];

    int tl = tid;
    asm volatile("" : "+v"(tl));
    // token slots of this lane's rows, from the fresh thread index
    int qtl[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) qtl[nt] = (32 * (tl / kWave) + 16 * nt + (tl & 15)) / G;
    int rpos[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) rpos[nt] = B.pos[qtl[nt]];

    // ---- the whole block at once: S^T for its 128 keys, one softmax, O^T.
    // S^T tiles: keys 16 mt + 4 q4 + r (rows), query rows 16 nt + l16.
    // O^T = V^T P^T: dims (permuted, see vt_row_of_dim) rows 16 dt + 4 q4 +
    // r, query rows 16 nt + l16; k-slots e of the 32-key step kk: keys
    // 32 kk + 4 q4 + e (e < 4) and 32 kk + 16 + 4 q4 + (e - 4), the keys the
    // S^T tiles 2 kk, 2 kk + 1 hold.  One maximum over the block means the
    // output accumulator is never rescaled.
    const int tok0 = m0.j * kBlock;
    float mrow[2], lrow[2];
    f32x4_t st[8][2];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      st[mt][0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      st[mt][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8_t kf = lds_b128(&B.k[(16 * mt + l16) * kStrideK + 32 * ks + 8 * q4]);
        st[mt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[0][ks], st[mt][0], 0, 0, 0);
        st[mt][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[1][ks], st[mt][1], 0, 0, 0);
      }
    }
    // the query rows of tile i+1, now that S^T no longer needs qf
    load_q(q_off);

    // Softmax in base 2: p = 2^(s c - m), c = scale * log2(e) > 0, so the row
    // max of the raw scores gives m.  Masking (keys past the sequence end or
    // after the row's position) only where the block is not entirely visible
    // to every row of the wave.
    const bool full = kBlock - 1 < m0.nvalid && tok0 + kBlock - 1 <= min(rpos[0], rpos[1]);
    if (__builtin_amdgcn_ballot_w64(!full) != 0) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = 16 * mt + 4 * q4 + r;
            const bool ok = key < m0.nvalid && tok0 + key <= rpos[nt];
            st[mt][nt][r] = ok ? st[mt][nt][r] : -INFINITY;
          }
    }
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      float mr = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) mr = max_nan(mr, st[mt][nt][r]);
      const float mn = rows_max(mr) * a.qk_scale_log2;
      // a row with nothing visible keeps m = -inf; its p are 2^-inf = 0
      const float mu = mn == -INFINITY ? 0.f : mn;
      float l = 0.f;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float e = exp2_raw(fmaf(st[mt][nt][r], a.qk_scale_log2, -mu));
          st[mt][nt][r] = e;
          l += e;
        }
      mrow[nt] = mn;
      lrow[nt] = rows_sum(l);
    }
    f32x4_t o[8][2];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      // P as bf16 B operands
      bf16x8_t pb[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const uint32_t u[4] = {pack2_rne(st[2 * kk][nt][0], st[2 * kk][nt][1]),
                               pack2_rne(st[2 * kk][nt][2], st[2 * kk][nt][3]),
                               pack2_rne(st[2 * kk + 1][nt][0], st[2 * kk + 1][nt][1]),
                               pack2_rne(st[2 * kk + 1][nt][2], st[2 * kk + 1][nt][3])};
        __builtin_memcpy(&pb[nt], u, 16);
      }
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const uint16_t* row = &B.vt[(16 * dt + l16) * kStrideV + 32 * kk + 4 * q4];
        const u32x2_t lo = lds_b64(row), hi2 = lds_b64(row + 16);
        const u32x4_t cat = {lo[0], lo[1], hi2[0], hi2[1]};
        bf16x8_t vf;
        __builtin_memcpy(&vf, &cat, 16);
        const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
        o[dt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb[0], kk == 0 ? z : o[dt][0], 0, 0, 0);
        o[dt][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb[1], kk == 0 ? z : o[dt][1], 0, 0, 0);
      }
    }

    // ---- normalised partial and its log-sum-exp (natural log of the scaled logits)
    // Every row stores (rows past the tile's last token into the sink), so
    // the number of memory operations per iteration is fixed and later waits
    // on the prefetches never have to drain these stores.
    const int g = m0.g0 + kv;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int t = B.tok[qtl[nt]];
      const float l = lrow[nt];
      const float inv = l > 0.f ? a.v_scale * __builtin_amdgcn_rcpf(l) : 0.f;
      const int64_t base =
          ((static_cast<int64_t>(max(t, 0)) * a.hkv + g) * a.kmax + B.slot[qtl[nt]]) * G + qhh[nt];
      uint16_t* po = (t >= 0 ? a.part_o + base * 128 : a.sink_o + qhh[nt] * 128) + 8 * q4;
      float* pl = t >= 0 ? a.part_lse + base : a.sink_lse + qhh[nt];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const u32x4_t v = {pack2_rne(o[2 * k][nt][0] * inv, o[2 * k][nt][1] * inv),
                           pack2_rne(o[2 * k][nt][2] * inv, o[2 * k][nt][3] * inv),
                           pack2_rne(o[2 * k + 1][nt][0] * inv, o[2 * k + 1][nt][1] * inv),
                           pack2_rne(o[2 * k + 1][nt][2] * inv, o[2 * k + 1][nt][3] * inv)};
        *reinterpret_cast<u32x4_t*>(po + 32 * k) = v;
      }
      // (the four lanes of the row store the same value)
      *pl = l > 0.f ? (mrow[nt] + __builtin_amdgcn_logf(l)) * kLn2f : -INFINITY;
    }
    if (!has1) break;
    // tile i+1 is staged and every wave is done with tile i's stage
    __syncthreads();
    buf ^= 1;
    item += stride;
    m0 = m1;
    m1 = m2;
    m2 = m3;
    has1 = has2;
    has2 = has3;
  }
}

// ---------------------------------------------------------- forced blocks

// Workgroup (group grp of TQ = 128 / G consecutive tokens of sequence b, kv
// head g; four waves): the 128 query rows (token x G heads, row r = 32 w +
// 16 nt + l16 is token slot r / G, head r % G) keep their query rows in
// registers and run the union of their tokens' forced blocks: [0, init') and
// the local windows [nb_t - local, nb_t), which for consecutive tokens form
// one range.  Per block: K and V^T staged in LDS as in the tiles, S^T on the
// matrix cores, each row masking the keys after its position and the blocks
// outside its own forced set, an online softmax (base 2), O^T += V^T P^T.
// The normalised partial and its lse go to the token's first forced slot.
// Two workgroups share a CU, so one's block loads run under the other's
// matrix work; the grid holds two per CU over the kv heads, each walking
// units (sequence, token group) from the offsets the list scan computes.
constexpr int kFwWaves = 4;
constexpr int kFwThreads = kFwWaves * kWave;
constexpr int kFwRows = kForcedRows;
static_assert(kFwRows == 32 * kFwWaves, "each wave owns 32 query rows");

// One unit of the forced-block kernel: token group grp of sequence b, kv
// head blockIdx.y.
template <class KT, int G>
__device__ void forced_unit(const PrefillAttnArgs& a, int b, int grp, PfStage& S) {
  constexpr int TQ = kFwRows / G;
  const KT* ktag = nullptr;
  const BF16* qtag = nullptr;
  const int g = blockIdx.y;
  const int h = g / (a.hkv / a.hidx);
  const int cu0 = a.cu_seqlens_q[b];
  const int n_b = a.cu_seqlens_q[b + 1] - cu0;
  const int i0 = grp * TQ;
  if (i0 >= n_b) return;
  const int L = a.seq_lens[b];
  const int prefix = L - n_b;
  const int ilast = min(n_b, i0 + TQ) - 1;
  const ForcedRange f0 = forced_range(a, prefix + i0);
  const ForcedRange f1 = forced_range(a, prefix + ilast);
  // the union: blocks [0, f1.init_end), then [max(f1.init_end, f0.lo), f1.nb)
  // (f1.nb - 1 is the last token's own block, forced whenever local > 0)
  const int e_init = f1.init_end;
  const int lo2 = max(e_init, f0.lo);
  const int hi2 = a.local > 0 ? f1.nb : lo2;
  const int nblk = e_init + max(0, hi2 - lo2);
  if (nblk == 0) return;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int w = tid / kWave;
  const int l16 = lane & 15;
  const int q4 = lane >> 4;
  const int kr = tid >> 4;           // staging: K keys 16 i + kr, V keys 8 kr .. + 8
  const int dc = (tid & 15) * 8;     // staging dims dc .. dc + 8

  // this lane's two query rows, their positions and their tokens'
  // selection sizes (all loads of the unit's start in flight together with
  // the first block's); the rest is recomputed from them where needed
  int pos[2], cntv[2];
  bf16x8_t qf[2][4];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int r = 32 * w + 16 * nt + l16;
    const int i = i0 + r / G;
    pos[nt] = i <= ilast ? prefix + i : -1;  // -1 masks every key
    const int t = cu0 + min(i, ilast);
    cntv[nt] = a.cnt[static_cast<int64_t>(t) * a.hidx + h];
    const int64_t qo = (static_cast<int64_t>(t) * a.hkv * G + g * G + r % G) * 128 + 8 * q4;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[nt][ks] = load8_cached(qtag, a.q, qo + 32 * ks);
  }

  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
  f32x4_t o[8][2];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt][0] = o[dt][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto block_of = [&](int u) { return u < e_init ? u : lo2 + (u - e_init); };
  const int32_t* bt_row = a.block_table + static_cast<int64_t>(b) * a.max_blocks;
  int page_next = bt_row[block_of(0)];
  for (int u = 0; u < nblk; ++u) {
    const int j = block_of(u);
    // ---- stage block j: K rows as they are, V^T in the tiles' permuted dim
    // order; a missing page reads page 0 with every key masked (nvalid = 0),
    // V rows at or past the sequence end cleared (0 * NaN would reach the sums)
    const int page = page_next;
    if (u + 1 < nblk) page_next = bt_row[block_of(u + 1)];
    const bool page_ok = page >= 0 && page < a.num_pages;
    const int nvalid = page_ok ? max(0, min(kBlock, L - j * kBlock)) : 0;
    const int64_t h0 = (static_cast<int64_t>(page_ok ? page : 0) * a.hkv + g) * kBlock * 128;
    // K rows 16 i + kr and V rows 8 kr + i of the thread: all eight of each in
    // one pass, or for the MX formats in two passes of four, which keeps the
    // conversions' registers to one half
    constexpr int RP = (__is_same(KT, FP4) || __is_same(KT, FP6)) ? 4 : 8;  // rows per pass
#pragma unroll
    for (int hh = 0; hh < 8 / RP; ++hh) {
      bf16x8_t kraw[RP], vraw[RP];
      if constexpr (__is_same(KT, FP4)) {
        const int64_t rb = (h0 >> 14) * kFp4Run;
        const auto ks = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<char*>(reinterpret_cast<const char*>(a.k_pool)) + rb, 0, kFp4Run, 0x00020000);
        const auto vs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<char*>(reinterpret_cast<const char*>(a.v_pool)) + rb, 0, kFp4Run, 0x00020000);
#pragma unroll
        for (int i = 0; i < RP; ++i) {
          const int kro = 16 * (RP * hh + i) + kr, vro = 8 * kr + RP * hh + i;
          const uint32_t kw = __builtin_amdgcn_raw_buffer_load_b32(ks, kro * 64 + dc / 2, 0, 0);
          const uint32_t ke = __builtin_amdgcn_raw_buffer_load_b8(ks, kFp4Codes + kro * 4 + dc / 32, 0, 0);
          const uint32_t vw = __builtin_amdgcn_raw_buffer_load_b32(vs, vro * 64 + dc / 2, 0, 0);
          const uint32_t ve = __builtin_amdgcn_raw_buffer_load_b8(vs, kFp4Codes + vro * 4 + dc / 32, 0, 0);
          kraw[i] = fp4x8_to_bf16x8(kw, e8m0_to_f32(ke));
          vraw[i] = fp4x8_to_bf16x8(vw, e8m0_to_f32(ve));
        }
      } else if constexpr (__is_same(KT, FP6)) {
        const int64_t rb = (h0 >> 14) * kFp6Run;
        const auto ks = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<char*>(reinterpret_cast<const char*>(a.k_pool)) + rb, 0, kFp6Run, 0x00020000);
        const auto vs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<char*>(reinterpret_cast<const char*>(a.v_pool)) + rb, 0, kFp6Run, 0x00020000);
#pragma unroll
        for (int i = 0; i < RP; ++i) {
          const int kro = 16 * (RP * hh + i) + kr, vro = 8 * kr + RP * hh + i;
          kraw[i] = fp6x8_load(ks, kro * 96, dc, 0, kFp6Codes + kro * 4 + dc / 32);
          vraw[i] = fp6x8_load(vs, vro * 96, dc, 0, kFp6Codes + vro * 4 + dc / 32);
        }
      } else {
        constexpr int kEb = sizeof(typename RawOf<KT>::elem);
        const auto kr_src = run_rsrc(a.k_pool, h0 * kEb);
        const auto vr_src = run_rsrc(a.v_pool, h0 * kEb);
        const uint32_t k_lane = static_cast<uint32_t>(kr * 128 + dc) * kEb;
        const uint32_t v_lane = static_cast<uint32_t>(8 * kr * 128 + dc) * kEb;
#pragma unroll
        for (int i = 0; i < RP; ++i)
          kraw[i] = load8_buf(ktag, kr_src, k_lane, 16 * (RP * hh + i) * 128 * kEb);
#pragma unroll
        for (int i = 0; i < RP; ++i) vraw[i] = load8_buf(ktag, vr_src, v_lane, (RP * hh + i) * 128 * kEb);
      }
      if (nvalid < kBlock) {
#pragma unroll
        for (int i = 0; i < RP; ++i) mask_bf16x8(vraw[i], 8 * kr + RP * hh + i < nvalid);
      }
#pragma unroll
      for (int i = 0; i < RP; ++i)
        *reinterpret_cast<bf16x8_t*>(&S.k[(16 * (RP * hh + i) + kr) * kStrideK + dc]) = kraw[i];
      uint16_t v[RP][8];
#pragma unroll
      for (int i = 0; i < RP; ++i) __builtin_memcpy(&v[i][0], &vraw[i], 16);
#pragma unroll
      for (int d = 0; d < 8; ++d) {
#pragma unroll
        for (int q = 0; q < RP / 4; ++q) {
          const uint32_t w0 = static_cast<uint32_t>(v[4 * q][d]) | (static_cast<uint32_t>(v[4 * q + 1][d]) << 16);
          const uint32_t w1 = static_cast<uint32_t>(v[4 * q + 2][d]) | (static_cast<uint32_t>(v[4 * q + 3][d]) << 16);
          *reinterpret_cast<u32x2_t*>(&S.vt[vt_row_of_dim(dc + d) * kStrideV + 8 * kr + RP * hh + 4 * q]) =
              u32x2_t{w0, w1};
        }
      }
    }
    __syncthreads();

    // The whole block at once: S^T for its 128 keys, one online-softmax step.
    // S^T tiles: keys 16 mt + 4 q4 + r, query rows 16 nt + l16.
    const int tok0 = j * kBlock;
    f32x4_t st[8][2];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      st[mt][0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      st[mt][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8_t kf = lds_b128(&S.k[(16 * mt + l16) * kStrideK + 32 * ks + 8 * q4]);
        st[mt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[0][ks], st[mt][0], 0, 0, 0);
        st[mt][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[1][ks], st[mt][1], 0, 0, 0);
      }
    }
    // Masking (keys past the sequence end or after the row's position, or a
    // block outside the row's forced set) only where the block is not
    // entirely visible to every row of the wave.
    bool in[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) in[nt] = forced_range(a, pos[nt]).has(j);
    const bool full = in[0] && in[1] && nvalid == kBlock && tok0 + kBlock - 1 <= min(pos[0], pos[1]);
    if (__builtin_amdgcn_ballot_w64(!full) != 0) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = 16 * mt + 4 * q4 + r;
            const bool ok = in[nt] && key < nvalid && tok0 + key <= pos[nt];
            st[mt][nt][r] = ok ? st[mt][nt][r] : -INFINITY;
          }
    }
    float alpha[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      float mr = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) mr = max_nan(mr, st[mt][nt][r]);
      const float mn = max_nan(m_run[nt], rows_max(mr) * a.qk_scale_log2);
      // a row with nothing visible so far keeps m = -inf; its p are 2^-inf = 0
      const float mu = mn == -INFINITY ? 0.f : mn;
      alpha[nt] = exp2_raw(m_run[nt] - mu);
      float ls = 0.f;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float e = exp2_raw(fmaf(st[mt][nt][r], a.qk_scale_log2, -mu));
          st[mt][nt][r] = e;
          ls += e;
        }
      l_run[nt] = l_run[nt] * alpha[nt] + rows_sum(ls);
      m_run[nt] = mn;
    }
    // the output is rescaled only where some row's maximum moved
    if (__builtin_amdgcn_ballot_w64(alpha[0] != 1.f || alpha[1] != 1.f) != 0) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        o[dt][0] *= alpha[0];
        o[dt][1] *= alpha[1];
      }
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      // 32-key step: keys 32 kk + 4 q4 + e (e < 4) and + 16 (e >= 4)
      bf16x8_t pb[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const uint32_t pu[4] = {pack2_rne(st[2 * kk][nt][0], st[2 * kk][nt][1]),
                                pack2_rne(st[2 * kk][nt][2], st[2 * kk][nt][3]),
                                pack2_rne(st[2 * kk + 1][nt][0], st[2 * kk + 1][nt][1]),
                                pack2_rne(st[2 * kk + 1][nt][2], st[2 * kk + 1][nt][3])};
        __builtin_memcpy(&pb[nt], pu, 16);
      }
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const uint16_t* row = &S.vt[(16 * dt + l16) * kStrideV + 32 * kk + 4 * q4];
        const u32x2_t lo = lds_b64(row), hi2 = lds_b64(row + 16);
        const u32x4_t cat = {lo[0], lo[1], hi2[0], hi2[1]};
        bf16x8_t vf;
        __builtin_memcpy(&vf, &cat, 16);
        o[dt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb[0], o[dt][0], 0, 0, 0);
        o[dt][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb[1], o[dt][1], 0, 0, 0);
      }
    }
    // every wave is done with the stage before the next block is written
    __syncthreads();
  }

  // the normalised partial and its lse, in the token's first forced slot
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    if (pos[nt] < 0) continue;
    const int r = 32 * (threadIdx.x / kWave) + 16 * nt + (threadIdx.x & 15);
    const int t = cu0 + i0 + r / G;
    const int cnt = min(max(cntv[nt], 0), a.kmax);
    // (a selection always holds its forced blocks: cnt >= their count)
    const int slot = min(max(forced_range(a, pos[nt]).first_slot(cnt), 0), a.kmax - 1);
    const float l = l_run[nt];
    const float inv = l > 0.f ? a.v_scale * __builtin_amdgcn_rcpf(l) : 0.f;
    const int64_t base = ((static_cast<int64_t>(t) * a.hkv + g) * a.kmax + slot) * G + r % G;
    uint16_t* po = a.part_o + base * 128 + 8 * q4;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const u32x4_t v = {pack2_rne(o[2 * k][nt][0] * inv, o[2 * k][nt][1] * inv),
                         pack2_rne(o[2 * k][nt][2] * inv, o[2 * k][nt][3] * inv),
                         pack2_rne(o[2 * k + 1][nt][0] * inv, o[2 * k + 1][nt][1] * inv),
                         pack2_rne(o[2 * k + 1][nt][2] * inv, o[2 * k + 1][nt][3] * inv)};
      *reinterpret_cast<u32x4_t*>(po + 32 * k) = v;
    }
    if (q4 == 0)
      a.part_lse[base] = l > 0.f ? (m_run[nt] + __builtin_amdgcn_logf(l)) * kLn2f : -INFINITY;
  }
}


template <class KT, int G>
__global__ __launch_bounds__(kFwThreads, 2) void prefill_forced_kernel(PrefillAttnArgs a) {
  __shared__ PfStage S;
  // the workgroups of one XCD (x, x + 8, ...) walk a contiguous range of
  // units, so a sequence's init blocks and the local blocks its neighbouring
  // groups share are fetched into one L2
  const int total = a.forced_off[a.num_seqs];
  const int per = (total + 7) / 8;
  const int hi = min((static_cast<int>(blockIdx.x) % 8 + 1) * per, total);
  for (int unit = (blockIdx.x % 8) * per + blockIdx.x / 8; unit < hi; unit += gridDim.x / 8) {
    int lo = 0, up = a.num_seqs;  // forced_off[lo] <= unit < forced_off[up]
    while (up - lo > 1) {
      const int mid = (lo + up) / 2;
      if (a.forced_off[mid] <= unit) lo = mid; else up = mid;
    }
    forced_unit<KT, G>(a, lo, unit - a.forced_off[lo], S);
  }
}

// ---------------------------------------------------------------- combine

// out = sum_s exp(lse_s - lse) o_s per (token, kv head), lse = log sum_s
// exp(lse_s).  A thread owns 8 dims of one q head (16 threads per head row,
// 16 head rows per workgroup, so 16 / G (token, kv head) units per
// workgroup) and walks the slots in batches of 8 with an online max: each
// batch is one round trip of 8 partial loads (16 bytes each, non-temporal:
// the partials are read once) and 8 lse loads, with no LDS and no barrier.
template <int G>
__global__ __launch_bounds__(kWgThreads) void prefill_combine_kernel(PrefillAttnArgs a) {
  constexpr int kUnits = 16 / G;  // (token, kv head) units per workgroup
  const int tid = threadIdx.x;
  const int unit = blockIdx.x * kUnits + tid / (16 * G);
  if (unit >= a.num_tokens * a.hkv) return;
  const int t = unit / a.hkv;
  const int g = unit - t * a.hkv;
  const int hh = (tid / 16) % G;
  const int d0 = (tid % 16) * 8;
  const int h = g / (a.hkv / a.hidx);
  const int cnt = min(max(a.cnt[t * a.hidx + h], 0), a.kmax);
  // With the forced blocks split off, the token's forced slots hold one
  // partial, in the first of them (slot 0, or the first local slot when
  // init' = 0): the slots read are that one and the top-k slots
  // [init', cnt - local'), n = cnt - forced + 1 of them.
  int n = cnt, skip_from = 1, skip = 0;
  if (a.forced_split) {
    int lo = 0, hi = a.num_seqs;  // cu[lo] <= t < cu[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) / 2;
      if (a.cu_seqlens_q[mid] <= t) lo = mid; else hi = mid;
    }
    const int p = a.seq_lens[lo] - (a.cu_seqlens_q[lo + 1] - a.cu_seqlens_q[lo]) +
                  (t - a.cu_seqlens_q[lo]);
    const ForcedRange fr = forced_range(a, p);
    const int nf = fr.count();
    if (nf > 0 && cnt >= nf) {
      n = cnt - nf + 1;
      skip = fr.init_end > 0 ? fr.init_end - 1 : 0;  // read u >= 1 at slot u + skip
    }
  }
  const int64_t row0 = (static_cast<int64_t>(t) * a.hkv + g) * a.kmax * G + hh;  // slot 0
  const float* lse_p = a.part_lse + row0;
  const uint16_t* po = a.part_o + row0 * 128 + d0;
  float m = -INFINITY, wsum = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < n; s0 += 8) {
    // straight-line batch: slots past the last re-read it and get weight 0
    float ls[8];
    u32x4_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int uc = min(s0 + u, n - 1);
      const int64_t s = uc >= skip_from ? uc + skip : uc;
      ls[u] = lse_p[s * G];
      v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(po + s * G * 128));
    }
    float mb = m;
#pragma unroll
    for (int u = 0; u < 8; ++u) mb = fmaxf(mb, s0 + u < n ? ls[u] : -INFINITY);
    if (mb == -INFINITY) continue;  // nothing visible in any slot so far
    const float sc = __expf(m - mb);  // 0 while m is still -inf
    wsum *= sc;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= sc;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float wv = s0 + u < n ? __expf(ls[u] - mb) : 0.f;
      wsum += wv;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] = fmaf(wv, __uint_as_float(v[u][q] << 16), acc[2 * q]);
        acc[2 * q + 1] = fmaf(wv, __uint_as_float(v[u][q] & 0xffff0000u), acc[2 * q + 1]);
      }
    }
    m = mb;
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  const int64_t out0 = (static_cast<int64_t>(t) * a.hkv + g) * G + hh;  // q head row
  const u32x4_t r = {pack2_rne(acc[0] * inv, acc[1] * inv), pack2_rne(acc[2] * inv, acc[3] * inv),
                     pack2_rne(acc[4] * inv, acc[5] * inv), pack2_rne(acc[6] * inv, acc[7] * inv)};
  *reinterpret_cast<u32x4_t*>(reinterpret_cast<uint16_t*>(a.out) + out0 * 128 + d0) = r;
  if (d0 == 0 && a.lse_out != nullptr) a.lse_out[out0] = wsum > 0.f ? m + __logf(wsum) : -INFINITY;
}

// -------------------------------------------------------------- launchers

hipError_t launch_prefill_k2q(const PrefillAttnArgs& a, hipStream_t s) {
  if (a.num_tokens == 0 || a.num_seqs == 0) return hipSuccess;
  // chunks of 256 tokens of the longest possible sequence (all T tokens)
  const dim3 grid((a.num_tokens + kWgThreads - 1) / kWgThreads, a.num_seqs, a.hidx);
  const size_t lds = sizeof(int) * static_cast<size_t>(a.max_blocks);
  const int n = a.num_seqs * a.hidx * a.max_blocks;
  k2q_count_kernel<<<grid, kWgThreads, lds, s>>>(a);
  k2q_scan_kernel<<<1, 1024, 0, s>>>(a, n);
  k2q_fill_kernel<<<grid, kWgThreads, lds, s>>>(a);
  return hipGetLastError();
}

// Resident workgroups: one per CU, a multiple of 8 (one set per XCD).
constexpr int kPrefillAttendGrid = 256;

template <class KT>
static bool launch_pf_attend_g(const PrefillAttnArgs& a, int group, hipStream_t s) {
  const dim3 grid(kPrefillAttendGrid, a.hkv / a.hidx);
  switch (group) {
    case 1: prefill_attend_kernel<KT, 1><<<grid, kPfThreads, 0, s>>>(a); return true;
    case 2: prefill_attend_kernel<KT, 2><<<grid, kPfThreads, 0, s>>>(a); return true;
    case 4: prefill_attend_kernel<KT, 4><<<grid, kPfThreads, 0, s>>>(a); return true;
    case 8: prefill_attend_kernel<KT, 8><<<grid, kPfThreads, 0, s>>>(a); return true;
    case 16: prefill_attend_kernel<KT, 16><<<grid, kPfThreads, 0, s>>>(a); return true;
    default: return false;
  }
}

// Two resident four-wave workgroups per CU over all kv heads.
constexpr int kForcedWorkgroups = 512;

template <class KT>
static bool launch_pf_forced_g(const PrefillAttnArgs& a, int group, hipStream_t s) {
  // (a multiple of 8: one set per XCD)
  const dim3 grid(static_cast<unsigned>(max(8, kForcedWorkgroups / a.hkv / 8 * 8)), a.hkv);
  switch (group) {
    case 1: prefill_forced_kernel<KT, 1><<<grid, kFwThreads, 0, s>>>(a); return true;
    case 2: prefill_forced_kernel<KT, 2><<<grid, kFwThreads, 0, s>>>(a); return true;
    case 4: prefill_forced_kernel<KT, 4><<<grid, kFwThreads, 0, s>>>(a); return true;
    case 8: prefill_forced_kernel<KT, 8><<<grid, kFwThreads, 0, s>>>(a); return true;
    case 16: prefill_forced_kernel<KT, 16><<<grid, kFwThreads, 0, s>>>(a); return true;
    default: return false;
  }
}

hipError_t launch_prefill_attend(const PrefillAttnArgs& a, int kv_dtype, int group,
                                 hipStream_t s) {
  if (a.num_tokens == 0) return hipSuccess;
  bool ok = false;
  if (a.max_items > 0) {
    if (kv_dtype == 0) ok = launch_pf_attend_g<BF16>(a, group, s);
    else if (kv_dtype == 2) ok = launch_pf_attend_g<FP8>(a, group, s);
    else if (kv_dtype == 3) ok = launch_pf_attend_g<BF8>(a, group, s);
    else if (kv_dtype == 4) ok = launch_pf_attend_g<FP4>(a, group, s);
    else if (kv_dtype == 5) ok = launch_pf_attend_g<FP6>(a, group, s);
    if (!ok) return hipErrorInvalidValue;
  }
  if (a.forced_split) {
    if (kv_dtype == 0) ok = launch_pf_forced_g<BF16>(a, group, s);
    else if (kv_dtype == 2) ok = launch_pf_forced_g<FP8>(a, group, s);
    else if (kv_dtype == 3) ok = launch_pf_forced_g<BF8>(a, group, s);
    else if (kv_dtype == 4) ok = launch_pf_forced_g<FP4>(a, group, s);
    else if (kv_dtype == 5) ok = launch_pf_forced_g<FP6>(a, group, s);
    else ok = false;
    if (!ok) return hipErrorInvalidValue;
  }
  // 16 / G (token, kv head) units per combine workgroup
  const int64_t units = static_cast<int64_t>(a.num_tokens) * a.hkv;
  auto cgrid = [&](int g) { return static_cast<unsigned>((units + 16 / g - 1) / (16 / g)); };
  switch (group) {
    case 1: prefill_combine_kernel<1><<<cgrid(1), kWgThreads, 0, s>>>(a); break;
    case 2: prefill_combine_kernel<2><<<cgrid(2), kWgThreads, 0, s>>>(a); break;
    case 4: prefill_combine_kernel<4><<<cgrid(4), kWgThreads, 0, s>>>(a); break;
    case 8: prefill_combine_kernel<8><<<cgrid(8), kWgThreads, 0, s>>>(a); break;
    case 16: prefill_combine_kernel<16><<<cgrid(16), kWgThreads, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace msa
