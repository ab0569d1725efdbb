// Decode block scoring (index-head scan) with the selection fused behind it,
// the standalone selection kernel, and small utility kernels.
//
// Scoring (sglang page minimax_sparse_backend.py: the index query
// idx_q, sparse_index_dim wide, is scored against the index-key cache of
// every block_size_k block; the score is the max over the block's tokens of
// q_idx . k_idx, tokens after the query excluded):
//
// One workgroup (4 waves) scores `pages_per_item` consecutive blocks of one
// (sequence, index head) pair; each wave streams whole 128-token pages.  A
// page of index keys is one contiguous run of 128 * Di elements (head-major
// pages), read with 16-byte loads: Di/8 lanes cover one token row, so a wave
// instruction reads 64/(Di/8) full rows.  Every lane keeps the 8 query
// elements of its column slice in registers, forms an 8-term partial dot
// product, the row is summed across its lanes with DPP, tokens past the query
// are masked by select (never by multiplying, so stale bytes cannot leak),
// and the wave reduces the block max.  The workgroup that finishes last for a
// pair (atomic ticket, agent-scope fences) runs the selection for that pair
// while other workgroups keep streaming.
#include "msa_device.h"
#include "msa_internal.h"
#include "msa_select.h"

namespace msa {

template <class IT, int DI, int MAXPER>
__global__ __launch_bounds__(kWgThreads) void decode_score_kernel(ScoreArgs a) {
  constexpr int LPR = DI / 8;          // lanes per token row
  constexpr int RPL = kWave / LPR;     // token rows per wave load
  constexpr int NLOAD = kBlock / RPL;  // loads per page per lane
  // up to 128 VGPRs of loads in flight per lane
  constexpr int BATCH = (__is_same(IT, F32) ? 16 : 32) < NLOAD ? (__is_same(IT, F32) ? 16 : 32)
                                                               : NLOAD;
  static_assert(NLOAD % BATCH == 0, "batch must divide the page");

  __shared__ SelectLds sl;
  __shared__ int is_last;

  const int pair = blockIdx.x / a.chunks_per_pair;
  const int chunk = blockIdx.x - pair * a.chunks_per_pair;
  const int b = pair / a.hidx;
  const int h = pair - b * a.hidx;
  const int L = a.seq_lens[b];
  // (a sequence longer than its table row is a caller error: clamp to the row)
  const int nb = L > 0 ? min((L - 1) / kBlock + 1, a.max_blocks) : 0;
  const int nchunks = div_up(nb, a.pages_per_item);
  float* srow = a.scores + static_cast<int64_t>(pair) * a.max_blocks;

  if (a.fill_tail && chunk == 0)
    for (int j = nb + threadIdx.x; j < a.max_blocks; j += kWgThreads) srow[j] = -INFINITY;
  if (nb == 0) {
    if (a.fuse_select && chunk == 0) {
      for (int i = threadIdx.x; i < a.kmax; i += kWgThreads) {
        a.sel[static_cast<int64_t>(pair) * a.kmax + i] = -1;
        if (a.sel_pages) a.sel_pages[static_cast<int64_t>(pair) * a.kmax + i] = -1;
      }
      if (threadIdx.x == 0) a.cnt[pair] = 0;
    }
    return;
  }
  if (chunk >= nchunks) return;

  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  const int row = lane / LPR;
  const int col = lane % LPR;
  const IT* tag = nullptr;

  float qv[8];
  load8(tag, a.idx_q, (static_cast<int64_t>(b) * a.hidx + h) * DI + col * 8, qv);

  const int p = L - 1;
  const int j0 = chunk * a.pages_per_item;
  const int j1 = min(nb, j0 + a.pages_per_item);
  for (int j = j0 + w; j < j1; j += kWgThreads / kWave) {
    const int page = a.block_table[static_cast<int64_t>(b) * a.max_blocks + j];
    float m = -INFINITY;
    if (page >= 0 && page < a.num_pages) {
      const int nvalid = min(kBlock, p + 1 - j * kBlock);
      const int64_t base =
          (static_cast<int64_t>(page) * a.hidx + h) * kBlock * DI + row * DI + col * 8;
#pragma unroll
      for (int i0 = 0; i0 < NLOAD; i0 += BATCH) {
        Raw8<IT> raw[BATCH];
#pragma unroll
        for (int i = 0; i < BATCH; ++i)
          raw[i] = load_raw(tag, a.idx_k, base + static_cast<int64_t>((i0 + i) * RPL) * DI);
#pragma unroll
        for (int i = 0; i < BATCH; ++i) {
          float x[8];
          unpack(raw[i], x);
          float d = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) d = fmaf(qv[e], x[e], d);
          d = group_sum<LPR>(d);
          const int t = (i0 + i) * RPL + row;
          m = fmaxf(m, t < nvalid ? d : -INFINITY);
        }
      }
      m = wave_max(m);
    }
    if (lane == 0) {
      if (a.fuse_select) store_shared_f32(srow + j, m); else srow[j] = m;
    }
  }

  if (!a.fuse_select) return;
  // The last chunk of the pair to finish selects over all of the pair's scores.
  if (!take_last_ticket(&a.tickets[pair], nchunks, &is_last)) return;
  select_row<MAXPER, true>(srow, nb, a.topk, a.init, a.local, a.kmax,
                           a.sel + static_cast<int64_t>(pair) * a.kmax, a.cnt + pair, sl,
                           a.block_table + static_cast<int64_t>(b) * a.max_blocks,
                           a.sel_pages ? a.sel_pages + static_cast<int64_t>(pair) * a.kmax
                                       : nullptr);
}

// One workgroup per (query token, index head) row.
template <int MAXPER>
__global__ __launch_bounds__(kWgThreads) void select_kernel(SelectArgs a) {
  __shared__ SelectLds sl;
  const int rowi = blockIdx.x;
  const int t = rowi / a.hidx;
  int b, p;
  if (a.cu_seqlens_q == nullptr) {
    b = t;
    p = a.seq_lens[b] - 1;
  } else {
    int lo = 0, hi = a.num_seqs;  // find b with cu[b] <= t < cu[b+1]
    while (hi - lo > 1) {
      const int mid = (lo + hi) / 2;
      if (a.cu_seqlens_q[mid] <= t) lo = mid; else hi = mid;
    }
    b = lo;
    const int n = a.cu_seqlens_q[b + 1] - a.cu_seqlens_q[b];
    p = a.seq_lens[b] - n + (t - a.cu_seqlens_q[b]);
  }
  const int nb = p >= 0 ? min(p / kBlock + 1, a.max_blocks) : 0;
  select_row<MAXPER>(a.scores + static_cast<int64_t>(rowi) * a.max_blocks, nb, a.topk,
                     a.init, a.local, a.kmax, a.sel + static_cast<int64_t>(rowi) * a.kmax,
                     a.cnt + rowi, sl);
}

__global__ void fill_u32_kernel(uint32_t* p, int64_t n, uint32_t value) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[i] = value;
}

__global__ void fp8_dequant_kernel(const uint8_t* in, float* out, int64_t n, float scale) {
  const int64_t i = (blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x) * 4;
  if (i >= n) return;
  uint32_t w = 0;
  for (int k = 0; k < 4 && i + k < n; ++k) w |= static_cast<uint32_t>(in[i + k]) << (8 * k);
  float x[4];
  fp8x4_to_f32(w, x);
  for (int k = 0; k < 4 && i + k < n; ++k) out[i + k] = x[k] * scale;
}

// ------------------------------------------------------------- launchers

hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t value, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  fill_u32_kernel<<<static_cast<int>(blocks < 1024 ? blocks : 1024), 256, 0, s>>>(p, n, value);
  return hipGetLastError();
}

template <class IT, int DI>
static void launch_score_t(const ScoreArgs& a, hipStream_t s) {
  const int grid = a.num_seqs * a.hidx * a.chunks_per_pair;
  if (a.max_blocks <= 1024)
    decode_score_kernel<IT, DI, 4><<<grid, kWgThreads, 0, s>>>(a);
  else
    decode_score_kernel<IT, DI, 32><<<grid, kWgThreads, 0, s>>>(a);
}

hipError_t launch_decode_score(const ScoreArgs& a, int idx_dtype, int idx_dim,
                               hipStream_t s) {
  if (a.num_seqs * a.hidx * a.chunks_per_pair == 0) return hipSuccess;
  const bool f32 = idx_dtype == 1;
  if (idx_dim == 128) {
    if (f32) launch_score_t<F32, 128>(a, s); else launch_score_t<BF16, 128>(a, s);
  } else {
    if (f32) launch_score_t<F32, 64>(a, s); else launch_score_t<BF16, 64>(a, s);
  }
  return hipGetLastError();
}

hipError_t launch_select(const SelectArgs& a, hipStream_t s) {
  const int grid = a.num_tokens * a.hidx;
  if (grid == 0) return hipSuccess;
  if (a.max_blocks <= 1024)
    select_kernel<4><<<grid, kWgThreads, 0, s>>>(a);
  else
    select_kernel<32><<<grid, kWgThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_fp8_dequant(const uint8_t* in, float* out, int64_t n, float scale,
                              hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t threads = (n + 3) / 4;
  fp8_dequant_kernel<<<static_cast<int>((threads + 255) / 256), 256, 0, s>>>(in, out, n, scale);
  return hipGetLastError();
}

}  // namespace msa
