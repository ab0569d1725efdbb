// Decode block scoring (index-head scan) of one chunk of pages.
//
// Scoring (sglang page minimax_sparse_backend.py: the index query idx_q,
// sparse_index_dim wide, is scored against the index-key cache of every
// block_size_k block; the score is the max over the block's tokens of
// q_idx . k_idx, tokens after the query excluded):
//
// A workgroup (4 waves) scores `pages_per_item` consecutive blocks of one
// (sequence, index head) pair; each wave streams whole 128-token pages.  A
// page of index keys is one contiguous run of 128 * Di elements (head-major
// pages), read with non-temporal 16-byte loads, 32 per lane in flight: Di/8
// lanes cover one token row, so a wave instruction reads 64/(Di/8) full rows.
// Every lane keeps the 8 query elements of its column slice in registers,
// forms an 8-term partial dot product, the row is summed across its lanes
// with DPP, tokens past the query are masked by select (never by
// multiplying, so stale bytes cannot leak), and the wave reduces the block
// max.
#pragma once

#include "msa_device.h"
#include "msa_internal.h"

namespace msa {

template <class IT, int DI>
__device__ void score_chunk(const ScoreArgs& a, int pair, int chunk) {
  constexpr int LPR = DI / 8;          // lanes per token row
  constexpr int RPL = kWave / LPR;     // token rows per wave load
  constexpr int NLOAD = kBlock / RPL;  // loads per page per lane
  // up to 128 VGPRs of loads in flight per lane
  constexpr int BATCH = (__is_same(IT, F32) ? 16 : 32) < NLOAD ? (__is_same(IT, F32) ? 16 : 32)
                                                               : NLOAD;
  static_assert(NLOAD % BATCH == 0, "batch must divide the page");

  const int b = pair / a.hidx;
  const int h = pair - b * a.hidx;
  const int L = a.seq_lens[b];
  // (a sequence longer than its table row is a caller error: clamp to the row)
  const int nb = L > 0 ? min((L - 1) / kBlock + 1, a.max_blocks) : 0;
  const int nchunks = div_up(nb, a.pages_per_item);
  float* srow = a.scores + static_cast<int64_t>(pair) * a.max_blocks;

  if (a.fill_tail && chunk == 0)
    for (int j = nb + threadIdx.x; j < a.max_blocks; j += kWgThreads) srow[j] = -INFINITY;
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
    if (lane == 0) srow[j] = m;
  }
}

// Short chunks: the n newest tokens of a sequence (positions L - n + i) are
// scored in one pass over the sequence's pages, QG queries at a time: each
// token row of a page is dotted with every query of the group and masked by
// that query's own position, so a page is read once for up to QG queries
// (and re-read from the L2 for further groups).  Rows of the sequence's
// queries get -inf past their last visible block.
template <class IT, int DI, int QG>
__device__ void score_chunk_multi(const ScoreArgs& a, int pair, int chunk) {
  constexpr int LPR = DI / 8;
  constexpr int RPL = kWave / LPR;
  constexpr int NLOAD = kBlock / RPL;
  constexpr int BATCH = (__is_same(IT, F32) ? 16 : 32) < NLOAD ? (__is_same(IT, F32) ? 16 : 32)
                                                               : NLOAD;
  static_assert(NLOAD % BATCH == 0, "batch must divide the page");

  const int b = pair / a.hidx;
  const int h = pair - b * a.hidx;
  const int L = a.seq_lens[b];
  const int c0 = a.cu_seqlens_q[b];
  const int n = a.cu_seqlens_q[b + 1] - c0;
  const int nb = n > 0 && L > 0 ? min((L - 1) / kBlock + 1, a.max_blocks) : 0;
  const int nchunks = div_up(nb, a.pages_per_item);
  auto srow = [&](int i) {
    return a.scores + (static_cast<int64_t>(c0 + i) * a.hidx + h) * a.max_blocks;
  };

  if (a.fill_tail && chunk == 0)
    for (int i = 0; i < n; ++i)
      for (int j = nb + threadIdx.x; j < a.max_blocks; j += kWgThreads) srow(i)[j] = -INFINITY;
  if (chunk >= nchunks) return;

  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  const int row = lane / LPR;
  const int col = lane % LPR;
  const IT* tag = nullptr;
  const int j0 = chunk * a.pages_per_item;
  const int j1 = min(nb, j0 + a.pages_per_item);

  for (int q0 = 0; q0 < n; q0 += QG) {
    float qv[QG][8];
    int pq[QG];  // position of each query of the group (-1: past the chunk)
#pragma unroll
    for (int qi = 0; qi < QG; ++qi) {
      const int i = q0 + qi;
      if (i < n) {
        load8(tag, a.idx_q, (static_cast<int64_t>(c0 + i) * a.hidx + h) * DI + col * 8, qv[qi]);
        pq[qi] = L - n + i;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[qi][e] = 0.f;
        pq[qi] = -1;
      }
    }
    for (int j = j0 + w; j < j1; j += kWgThreads / kWave) {
      const int page = a.block_table[static_cast<int64_t>(b) * a.max_blocks + j];
      float m[QG];
#pragma unroll
      for (int qi = 0; qi < QG; ++qi) m[qi] = -INFINITY;
      if (page >= 0 && page < a.num_pages) {
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
            const int t = j * kBlock + (i0 + i) * RPL + row;  // token position
#pragma unroll
            for (int qi = 0; qi < QG; ++qi) {
              float d = 0.f;
#pragma unroll
              for (int e = 0; e < 8; ++e) d = fmaf(qv[qi][e], x[e], d);
              d = group_sum<LPR>(d);
              m[qi] = fmaxf(m[qi], t <= pq[qi] ? d : -INFINITY);
            }
          }
        }
#pragma unroll
        for (int qi = 0; qi < QG; ++qi) m[qi] = wave_max(m[qi]);
      }
      if (lane == 0) {
#pragma unroll
        for (int qi = 0; qi < QG; ++qi)
          if (q0 + qi < n) srow(q0 + qi)[j] = m[qi];
      }
    }
  }
}

}  // namespace msa
