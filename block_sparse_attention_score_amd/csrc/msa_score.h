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
// forms an 8-term partial dot product (bf16 pairs on v_dot2c_f32_bf16), the
// row is summed across its lanes with DPP, tokens past the query are masked
// by select (never by multiplying, so stale bytes cannot leak), and the wave
// reduces the block max.
#pragma once

#include "msa_device.h"
#include "msa_internal.h"

namespace msa {

// The slice of the index query a lane dots with its 8 keys.  bf16 keys feed
// the query's bf16 pairs and their own straight into v_dot2c_f32_bf16 (two
// products and the running sum per instruction, no unpacking); f32 keys are
// unpacked and chained with fmaf.  Every scan sums in the same order, so the
// decode scan and the short-chunk scan give the same bits for one query.
template <class IT>
struct QSlice;
template <>
struct QSlice<BF16> {
  uint32_t w[4];
};
template <>
struct QSlice<F32> {
  float v[8];
};

__device__ __forceinline__ void load_qslice(const BF16* tag, const void* q, int64_t idx,
                                            QSlice<BF16>& s) {
  const Raw8<BF16> r = load_raw(tag, q, idx);
  s.w[0] = r.v.x; s.w[1] = r.v.y; s.w[2] = r.v.z; s.w[3] = r.v.w;
}
__device__ __forceinline__ void load_qslice(const F32* tag, const void* q, int64_t idx,
                                            QSlice<F32>& s) {
  load8(tag, q, idx, s.v);
}
__device__ __forceinline__ void zero_qslice(QSlice<BF16>& s) {
#pragma unroll
  for (int k = 0; k < 4; ++k) s.w[k] = 0u;
}
__device__ __forceinline__ void zero_qslice(QSlice<F32>& s) {
#pragma unroll
  for (int k = 0; k < 8; ++k) s.v[k] = 0.f;
}

__device__ __forceinline__ float dot8(const QSlice<BF16>& q, const Raw8<BF16>& k) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const uint32_t kw[4] = {k.v.x, k.v.y, k.v.z, k.v.w};
  float d = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.w[i]),
                                        __builtin_bit_cast(bf16x2_t, kw[i]), d, false);
  return d;
}
__device__ __forceinline__ float dot8(const QSlice<F32>& q, const Raw8<F32>& k) {
  float x[8];
  unpack(k, x);
  float d = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) d = fmaf(q.v[e], x[e], d);
  return d;
}

template <class IT, int DI, int ST = kScoreMax>
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

  QSlice<IT> qs;
  load_qslice(tag, a.idx_q, (static_cast<int64_t>(b) * a.hidx + h) * DI + col * 8, qs);

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
      BlockScore<ST> red;
#pragma unroll
      for (int i0 = 0; i0 < NLOAD; i0 += BATCH) {
        Raw8<IT> raw[BATCH];
#pragma unroll
        for (int i = 0; i < BATCH; ++i)
          raw[i] = load_raw(tag, a.idx_k, base + static_cast<int64_t>((i0 + i) * RPL) * DI);
        // the whole batch is in flight before the first dot product (the
        // scheduler would otherwise interleave loads and dot products and
        // keep about ten loads in flight)
        __builtin_amdgcn_sched_barrier(0);
        float d[BATCH];
        bool ok[BATCH];
#pragma unroll
        for (int i = 0; i < BATCH; ++i) {
          d[i] = group_sum<LPR>(dot8(qs, raw[i]));
          ok[i] = (i0 + i) * RPL + row < nvalid;
        }
        red.add(d, ok, col == 0, a.st_scale_log2);
      }
      m = red.finish(nvalid);
    }
    if (lane == 0) srow[j] = m;
  }
}

// Index-value branch, decode: one pass over the chunk's index keys yields its
// block scores (as score_chunk) and its share of the index-value attention
// (the sglang page hands the index-value cache to the decode op beside the
// index keys; the attention of the index query over every visible token's
// index key and value is the reading taken).  The logits are the block-score
// dots times 1/sqrt(Di); each lane keeps an online softmax (base 2) over the
// token rows it loads and the weighted sum of their values on its 8 dims; the
// rows of a wave, then the four waves, are merged, and the chunk's partial
// (Di sums, max, sum) goes to iv_part.  Value rows past the query are cleared
// before use (stale bytes may be NaN).  K and V loads go out 16 + 16 at a
// time per lane.
template <int DI>
struct IvLds {
  float m[4];
  float l[4];
  float o[4][DI];
};

__device__ __forceinline__ void clear_raw(Raw8<BF16>& r, bool keep) {
  const uint32_t k = keep ? 0xffffffffu : 0u;
  r.v.x &= k; r.v.y &= k; r.v.z &= k; r.v.w &= k;
}
__device__ __forceinline__ void clear_raw(Raw8<F32>& r, bool keep) {
  const uint32_t k = keep ? 0xffffffffu : 0u;
  r.a = make_float4(__uint_as_float(__float_as_uint(r.a.x) & k), __uint_as_float(__float_as_uint(r.a.y) & k),
                    __uint_as_float(__float_as_uint(r.a.z) & k), __uint_as_float(__float_as_uint(r.a.w) & k));
  r.b = make_float4(__uint_as_float(__float_as_uint(r.b.x) & k), __uint_as_float(__float_as_uint(r.b.y) & k),
                    __uint_as_float(__float_as_uint(r.b.z) & k), __uint_as_float(__float_as_uint(r.b.w) & k));
}

// (m, l, o) of two disjoint token sets merged into the first (base 2).
__device__ __forceinline__ void iv_merge(float& m, float& l, float (&o)[8], float m2, float l2,
                                         const float (&o2)[8]) {
  const float M = fmaxf(m, m2);
  const float mu = M == -INFINITY ? 0.f : M;
  const float a1 = __builtin_amdgcn_exp2f(m - mu);
  const float a2 = __builtin_amdgcn_exp2f(m2 - mu);
  l = l * a1 + l2 * a2;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = o[e] * a1 + o2[e] * a2;
  m = M;
}

template <class IT, int DI, int ST = kScoreMax>
__device__ void score_value_chunk(const ScoreArgs& a, int pair, int chunk, IvLds<DI>& S) {
  constexpr int LPR = DI / 8;          // lanes per token row
  constexpr int RPL = kWave / LPR;     // token rows per wave load
  constexpr int NLOAD = kBlock / RPL;  // loads per page per lane
  constexpr int BATCH = 16 < NLOAD ? 16 : NLOAD;
  static_assert(NLOAD % BATCH == 0, "batch must divide the page");

  const int b = pair / a.hidx;
  const int h = pair - b * a.hidx;
  const int L = a.seq_lens[b];
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

  QSlice<IT> qs;
  load_qslice(tag, a.idx_q, (static_cast<int64_t>(b) * a.hidx + h) * DI + col * 8, qs);

  const int p = L - 1;
  const int j0 = chunk * a.pages_per_item;
  const int j1 = min(nb, j0 + a.pages_per_item);
  float om = -INFINITY, ol = 0.f;
  float oacc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) oacc[e] = 0.f;
  for (int j = j0 + w; j < j1; j += kWgThreads / kWave) {
    const int page = a.block_table[static_cast<int64_t>(b) * a.max_blocks + j];
    float m = -INFINITY;
    if (page >= 0 && page < a.num_pages) {
      const int nvalid = min(kBlock, p + 1 - j * kBlock);
      const int64_t base =
          (static_cast<int64_t>(page) * a.hidx + h) * kBlock * DI + row * DI + col * 8;
      BlockScore<ST> red;
#pragma unroll
      for (int i0 = 0; i0 < NLOAD; i0 += BATCH) {
        Raw8<IT> rk[BATCH], rv[BATCH];
#pragma unroll
        for (int i = 0; i < BATCH; ++i)
          rk[i] = load_raw(tag, a.idx_k, base + static_cast<int64_t>((i0 + i) * RPL) * DI);
#pragma unroll
        for (int i = 0; i < BATCH; ++i)
          rv[i] = load_raw(tag, a.idx_v, base + static_cast<int64_t>((i0 + i) * RPL) * DI);
        float sc[BATCH], dd[BATCH];
        bool okv[BATCH];
        float mb = om;
#pragma unroll
        for (int i = 0; i < BATCH; ++i) {
          dd[i] = group_sum<LPR>(dot8(qs, rk[i]));
          okv[i] = (i0 + i) * RPL + row < nvalid;
          sc[i] = okv[i] ? dd[i] * a.iv_scale_log2 : -INFINITY;
          mb = fmaxf(mb, sc[i]);
        }
        red.add(dd, okv, col == 0, a.st_scale_log2);
        // online softmax over this lane's rows: rescale by the new maximum
        const float mu = mb == -INFINITY ? 0.f : mb;
        const float alpha = __builtin_amdgcn_exp2f(om - mu);
        ol *= alpha;
#pragma unroll
        for (int e = 0; e < 8; ++e) oacc[e] *= alpha;
#pragma unroll
        for (int i = 0; i < BATCH; ++i) {
          const float pr = __builtin_amdgcn_exp2f(sc[i] - mu);
          ol += pr;
          clear_raw(rv[i], (i0 + i) * RPL + row < nvalid);
          float v[8];
          unpack(rv[i], v);
#pragma unroll
          for (int e = 0; e < 8; ++e) oacc[e] = fmaf(pr, v[e], oacc[e]);
        }
        om = mb;
      }
      m = red.finish(nvalid);
    }
    if (lane == 0) srow[j] = m;
  }

  // rows of the wave (lanes col, col + LPR, ...), then the four waves
#pragma unroll
  for (int off = LPR; off < kWave; off <<= 1) {
    float o2[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o2[e] = __shfl_xor(oacc[e], off);
    const float m2 = __shfl_xor(om, off);
    const float l2 = __shfl_xor(ol, off);
    iv_merge(om, ol, oacc, m2, l2, o2);
  }
  if (lane < LPR) {
#pragma unroll
    for (int e = 0; e < 8; ++e) S.o[w][col * 8 + e] = oacc[e];
    if (lane == 0) {
      S.m[w] = om;
      S.l[w] = ol;
    }
  }
  __syncthreads();
  float* part = a.iv_part + (static_cast<int64_t>(pair) * a.chunks_per_pair + chunk) * (DI + 2);
  const int tid = threadIdx.x;
  if (tid < DI + 2) {
    float M = S.m[0];
#pragma unroll
    for (int ww = 1; ww < 4; ++ww) M = fmaxf(M, S.m[ww]);
    const float mu = M == -INFINITY ? 0.f : M;
    float v = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const float sw = __builtin_amdgcn_exp2f(S.m[ww] - mu);
      v += sw * (tid < DI ? S.o[ww][tid] : S.l[ww]);
    }
    part[tid] = tid < DI ? v : (tid == DI ? M : v);
  }
}

// Short chunks: the n newest tokens of a sequence (positions L - n + i) are
// scored in one pass over the sequence's pages, QG queries at a time: each
// token row of a page is dotted with every query of the group and masked by
// that query's own position, so a page is read once for up to QG queries
// (and re-read from the L2 for further groups).  Rows of the sequence's
// queries get -inf past their last visible block.
template <class IT, int DI, int QG, int ST = kScoreMax>
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
    QSlice<IT> qs[QG];
    int pq[QG];  // position of each query of the group (-1: past the chunk)
#pragma unroll
    for (int qi = 0; qi < QG; ++qi) {
      const int i = q0 + qi;
      if (i < n) {
        load_qslice(tag, a.idx_q, (static_cast<int64_t>(c0 + i) * a.hidx + h) * DI + col * 8,
                    qs[qi]);
        pq[qi] = L - n + i;
      } else {
        zero_qslice(qs[qi]);
        pq[qi] = -1;
      }
    }
    for (int j = j0 + w; j < j1; j += kWgThreads / kWave) {
      const int page = a.block_table[static_cast<int64_t>(b) * a.max_blocks + j];
      float m[QG];
#pragma unroll
      for (int qi = 0; qi < QG; ++qi) m[qi] = -INFINITY;
      BlockScore<ST> red[QG];
      if (page >= 0 && page < a.num_pages) {
        const int64_t base =
            (static_cast<int64_t>(page) * a.hidx + h) * kBlock * DI + row * DI + col * 8;
#pragma unroll
        for (int i0 = 0; i0 < NLOAD; i0 += BATCH) {
          Raw8<IT> raw[BATCH];
#pragma unroll
          for (int i = 0; i < BATCH; ++i)
            raw[i] = load_raw(tag, a.idx_k, base + static_cast<int64_t>((i0 + i) * RPL) * DI);
          // (no scheduling barrier here: with four queries' dot products per
          // load, interleaving loads and compute measured faster)
#pragma unroll
          for (int i = 0; i < BATCH; ++i) {
            const int t = j * kBlock + (i0 + i) * RPL + row;  // token position
#pragma unroll
            for (int qi = 0; qi < QG; ++qi) {
              const float d[1] = {group_sum<LPR>(dot8(qs[qi], raw[i]))};
              const bool ok[1] = {t <= pq[qi]};
              red[qi].add(d, ok, col == 0, a.st_scale_log2);
            }
          }
        }
        // visible tokens of the block for each query (keys past the sequence
        // end are after every query)
#pragma unroll
        for (int qi = 0; qi < QG; ++qi)
          m[qi] = red[qi].finish(min(kBlock, pq[qi] + 1 - j * kBlock));
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
