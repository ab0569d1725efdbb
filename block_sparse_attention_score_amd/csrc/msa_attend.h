// Decode attention over the selected blocks (one split of one (sequence, kv
// head) unit): split-K flash-decode with a fused log-sum-exp combine.
//
// vLLM page sparse_attention_msa.py (module docstring and
// MiniMaxM3SparseMSAImpl.forward): decode attends over the top-k blocks of a
// paged cache with a split-K kernel, fp8 caches carrying k/v scales.  Here a
// workgroup owns (sequence b, kv head g, split c) and handles the `bps`
// selected blocks c*bps .. of the index head that serves g, for all G query
// heads of g at once (the GQA group shares every K/V byte it loads).
//
// Per 128-token block:
//  * S = q K^T on the matrix cores: q (G heads, zero-padded to 16 rows) is
//    the A operand, K rows are read straight from the page into the B
//    operand (16 tokens x 32 dims per instruction, 64 contiguous bytes per
//    token), v_mfma_f32_16x16x32_bf16 (fp8 codes widen to bf16 exactly) or
//    v_mfma_f32_16x16x4_f32 for f32 caches;
//  * tokens past the query are masked to -inf by select; online softmax in
//    base 2 (max and sum reduced over DPP rows, then across waves in LDS);
//  * P V on the vector ALUs: each lane owns 4 dims of one token row (two rows
//    per wave load), reads V with coalesced 8-byte loads, zeroes rows past
//    the query (V may hold stale NaN bytes there) and accumulates all G heads,
//    whose probabilities it reads from LDS as 16-byte vectors;
//  * the next block's K and V loads are issued before the current block is
//    computed (two-stage pipeline over the split's blocks).
// The split writes its normalised partial output and lse; the last split to
// finish (atomic ticket) merges the partials:
//   lse = log sum_c exp(lse_c),  out = sum_c exp(lse_c - lse) o_c.
#pragma once

#include "msa_device.h"
#include "msa_internal.h"

namespace msa {

constexpr float kLn2 = 0.69314718055994530942f;
constexpr int kMaxBps = 32;  // selected blocks per split workgroup, at most

// ----------------------------------------------------------- q fragments

template <class QT>
struct QFrag;

// bf16 queries: A operand of four 16x16x32 steps; lane holds 8 dims of head
// row (lane % 16): dims 32*s + 8*(lane / 16) .. +8.
template <>
struct QFrag<BF16> {
  bf16x8_t a[4];
};

// f32 queries: A operand of 32 16x16x4 steps; step (m, e) contracts dim
// 16*m + 4*(lane / 16) + e, the same dims the K loads below deliver.
template <>
struct QFrag<F32> {
  float4 a[8];
};

template <int G>
__device__ __forceinline__ void load_qfrag(const BF16*, const void* q, int64_t row0,
                                           int qrow, int kgrp, QFrag<BF16>& f) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    if (qrow < G) {
      f.a[s] = *reinterpret_cast<const bf16x8_t*>(reinterpret_cast<const uint16_t*>(q) +
                                                  (row0 + qrow) * 128 + 32 * s + 8 * kgrp);
    } else {
      f.a[s] = bf16x8_t{};
    }
  }
}

template <int G>
__device__ __forceinline__ void load_qfrag(const F32*, const void* q, int64_t row0,
                                           int qrow, int kgrp, QFrag<F32>& f) {
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    if (qrow < G) {
      f.a[m] = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(q) +
                                                (row0 + qrow) * 128 + 16 * m + 4 * kgrp);
    } else {
      f.a[m] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
}

// K rows of one block for this wave's two 16-token tiles (the B operand of
// S = q K^T), kept as loaded until the MFMAs consume them.
template <class KT>
struct KFrag;
template <>
struct KFrag<BF16> {
  bf16x8_t k[2][4];
};
template <>
struct KFrag<FP8> {
  Raw8<FP8> k[2][4];
};
template <>
struct KFrag<F32> {
  f32x4v_t k[2][8];
};

// `row0` indexes element 0 of token (16 * tile0 + lane % 16) of the block.
__device__ __forceinline__ void load_kfrag(const void* kp, int64_t row0, int kgrp,
                                           KFrag<BF16>& f) {
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int s = 0; s < 4; ++s)
      f.k[tt][s] = load8_bf16(static_cast<const BF16*>(nullptr), kp,
                              row0 + tt * 16 * 128 + 32 * s + 8 * kgrp);
}
__device__ __forceinline__ void load_kfrag(const void* kp, int64_t row0, int kgrp,
                                           KFrag<FP8>& f) {
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int s = 0; s < 4; ++s)
      f.k[tt][s] = load_raw(static_cast<const FP8*>(nullptr), kp,
                            row0 + tt * 16 * 128 + 32 * s + 8 * kgrp);
}
__device__ __forceinline__ void load_kfrag(const void* kp, int64_t row0, int kgrp,
                                           KFrag<F32>& f) {
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int m = 0; m < 8; ++m)
      f.k[tt][m] = __builtin_nontemporal_load(reinterpret_cast<const f32x4v_t*>(
          reinterpret_cast<const float*>(kp) + row0 + tt * 16 * 128 + 16 * m + 4 * kgrp));
}

__device__ __forceinline__ bf16x8_t fp8_to_bf16x8(const Raw8<FP8>& r) {
  float x[8];
  unpack(r, x);
  uint32_t u[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    u[i] = (__float_as_uint(x[2 * i]) >> 16) | (__float_as_uint(x[2 * i + 1]) & 0xffff0000u);
  bf16x8_t v;
  __builtin_memcpy(&v, u, 16);
  return v;
}

// S tile tt (16 head rows x 16 tokens) from a K fragment.
__device__ __forceinline__ f32x4_t qk_tile(const QFrag<BF16>& q, const KFrag<BF16>& f, int tt) {
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; ++s)
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(q.a[s], f.k[tt][s], acc, 0, 0, 0);
  return acc;
}
__device__ __forceinline__ f32x4_t qk_tile(const QFrag<BF16>& q, const KFrag<FP8>& f, int tt) {
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; ++s)
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(q.a[s], fp8_to_bf16x8(f.k[tt][s]), acc, 0, 0, 0);
  return acc;
}
__device__ __forceinline__ f32x4_t qk_tile(const QFrag<F32>& q, const KFrag<F32>& f, int tt) {
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(q.a[m].x, f.k[tt][m].x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(q.a[m].y, f.k[tt][m].y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(q.a[m].z, f.k[tt][m].z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(q.a[m].w, f.k[tt][m].w, acc, 0, 0, 0);
  }
  return acc;
}

__device__ __forceinline__ void store_out(const BF16*, void* out, int64_t idx, float v) {
  reinterpret_cast<uint16_t*>(out)[idx] = f32_to_bf16(v);
}
__device__ __forceinline__ void store_out(const F32*, void* out, int64_t idx, float v) {
  reinterpret_cast<float*>(out)[idx] = v;
}

__device__ __forceinline__ float exp2_or_zero(float x, float m) {
  return x == -INFINITY ? 0.f : exp2f(x - m);
}

// ---------------------------------------------------------- split unit

template <int G>
struct AttendLds {
  alignas(16) float Ps[kBlock][G < 4 ? 4 : G];  // probabilities of the current block, token-major
  float red_max[4][16];
  float red_sum[4][16];
  float m_run[16];
  float l_run[16];
  float alpha_s[16];
  float red_o[4][G][kBlock];
  int blk_nvalid[kMaxBps];
  int blk_page[kMaxBps];
  int is_last;
};

// Sequence and position of query token t: decode has one query per sequence
// at its last position; prefill tokens are the last n_b tokens of their
// sequence (cu_seqlens_q).
__device__ __forceinline__ void query_of(const AttendArgs& a, int t, int& b, int& p) {
  if (a.cu_seqlens_q == nullptr) {
    b = t;
    p = a.seq_lens[t] - 1;
    return;
  }
  int lo = 0, hi = a.num_seqs;  // cu[lo] <= t < cu[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) / 2;
    if (a.cu_seqlens_q[mid] <= t) lo = mid; else hi = mid;
  }
  b = lo;
  p = a.seq_lens[b] - (a.cu_seqlens_q[b + 1] - a.cu_seqlens_q[b]) + (t - a.cu_seqlens_q[b]);
}

// One split (blocks split*bps ..) of the (query token t, kv head g) unit.
// Called by all 256 threads of a workgroup.  FUSED: the selection was produced
// by other workgroups of the same launch (coherent loads, after the pair's
// ready flag).
template <class QT, class KT, int G, bool FUSED>
__device__ void attend_split(const AttendArgs& a, int split, int g, int t, AttendLds<G>& S) {
  const int h = g / (a.hkv / a.hidx);
  const int sel_row = t * a.hidx + h;
  int b, p;
  query_of(a, t, b, p);
  const int cnt_raw = FUSED ? load_shared_i32(a.cnt + sel_row) : a.cnt[sel_row];
  const int count = p >= 0 ? min(max(cnt_raw, 0), a.kmax) : 0;
  const int nsplit = div_up(count, a.bps);
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int w = tid / kWave;
  const int64_t hq0 = static_cast<int64_t>(t) * a.hkv * G + static_cast<int64_t>(g) * G;
  const QT* qtag = nullptr;
  const KT* ktag = nullptr;

  if (count == 0) {
    if (split == 0) {
      for (int i = tid; i < G * 128; i += kWgThreads) store_out(qtag, a.out, hq0 * 128 + i, 0.f);
      if (a.lse_out != nullptr && tid < G) a.lse_out[hq0 + tid] = -INFINITY;
    }
    return;
  }
  if (split >= nsplit) return;

  const int qrow = lane & 15;   // MFMA row (head) / column (token) index
  const int kgrp = lane >> 4;   // MFMA k-slot group; D rows 4*kgrp .. +3
  const int prow = lane >> 5;   // P V: token row within a pair
  const int pcol = lane & 31;   // P V: dims 4*pcol .. +4
  constexpr int GP = G < 4 ? 4 : G;  // row stride of Ps

  QFrag<QT> qf;
  load_qfrag<G>(qtag, a.q, hq0, qrow, kgrp, qf);
  if (tid < 16) {
    S.m_run[tid] = -INFINITY;
    S.l_run[tid] = 0.f;
  }
  float acc[G][4];
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[hh][e] = 0.f;

  // Block ids and pages of this split (at most kMaxBps), resolved up front.
  const int bi0 = split * a.bps;
  const int nblk = min(count, bi0 + a.bps) - bi0;
  if (tid < nblk) {
    const int64_t at = static_cast<int64_t>(sel_row) * a.kmax + bi0 + tid;
    const int j = FUSED ? load_shared_i32(a.sel + at) : a.sel[at];
    int page;
    if (a.sel_pages != nullptr)
      page = FUSED ? load_shared_i32(a.sel_pages + at) : a.sel_pages[at];
    else
      page = j >= 0 && j < a.max_blocks ? a.block_table[static_cast<int64_t>(b) * a.max_blocks + j]
                                        : -1;
    const bool ok = page >= 0 && page < a.num_pages && j >= 0;
    S.blk_nvalid[tid] = ok ? max(0, min(kBlock, p + 1 - j * kBlock)) : 0;
    S.blk_page[tid] = ok ? page : 0;
  }
  __syncthreads();

  // Element 0 of this lane's K row (tile 2w) and V row (token row prow) of block i.
  auto k_row0 = [&](int i) {
    return (static_cast<int64_t>(S.blk_page[i]) * a.hkv + g) * kBlock * 128 +
           static_cast<int64_t>(32 * w + qrow) * 128;
  };
  auto v_row0 = [&](int i) {
    return (static_cast<int64_t>(S.blk_page[i]) * a.hkv + g) * kBlock * 128 +
           static_cast<int64_t>(32 * w + prow) * 128 + 4 * pcol;
  };

  // Two-stage pipeline: the next block's K and V are in flight while the
  // current block is computed.
  KFrag<KT> kc, kn;
  Raw4<KT> vc[16], vn[16];
  load_kfrag(a.k_pool, k_row0(0), kgrp, kc);
#pragma unroll
  for (int i = 0; i < 16; ++i)
    vc[i] = load_raw4(ktag, a.v_pool, v_row0(0) + static_cast<int64_t>(2 * i) * 128);

  for (int bi = 0; bi < nblk; ++bi) {
    const int nvalid = S.blk_nvalid[bi];
    const bool more = bi + 1 < nblk;
    if (more) load_kfrag(a.k_pool, k_row0(bi + 1), kgrp, kn);

    // S for this wave's 32 tokens: tiles n = 2w and 2w+1.
    f32x4_t s[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int tok = 32 * w + 16 * tt + qrow;
      s[tt] = qk_tile(qf, kc, tt);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        s[tt][r] = tok < nvalid ? s[tt][r] * a.qk_scale_log2 : -INFINITY;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float mx = group_max<16>(fmaxf(s[0][r], s[1][r]));
      if (qrow == 0) S.red_max[w][4 * kgrp + r] = mx;
    }
    __syncthreads();
    if (tid < 16) {
      const float mb = fmaxf(fmaxf(S.red_max[0][tid], S.red_max[1][tid]),
                             fmaxf(S.red_max[2][tid], S.red_max[3][tid]));
      const float mo = S.m_run[tid];
      const float mn = fmaxf(mo, mb);
      S.alpha_s[tid] = mo == mn ? 1.f : exp2f(mo - mn);
      S.m_run[tid] = mn;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int hr = 4 * kgrp + r;
      const float mr = S.m_run[hr];
      const float p0 = exp2_or_zero(s[0][r], mr);
      const float p1 = exp2_or_zero(s[1][r], mr);
      if (hr < G) {
        S.Ps[32 * w + qrow][hr] = p0;
        S.Ps[32 * w + 16 + qrow][hr] = p1;
      }
      const float sm = group_sum<16>(p0 + p1);
      if (qrow == 0) S.red_sum[w][hr] = sm;
    }
    __syncthreads();
    if (more) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        vn[i] = load_raw4(ktag, a.v_pool, v_row0(bi + 1) + static_cast<int64_t>(2 * i) * 128);
    }
    if (tid < 16)
      S.l_run[tid] = S.l_run[tid] * S.alpha_s[tid] +
                   (S.red_sum[0][tid] + S.red_sum[1][tid]) + (S.red_sum[2][tid] + S.red_sum[3][tid]);
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const float al = S.alpha_s[hh];
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[hh][e] *= al;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int tok = 32 * w + 2 * i + prow;
      float v[4];
      unpack4(vc[i], v);
      const bool valid = tok < nvalid;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = valid ? v[e] : 0.f;
#pragma unroll
      for (int h4 = 0; h4 < GP; h4 += 4) {
        const float4 pp = *reinterpret_cast<const float4*>(&S.Ps[tok][h4]);
        const float pv[4] = {pp.x, pp.y, pp.z, pp.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (h4 + u < G) {
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[h4 + u][e] = fmaf(pv[u], v[e], acc[h4 + u][e]);
          }
        }
      }
    }
    __syncthreads();
    if (more) {
      kc = kn;
#pragma unroll
      for (int i = 0; i < 16; ++i) vc[i] = vn[i];
    }
  }

  // Sum the two token rows of each wave, then the four waves.
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[hh][e] += __shfl_xor(acc[hh][e], 32);
  if (prow == 0) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int e = 0; e < 4; ++e) S.red_o[w][hh][4 * pcol + e] = acc[hh][e];
  }
  __syncthreads();

  const int64_t part0 =
      ((static_cast<int64_t>(t) * a.hkv + g) * a.nsplit_max + split) * G;
  for (int i = tid; i < G * 128; i += kWgThreads) {
    const int hh = i / 128;
    const int d = i % 128;
    const float l = S.l_run[hh];
    const float o = l > 0.f ? ((S.red_o[0][hh][d] + S.red_o[1][hh][d]) +
                               (S.red_o[2][hh][d] + S.red_o[3][hh][d])) * (a.v_scale / l)
                            : 0.f;
    if (nsplit == 1) {
      store_out(qtag, a.out, (hq0 + hh) * 128 + d, o);
    } else {
      store_shared_f32(a.part_o + (part0 + hh) * 128 + d, o);
    }
  }
  if (tid < G) {
    const float lse = S.l_run[tid] > 0.f ? (S.m_run[tid] + log2f(S.l_run[tid])) * kLn2 : -INFINITY;
    if (nsplit == 1) {
      if (a.lse_out != nullptr) a.lse_out[hq0 + tid] = lse;
    } else {
      store_shared_f32(a.part_lse + part0 + tid, lse);
    }
  }
  if (nsplit == 1) return;

  // The last split of (b, g) to finish merges all partials.
  if (!take_last_ticket(&a.tickets[static_cast<int64_t>(t) * a.hkv + g], nsplit, &S.is_last))
    return;
  const int64_t base0 = (static_cast<int64_t>(t) * a.hkv + g) * a.nsplit_max * G;
  // Split weights exp(lse_c - lse) of every head, once, in LDS (the partial
  // lse values are loaded by many threads at once).
  float* w_lds = &S.red_o[0][0][0];  // reused: nsplit_max * G <= 4 * G * 128 floats
  for (int i = tid; i < nsplit * G; i += kWgThreads) w_lds[i] = load_shared_f32(a.part_lse + base0 + i);
  __syncthreads();
  if (tid < G) {
    float mx = -INFINITY;
    for (int c = 0; c < nsplit; ++c) mx = fmaxf(mx, w_lds[c * G + tid]);
    float ws = 0.f;
    if (mx != -INFINITY)
      for (int c = 0; c < nsplit; ++c) ws += __expf(w_lds[c * G + tid] - mx);
    const float inv = ws > 0.f ? 1.f / ws : 0.f;
    for (int c = 0; c < nsplit; ++c)
      w_lds[c * G + tid] = mx != -INFINITY ? __expf(w_lds[c * G + tid] - mx) * inv : 0.f;
    if (a.lse_out != nullptr) a.lse_out[hq0 + tid] = ws > 0.f ? mx + __logf(ws) : -INFINITY;
  }
  __syncthreads();
  // out = sum_c w_c o_c, partials read in independent batches of 8.
  for (int i = tid; i < G * 128; i += kWgThreads) {
    const int hh = i / 128;
    const int d = i % 128;
    const float* po = a.part_o + (base0 + hh) * 128 + d;
    float o = 0.f;
    for (int c0 = 0; c0 < nsplit; c0 += 8) {
      // straight-line batch: indices past the last split re-read the last one
      // and get weight 0
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        v[u] = load_shared_f32(po + static_cast<int64_t>(min(c0 + u, nsplit - 1)) * G * 128);
#pragma unroll
      for (int u = 0; u < 8; ++u)
        o = fmaf(c0 + u < nsplit ? w_lds[(c0 + u) * G + hh] : 0.f, v[u], o);
    }
    store_out(qtag, a.out, (hq0 + hh) * 128 + d, o);
  }
}


}  // namespace msa
