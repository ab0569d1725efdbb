// Decode attention over the selected blocks: split-K flash-decode with a fused
// log-sum-exp combine.
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
//  * P V on the vector ALUs: each lane owns 8 dims of one token row, reads V
//    with one coalesced 16-byte load, zeroes rows past the query (V may hold
//    stale NaN bytes there) and accumulates all G heads.
// The split writes its normalised partial output and lse; the last split to
// finish (atomic ticket) merges the partials:
//   lse = log sum_c exp(lse_c),  out = sum_c exp(lse_c - lse) o_c.
#include "msa_device.h"
#include "msa_internal.h"

namespace msa {

constexpr float kLn2 = 0.69314718055994530942f;

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

// S tile (16 head rows x 16 tokens): `krow` indexes element 0 of this lane's
// token row in the K pool.
template <class KT>
__device__ __forceinline__ f32x4_t qk_tile(const QFrag<BF16>& f, const void* kp,
                                           int64_t krow, int kgrp) {
  const KT* tag = nullptr;
  bf16x8_t kb[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) kb[s] = load8_bf16(tag, kp, krow + 32 * s + 8 * kgrp);
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; ++s)
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.a[s], kb[s], acc, 0, 0, 0);
  return acc;
}

template <class KT>
__device__ __forceinline__ f32x4_t qk_tile(const QFrag<F32>& f, const void* kp,
                                           int64_t krow, int kgrp) {
  f32x4v_t kb[8];
#pragma unroll
  for (int m = 0; m < 8; ++m)
    kb[m] = __builtin_nontemporal_load(reinterpret_cast<const f32x4v_t*>(
        reinterpret_cast<const float*>(kp) + krow + 16 * m + 4 * kgrp));
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(f.a[m].x, kb[m].x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(f.a[m].y, kb[m].y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(f.a[m].z, kb[m].z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(f.a[m].w, kb[m].w, acc, 0, 0, 0);
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

// ------------------------------------------------------------------ kernel

template <class QT, class KT, int G>
__global__ __launch_bounds__(kWgThreads) void decode_attend_kernel(AttendArgs a) {
  __shared__ float Ps[G][kBlock];
  __shared__ float red_max[4][16];
  __shared__ float red_sum[4][16];
  __shared__ float m_run[16];
  __shared__ float l_run[16];
  __shared__ float alpha_s[16];
  __shared__ float red_o[4][G][kBlock];
  __shared__ int is_last;

  const int split = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int h = g / (a.hkv / a.hidx);
  const int sel_row = b * a.hidx + h;
  // independent loads, all in flight together
  const int L = a.seq_lens[b];
  const int cnt_raw = a.cnt[sel_row];
  const int count = L > 0 ? min(max(cnt_raw, 0), a.kmax) : 0;
  const int nsplit = div_up(count, a.bps);
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int w = tid / kWave;
  const int64_t hq0 = static_cast<int64_t>(b) * a.hkv * G + static_cast<int64_t>(g) * G;
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

  const int p = L - 1;
  const int qrow = lane & 15;   // MFMA row (head) / column (token) index
  const int kgrp = lane >> 4;   // MFMA k-slot group; D rows 4*kgrp .. +3
  const int prow = lane >> 4;   // P V: token row within a group of 4
  const int pcol = lane & 15;   // P V: dims 8*pcol .. +8

  QFrag<QT> qf;
  load_qfrag<G>(qtag, a.q, hq0, qrow, kgrp, qf);
  if (tid < 16) {
    m_run[tid] = -INFINITY;
    l_run[tid] = 0.f;
  }
  float acc[G][8];
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[hh][e] = 0.f;

  const int32_t* selrow = a.sel + static_cast<int64_t>(sel_row) * a.kmax;
  const int bi0 = split * a.bps;
  const int bi1 = min(count, bi0 + a.bps);
  __syncthreads();

  const int32_t* pagerow =
      a.sel_pages != nullptr ? a.sel_pages + static_cast<int64_t>(sel_row) * a.kmax : nullptr;
  for (int bi = bi0; bi < bi1; ++bi) {
    const int j = selrow[bi];
    int page;
    if (pagerow != nullptr)
      page = pagerow[bi];
    else
      page = j >= 0 && j < a.max_blocks ? a.block_table[static_cast<int64_t>(b) * a.max_blocks + j]
                                        : -1;
    const bool ok = page >= 0 && page < a.num_pages;
    const int nvalid = ok ? min(kBlock, p + 1 - j * kBlock) : 0;
    const int64_t kvb = ok ? (static_cast<int64_t>(page) * a.hkv + g) * kBlock * 128 : 0;

    // V rows of this lane, loaded early so their latency overlaps the softmax.
    Raw8<KT> vraw[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int tok = 32 * w + 4 * i + prow;
      vraw[i] = load_raw(ktag, a.v_pool, kvb + static_cast<int64_t>(tok) * 128 + 8 * pcol);
    }

    // S for this wave's 32 tokens: tiles n = 2w and 2w+1.
    f32x4_t s[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int tok = 16 * (2 * w + tt) + qrow;
      s[tt] = qk_tile<KT>(qf, a.k_pool, kvb + static_cast<int64_t>(tok) * 128, kgrp);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        s[tt][r] = tok < nvalid ? s[tt][r] * a.qk_scale_log2 : -INFINITY;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float mx = group_max<16>(fmaxf(s[0][r], s[1][r]));
      if (qrow == 0) red_max[w][4 * kgrp + r] = mx;
    }
    __syncthreads();
    if (tid < 16) {
      const float mb = fmaxf(fmaxf(red_max[0][tid], red_max[1][tid]),
                             fmaxf(red_max[2][tid], red_max[3][tid]));
      const float mo = m_run[tid];
      const float mn = fmaxf(mo, mb);
      alpha_s[tid] = mo == mn ? 1.f : exp2f(mo - mn);
      m_run[tid] = mn;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int hr = 4 * kgrp + r;
      const float mr = m_run[hr];
      const float p0 = exp2_or_zero(s[0][r], mr);
      const float p1 = exp2_or_zero(s[1][r], mr);
      if (hr < G) {
        Ps[hr][32 * w + qrow] = p0;
        Ps[hr][32 * w + 16 + qrow] = p1;
      }
      const float sm = group_sum<16>(p0 + p1);
      if (qrow == 0) red_sum[w][hr] = sm;
    }
    __syncthreads();
    if (tid < 16)
      l_run[tid] = l_run[tid] * alpha_s[tid] +
                   (red_sum[0][tid] + red_sum[1][tid]) + (red_sum[2][tid] + red_sum[3][tid]);
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const float al = alpha_s[hh];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[hh][e] *= al;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int tok = 32 * w + 4 * i + prow;
      float v[8];
      unpack(vraw[i], v);
      const bool valid = tok < nvalid;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = valid ? v[e] : 0.f;
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float pp = Ps[hh][tok];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[hh][e] = fmaf(pp, v[e], acc[hh][e]);
      }
    }
    __syncthreads();
  }

  // Sum the four token rows of each wave, then the four waves.
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = acc[hh][e];
      x += __shfl_xor(x, 16);
      x += __shfl_xor(x, 32);
      acc[hh][e] = x;
    }
  if (prow == 0) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int e = 0; e < 8; ++e) red_o[w][hh][8 * pcol + e] = acc[hh][e];
  }
  __syncthreads();

  const int64_t part0 =
      ((static_cast<int64_t>(b) * a.hkv + g) * a.nsplit_max + split) * G;
  for (int i = tid; i < G * 128; i += kWgThreads) {
    const int hh = i / 128;
    const int d = i % 128;
    const float l = l_run[hh];
    const float o = l > 0.f ? ((red_o[0][hh][d] + red_o[1][hh][d]) +
                               (red_o[2][hh][d] + red_o[3][hh][d])) * (a.v_scale / l)
                            : 0.f;
    if (nsplit == 1) {
      store_out(qtag, a.out, (hq0 + hh) * 128 + d, o);
    } else {
      store_shared_f32(a.part_o + (part0 + hh) * 128 + d, o);
    }
  }
  if (tid < G) {
    const float lse = l_run[tid] > 0.f ? (m_run[tid] + log2f(l_run[tid])) * kLn2 : -INFINITY;
    if (nsplit == 1) {
      if (a.lse_out != nullptr) a.lse_out[hq0 + tid] = lse;
    } else {
      store_shared_f32(a.part_lse + part0 + tid, lse);
    }
  }
  if (nsplit == 1) return;

  // The last split of (b, g) to finish merges all partials.
  if (!take_last_ticket(&a.tickets[b * a.hkv + g], nsplit, &is_last)) return;
  const int64_t base0 = (static_cast<int64_t>(b) * a.hkv + g) * a.nsplit_max * G;
  // Split weights exp(lse_c - lse) of every head, once, in LDS (the partial
  // lse values are loaded by many threads at once).
  float* w_lds = &red_o[0][0][0];  // reused: nsplit_max * G <= 4 * G * 128 floats
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

// ------------------------------------------------------------ launcher

template <class QT, class KT, int G>
static void launch_attend_t(const AttendArgs& a, hipStream_t s) {
  const dim3 grid(a.nsplit_max, a.hkv, a.num_seqs);
  decode_attend_kernel<QT, KT, G><<<grid, kWgThreads, 0, s>>>(a);
}

template <class QT, class KT>
static bool launch_attend_g(const AttendArgs& a, int group, hipStream_t s) {
  switch (group) {
    case 1: launch_attend_t<QT, KT, 1>(a, s); return true;
    case 2: launch_attend_t<QT, KT, 2>(a, s); return true;
    case 4: launch_attend_t<QT, KT, 4>(a, s); return true;
    case 8: launch_attend_t<QT, KT, 8>(a, s); return true;
    case 16: launch_attend_t<QT, KT, 16>(a, s); return true;
    default: return false;
  }
}

hipError_t launch_decode_attend(const AttendArgs& a, int q_dtype, int kv_dtype, int group,
                                hipStream_t s) {
  if (a.num_seqs == 0) return hipSuccess;
  bool ok = false;
  if (q_dtype == 0 && kv_dtype == 0) ok = launch_attend_g<BF16, BF16>(a, group, s);
  else if (q_dtype == 0 && kv_dtype == 2) ok = launch_attend_g<BF16, FP8>(a, group, s);
  else if (q_dtype == 1 && kv_dtype == 1) ok = launch_attend_g<F32, F32>(a, group, s);
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace msa
