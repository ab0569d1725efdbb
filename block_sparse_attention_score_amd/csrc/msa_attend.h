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
// The split's selected blocks are cut into 32-token chunks that the
// workgroup's waves take round-robin, each wave with its own online softmax
// (at five blocks per split no wave streams more than three chunks, where
// 64-token chunks would give two waves of eight a second 64-token chunk);
// per chunk:
//  * S^T = K q^T on the matrix cores: K rows are read straight from the page
//    into the A operand (16 tokens x 32 dims per instruction, 64 contiguous
//    bytes per token), q^T (G heads, zero-padded to 16 columns) is the B
//    operand; v_mfma_f32_16x16x32_bf16 (fp8 codes widen to bf16 exactly) or
//    v_mfma_f32_16x16x4_f32 for f32 caches;
//  * tokens past the query are masked to -inf by select; online softmax in
//    base 2 per head column (max and sum over the lane's four tokens, then
//    across the four 16-lane rows);
//  * O^T = V^T P^T on the matrix cores: V^T is formed exactly by an MFMA of
//    the V rows against a 0/1 selector, P is rounded to bf16 by the hardware
//    pair conversion; V rows past the query are cleared first (stale bytes
//    may be NaN, and 0 * NaN would reach the sums);
//  * the next chunk's K loads are issued right after S^T and its V loads
//    right after P V (two-stage pipeline over the wave's chunks).
// The waves merge in LDS.  The split writes its normalised partial output
// and lse; the last split to finish (atomic ticket) merges the partials:
//   lse = log sum_c exp(lse_c),  out = sum_c exp(lse_c - lse) o_c.
#pragma once

#include "msa_device.h"
#include "msa_internal.h"
#include "msa_select.h"

namespace msa {

constexpr float kLn2 = 0.69314718055994530942f;
constexpr int kMaxBps = 32;  // selected blocks per split workgroup, at most
constexpr int kWaveSelectMax = 1024;  // longest row selected on one wave

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

// kGroupMajor (MX-fp6 K/V, below): step s takes dims 32 * (lane / 16) + 8 s
// .. +8 instead, the dims a lane converts from one 32-element scale group.
template <int G, bool kGroupMajor = false>
__device__ __forceinline__ void load_qfrag(const BF16*, const void* q, int64_t row0,
                                           int qrow, int kgrp, QFrag<BF16>& f) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    if (qrow < G) {
      const int d0 = kGroupMajor ? 32 * kgrp + 8 * s : 32 * s + 8 * kgrp;
      f.a[s] = *reinterpret_cast<const bf16x8_t*>(reinterpret_cast<const uint16_t*>(q) +
                                                  (row0 + qrow) * 128 + d0);
    } else {
      f.a[s] = bf16x8_t{};
    }
  }
}

template <int G, bool kGroupMajor = false>
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

// ------------------------------------------------- per-lane token rows
//
// In the MFMA tiles below a lane serves token row (lane % 16) of a 16-token
// tile and k-slot group q = lane / 16.  Row<KT> holds the elements of that
// token row the lane feeds to the matrix cores: for bf16/fp8 four 8-element
// chunks (dims 32c + 8q .. +8, c = 0..3), for f32 eight 4-element chunks
// (dims 16c + 4q .. +4, c = 0..7).  The same dims are used for K (A operand
// of S^T = K q^T) and for V (A operand of the exact 0/1 transpose below).

template <class KT>
struct Row;
template <>
struct Row<BF16> {
  bf16x8_t c[4];
};
template <>
struct Row<FP8> {
  Raw8<FP8> c[4];
};
template <>
struct Row<BF8> {
  Raw8<BF8> c[4];
};
template <>
struct Row<F32> {
  f32x4v_t c[8];
};
// MX-fp4: the four 8-code words of dims 32c + 8q .. +8 and the row's four
// scale bytes (byte c scales dims 32c .. 32c + 31).
template <>
struct Row<FP4> {
  uint32_t c[4];
  uint32_t sc;
};
// MX-fp6: the lane's whole 32-element group q (dims 32q .. 32q + 31: 24 code
// bytes) and its scale byte, converted by one instruction.  Chunk c is then
// dims 32q + 8c .. +8: the contraction runs over the dims in another order
// (the q fragment follows, load_qfrag<G, true>), and the V^T tiles come out
// with dims permuted (fp6_dim_of below).
template <>
struct Row<FP6> {
  uint32_t c[6];
  uint32_t sc;
};

__device__ __forceinline__ void load_row(const void* pool, int64_t row0, int q, Row<BF16>& r) {
#pragma unroll
  for (int c = 0; c < 4; ++c)
    r.c[c] = load8_bf16(static_cast<const BF16*>(nullptr), pool, row0 + 32 * c + 8 * q);
}
__device__ __forceinline__ void load_row(const void* pool, int64_t row0, int q, Row<FP8>& r) {
#pragma unroll
  for (int c = 0; c < 4; ++c)
    r.c[c] = load_raw(static_cast<const FP8*>(nullptr), pool, row0 + 32 * c + 8 * q);
}
__device__ __forceinline__ void load_row(const void* pool, int64_t row0, int q, Row<BF8>& r) {
#pragma unroll
  for (int c = 0; c < 4; ++c)
    r.c[c] = load_raw(static_cast<const BF8*>(nullptr), pool, row0 + 32 * c + 8 * q);
}
// row0 is the element offset (page * Hkv + g) * 128 * 128 + token * 128 that
// the other formats use; an MX-fp4 (page, head) run is kFp4Run bytes.
__device__ __forceinline__ void load_row(const void* pool, int64_t row0, int q, Row<FP4>& r) {
  const uint8_t* run = reinterpret_cast<const uint8_t*>(pool) + (row0 >> 14) * kFp4Run;
  const int tok = static_cast<int>(row0 >> 7) & 127;
#pragma unroll
  for (int c = 0; c < 4; ++c)
    r.c[c] = __builtin_nontemporal_load(
        reinterpret_cast<const uint32_t*>(run + tok * 64 + 16 * c + 4 * q));
  r.sc = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(run + kFp4Codes + tok * 4));
}
__device__ __forceinline__ bf16x8_t fp4_chunk(const Row<FP4>& r, int c) {
  return fp4x8_to_bf16x8(r.c[c], e8m0_to_f32((r.sc >> (8 * c)) & 0xffu));
}
// An MX-fp6 (page, head) run is kFp6Run bytes: the lane's group sits at
// token * 96 + 24 q (8-byte aligned), its scale at kFp6Codes + token * 4 + q.
__device__ __forceinline__ void load_row(const void* pool, int64_t row0, int q, Row<FP6>& r) {
  const uint8_t* run = reinterpret_cast<const uint8_t*>(pool) + (row0 >> 14) * kFp6Run;
  const int tok = static_cast<int>(row0 >> 7) & 127;
  const uint8_t* g = run + tok * 96 + 24 * q;
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(g + 8 * i));
    r.c[2 * i] = v[0];
    r.c[2 * i + 1] = v[1];
  }
  r.sc = __builtin_nontemporal_load(run + kFp6Codes + tok * 4 + q);
}
__device__ __forceinline__ bf16x32_t fp6_group(const Row<FP6>& r) {
  return fp6x32_to_bf16x32(r.c, e8m0_to_f32(r.sc));
}
// Dim of result row 4 q + rr of V^T tile m (MX-fp6 order): tile m takes chunk
// m / 2 of lane groups 2 (m % 2) and 2 (m % 2) + 1.
__device__ __forceinline__ int fp6_dim_of(int m, int q, int rr) {
  return 64 * (m & 1) + 32 * (q >> 1) + 8 * (m >> 1) + 4 * (q & 1) + rr;
}
__device__ __forceinline__ void load_row(const void* pool, int64_t row0, int q, Row<F32>& r) {
#pragma unroll
  for (int c = 0; c < 8; ++c)
    r.c[c] = __builtin_nontemporal_load(reinterpret_cast<const f32x4v_t*>(
        reinterpret_cast<const float*>(pool) + row0 + 16 * c + 4 * q));
}

// Rows past the query hold stale bytes (possibly NaN): zero them so that
// 0 * NaN never enters an MFMA sum.
// Clears the row when `keep` is false, without a branch: an AND with an
// all-ones or all-zero mask, so no divergent region splits the chunk loop.
template <class KT>
__device__ __forceinline__ void mask_row(Row<KT>& r, bool keep) {
  constexpr int kWords = sizeof(Row<KT>) / 4;
  uint32_t u[kWords];
  __builtin_memcpy(u, &r, sizeof(r));
  const uint32_t m = keep ? 0xffffffffu : 0u;
#pragma unroll
  for (int i = 0; i < kWords; ++i) u[i] &= m;
  __builtin_memcpy(&r, u, sizeof(r));
}

__device__ __forceinline__ bf16x8_t fp8_to_bf16x8(const Raw8<FP8>& r) {
  return fp8x8_to_bf16x8(r.v.x, r.v.y);
}
__device__ __forceinline__ bf16x8_t as_bf16(const bf16x8_t& v) { return v; }
__device__ __forceinline__ bf16x8_t as_bf16(const Raw8<FP8>& v) { return fp8_to_bf16x8(v); }
__device__ __forceinline__ bf16x8_t fp8_to_bf16x8(const Raw8<BF8>& r) {
  return bf8x8_to_bf16x8(r.v.x, r.v.y);
}
__device__ __forceinline__ bf16x8_t as_bf16(const Raw8<BF8>& v) { return fp8_to_bf16x8(v); }

// S^T tile (16 tokens x 16 heads): lane holds S^T[4q + r][lane % 16].
__device__ __forceinline__ f32x4_t st_tile(const QFrag<BF16>& qf, const Row<BF16>& k) {
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < 4; ++c) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k.c[c], qf.a[c], acc, 0, 0, 0);
  return acc;
}
template <class K8>
__device__ __forceinline__ f32x4_t st_tile(const QFrag<BF16>& qf, const Row<K8>& k) {
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < 4; ++c)
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8_to_bf16x8(k.c[c]), qf.a[c], acc, 0, 0, 0);
  return acc;
}
__device__ __forceinline__ f32x4_t st_tile(const QFrag<BF16>& qf, const Row<FP4>& k) {
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < 4; ++c)
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp4_chunk(k, c), qf.a[c], acc, 0, 0, 0);
  return acc;
}
__device__ __forceinline__ f32x4_t st_tile(const QFrag<BF16>& qf, const Row<FP6>& k) {
  const bf16x32_t kv = fp6_group(k);
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < 4; ++c)
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf16x32_part(kv, c), qf.a[c], acc, 0, 0, 0);
  return acc;
}
__device__ __forceinline__ f32x4_t st_tile(const QFrag<F32>& qf, const Row<F32>& k) {
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(k.c[c].x, qf.a[c].x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(k.c[c].y, qf.a[c].y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(k.c[c].z, qf.a[c].z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(k.c[c].w, qf.a[c].w, acc, 0, 0, 0);
  }
  return acc;
}

// Transpose of a 16-token x 16-dim V tile (dims 16m .. +16) by an MFMA with a
// 0/1 selector as the B operand: the result lane holds V[4q + r][16m + lane%16]
// for r = 0..3, exactly (one product by 1.0, the rest by 0.0, rows zeroed
// where V is stale).  `sel` is the selector of half m % 2 of a 32-dim chunk.
__device__ __forceinline__ f32x4_t vt_tile(const Row<BF16>& v, int m, const bf16x8_t (&sel)[2]) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(v.c[m >> 1], sel[m & 1], f32x4_t{0.f, 0.f, 0.f, 0.f},
                                                 0, 0, 0);
}
template <class K8>
__device__ __forceinline__ f32x4_t vt_tile(const Row<K8>& v, int m, const bf16x8_t (&sel)[2]) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8_to_bf16x8(v.c[m >> 1]), sel[m & 1],
                                                 f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t vt_tile(const Row<FP4>& v, int m, const bf16x8_t (&sel)[2]) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp4_chunk(v, m >> 1), sel[m & 1],
                                                 f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
}
// The V operand of the tiles: the stored row, or for MX-fp6 its group
// converted once to bf16 (chunk c = dims 32 q + 8 c .. +8).
template <class KT>
__device__ __forceinline__ const Row<KT>& v_operand(const Row<KT>& r) {
  return r;
}
__device__ __forceinline__ Row<BF16> v_operand(const Row<FP6>& r) {
  const bf16x32_t v = fp6_group(r);
  Row<BF16> o;
#pragma unroll
  for (int c = 0; c < 4; ++c) o.c[c] = bf16x32_part(v, c);
  return o;
}
// f32: four 16x16x4 steps; step e contracts dim 16m + 4q + e against the
// selector column (4q + e == lane % 16).
__device__ __forceinline__ f32x4_t vt_tile(const Row<F32>& v, int m, const float (&self)[4]) {
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(v.c[m].x, self[0], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(v.c[m].y, self[1], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(v.c[m].z, self[2], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(v.c[m].w, self[3], acc, 0, 0, 0);
  return acc;
}

// O^T[16m + 4q + r][head] += sum over tokens of V^T * P^T for two token tiles
// a, b.  The k-slots of lane group q are the tokens 4q + r of tile a and of
// tile b, which is where both the transposed V and P^T already sit.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
}
// Round-to-nearest-even through the hardware pair conversion (one
// v_cvt_pk_bf16_f32 on gfx950, no branch for NaN).
__device__ __forceinline__ uint32_t pack_bf16x2_rne(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v;
  v[0] = static_cast<__bf16>(lo);
  v[1] = static_cast<__bf16>(hi);
  uint32_t u;
  __builtin_memcpy(&u, &v, 4);
  return u;
}
__device__ __forceinline__ bf16x8_t pack8_exact(const f32x4_t& a, const f32x4_t& b) {
  uint32_t u[4] = {pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]),
                   pack_bf16x2(b[2], b[3])};
  bf16x8_t v;
  __builtin_memcpy(&v, u, 16);
  return v;
}
__device__ __forceinline__ bf16x8_t pack8_rne(const f32x4_t& a, const f32x4_t& b) {
  uint32_t u[4] = {pack_bf16x2_rne(a[0], a[1]), pack_bf16x2_rne(a[2], a[3]),
                   pack_bf16x2_rne(b[0], b[1]), pack_bf16x2_rne(b[2], b[3])};
  bf16x8_t v;
  __builtin_memcpy(&v, u, 16);
  return v;
}

__device__ __forceinline__ void store_out(const BF16*, void* out, int64_t idx, float v) {
  reinterpret_cast<uint16_t*>(out)[idx] = f32_to_bf16(v);
}
__device__ __forceinline__ void store_out(const F32*, void* out, int64_t idx, float v) {
  reinterpret_cast<float*>(out)[idx] = v;
}

// 2^x on the hardware instruction: 2^-inf = 0, results below 2^-126 flush
// to zero (probabilities that small change neither a bf16 P nor an f32 sum).
__device__ __forceinline__ float exp2_raw(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------- split unit

// Row stride of the per-wave partial outputs in LDS: 132 floats (528 bytes)
// put the 16 head rows of one 16-byte store pass on 16 distinct groups of
// four banks; at 128 floats every row of the pass would hit the same banks.
constexpr int kOStride = kBlock + 4;

template <int G, int W>
struct AttendLds {
  alignas(16) float o[W][16][kOStride];  // per-wave partial outputs, [head][dim]
  float m[W][16];          // per-wave running max (base 2, scaled logits)
  float l[W][16];          // per-wave running sum
  float m_all[16];
  float l_all[16];
  int blk_nvalid[kMaxBps];
  int blk_page[kMaxBps];
  int blk_j[kMaxBps];      // block ids of the split (selection inside the kernel)
  int row_page[kWaveSelectMax];  // the row's block-table entries (one-wave selections)
  int is_last;
  SelectLds sl;
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
// Called by all 64 * W threads (W waves) of a workgroup.
template <class QT, class KT, int G, int W>
__device__ void attend_split(const AttendArgs& a, int split, int g, int t, AttendLds<G, W>& S) {
  constexpr int kThreads = kWave * W;
  const int h = g / (a.hkv / a.hidx);
  const int sel_row = t * a.hidx + h;
  const bool self_select = a.scores != nullptr;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int w = tid / kWave;
  // Rows of at most kWaveSelectMax blocks are selected on wave 0.  Their
  // scores (wave 0) and block-table entries (the other waves, into LDS) are
  // fetched over the whole max_blocks row before the sequence length is
  // known, so that neither waits for it; slots past the row are ignored.
  static_assert(W >= 2, "waves 1.. stage the block table");
  const bool wave_rows = self_select && a.max_blocks > 0 && a.max_blocks <= kWaveSelectMax;
  float sv[16];
  if (wave_rows && w == 0) {
    const float* srow = a.scores + static_cast<int64_t>(sel_row) * a.max_blocks;
    if (a.max_blocks <= 256) {
#pragma unroll
      for (int e = 0; e < 4; ++e) sv[e] = srow[min(lane + kWave * e, a.max_blocks - 1)];
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) sv[e] = srow[min(lane + kWave * e, a.max_blocks - 1)];
    }
  }
  int b, p;
  query_of(a, t, b, p);
  if (wave_rows && w > 0) {
    const int* bt = a.block_table + static_cast<int64_t>(b) * a.max_blocks;
    for (int j = tid - kWave; j < a.max_blocks; j += kThreads - kWave) S.row_page[j] = bt[j];
  }
  // Blocks visible to the query, and the selection size that follows from
  // them alone (init and local blocks plus min(topk, rest)).
  const int nb_vis = p >= 0 ? min(p / kBlock + 1, a.max_blocks) : 0;
  int count;
  const int topk_row = topk_beside_forced(a.topk, nb_vis, a.init, a.local, a.forced_in_budget);
  if (self_select) {
    const int nf = forced_count(nb_vis, a.init, a.local);
    count = nf + min(topk_row, nb_vis - nf);
  } else {
    const int cnt_raw = a.cnt[sel_row];
    count = p >= 0 ? min(max(cnt_raw, 0), a.kmax) : 0;
  }
  const int nsplit = div_up(count, a.bps);
  // The writer of the selection outputs: split 0 of the first kv head of
  // the index head.
  const bool sel_writer = self_select && a.sel_out != nullptr && split == 0 &&
                          g % (a.hkv / a.hidx) == 0;
  const int64_t hq0 = static_cast<int64_t>(t) * a.hkv * G + static_cast<int64_t>(g) * G;
  const QT* qtag = nullptr;

  // Index-value branch (decode): split 0 of the first kv head of each index
  // head merges the scan's chunk partials of its row into idx_out,
  //   out = sum_c 2^(m_c - M) o_c / sum_c 2^(m_c - M) l_c,
  // zeros for a row with nothing visible.
  if (a.iv_part != nullptr && split == 0 && g % (a.hkv / a.hidx) == 0) {
    const int di = a.idx_dim;
    const int nch = div_up(nb_vis, a.iv_pages);
    const float* part = a.iv_part + static_cast<int64_t>(sel_row) * a.iv_chunks * (di + 2);
    for (int d = tid; d < di; d += kThreads) {
      float M = -INFINITY;
      for (int c = 0; c < nch; ++c) M = fmaxf(M, part[c * (di + 2) + di]);
      float lsum = 0.f, o = 0.f;
      if (M != -INFINITY) {
        for (int c = 0; c < nch; ++c) {
          const float* pc = part + c * (di + 2);
          const float wgt = __builtin_amdgcn_exp2f(pc[di] - M);
          lsum = fmaf(wgt, pc[di + 1], lsum);
          o = fmaf(wgt, pc[d], o);
        }
      }
      store_out(qtag, a.idx_out, static_cast<int64_t>(sel_row) * di + d, lsum > 0.f ? o / lsum : 0.f);
    }
  }
  if (sel_writer && count == 0) {
    for (int i = threadIdx.x; i < a.kmax; i += kThreads)
      a.sel_out[static_cast<int64_t>(sel_row) * a.kmax + i] = -1;
    if (threadIdx.x == 0) a.cnt_out[sel_row] = 0;
  }
  if (count == 0) {
    if (split == 0) {
      for (int i = tid; i < G * 128; i += kThreads) store_out(qtag, a.out, hq0 * 128 + i, 0.f);
      if (a.lse_out != nullptr && tid < G) a.lse_out[hq0 + tid] = -INFINITY;
    }
    return;
  }
  if (split >= nsplit) return;

  const int l16 = lane & 15;  // token row (MFMA A rows) / head column (B, D columns)
  const int q4 = lane >> 4;   // k-slot group; D rows 4*q4 .. +3

  // q^T as the B operand of S^T = K q^T (heads past G are zero columns).
  constexpr bool kGroupMajor = __is_same(KT, FP6);
  QFrag<QT> qf;
  load_qfrag<G, kGroupMajor>(qtag, a.q, hq0, l16, q4, qf);

  // Block ids and pages of this split (at most kMaxBps), resolved up front.
  const int bi0 = split * a.bps;
  const int nblk = min(count, bi0 + a.bps) - bi0;
  if (self_select) {
    // Every split of the row runs the same selection; each keeps its slots.
    int32_t* so = sel_writer ? a.sel_out + static_cast<int64_t>(sel_row) * a.kmax : nullptr;
    const float* srow = a.scores + static_cast<int64_t>(sel_row) * a.max_blocks;
    auto emit = [&](int pos, int j) {
      if (pos >= bi0 && pos < bi0 + nblk) S.blk_j[pos - bi0] = j;
      if (sel_writer) so[pos] = j;
    };
    // One wave selects rows of up to 1024 blocks; longer rows take the
    // workgroup radix select.
    if (wave_rows) {
      if (w == 0) {
        if (nb_vis <= 256) {
          float v4[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = sv[e];
          select_wave_loaded<4>(v4, nb_vis, topk_row, a.init, a.local, emit);
        } else {
          select_wave_loaded<16>(sv, nb_vis, topk_row, a.init, a.local, emit);
        }
      }
    } else if (nb_vis <= 256) {
      if (w == 0) select_wave<4>(srow, nb_vis, topk_row, a.init, a.local, emit);
    } else if (nb_vis <= kWaveSelectMax) {
      if (w == 0) select_wave<16>(srow, nb_vis, topk_row, a.init, a.local, emit);
    } else {
      select_core<div_up(8192, kThreads), kThreads>(srow, nb_vis, topk_row, a.init, a.local, S.sl,
                                                     emit);
    }
    if (sel_writer) {
      for (int i = count + tid; i < a.kmax; i += kThreads) so[i] = -1;
      if (tid == 0) a.cnt_out[sel_row] = count;
    }
    __syncthreads();
  }
  if (tid < nblk) {
    const int64_t at = static_cast<int64_t>(sel_row) * a.kmax + bi0 + tid;
    const int j = self_select ? S.blk_j[tid] : a.sel[at];
    const int page = j >= 0 && j < a.max_blocks
                         ? (wave_rows ? S.row_page[j]
                                      : a.block_table[static_cast<int64_t>(b) * a.max_blocks + j])
                         : -1;
    const bool ok = page >= 0 && page < a.num_pages && j >= 0;
    S.blk_nvalid[tid] = ok ? max(0, min(kBlock, p + 1 - j * kBlock)) : 0;
    S.blk_page[tid] = ok ? page : 0;
  }
  __syncthreads();

  // The split's blocks are cut into chunks of TILES 16-token tiles, and wave w
  // streams chunks w, w+W, ... (so a split whose block count is not a multiple
  // of W still spreads evenly), with its own online softmax; no barrier until
  // the final merge.
  constexpr bool kF32 = __is_same(KT, F32);
  constexpr int TILES = 2;                      // tiles per chunk
  constexpr int CPB = 8 / TILES;                // chunks per 128-token block
  const int nchunk = nblk * CPB > w ? (nblk * CPB - w + W - 1) / W : 0;

  // 0/1 selectors for the V transpose.
  bf16x8_t sel_bf[2];
  float sel_f[4];
  {
    uint16_t e0[8], e1[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      e0[e] = (8 * q4 + e == l16) ? 0x3F80 : 0;
      e1[e] = (8 * q4 + e == 16 + l16) ? 0x3F80 : 0;
    }
    __builtin_memcpy(&sel_bf[0], e0, 16);
    __builtin_memcpy(&sel_bf[1], e1, 16);
#pragma unroll
    for (int e = 0; e < 4; ++e) sel_f[e] = (4 * q4 + e == l16) ? 1.f : 0.f;
  }

  auto chunk_block = [&](int c) { return (w + W * c) / CPB; };
  auto chunk_tok0 = [&](int c) { return ((w + W * c) % CPB) * TILES * 16; };
  auto row0 = [&](int c, int tt) {
    const int blk = chunk_block(c);
    const int tok = chunk_tok0(c) + 16 * tt + l16;
    return (static_cast<int64_t>(S.blk_page[blk]) * a.hkv + g) * kBlock * 128 +
           static_cast<int64_t>(tok) * 128;
  };
  auto tok_valid = [&](int c, int tt) {
    return chunk_tok0(c) + 16 * tt + l16 < S.blk_nvalid[chunk_block(c)];
  };

  Row<KT> kr[TILES], vr[TILES];
  if (nchunk > 0) {
#pragma unroll
    for (int tt = 0; tt < TILES; ++tt) load_row(a.k_pool, row0(0, tt), q4, kr[tt]);
#pragma unroll
    for (int tt = 0; tt < TILES; ++tt) load_row(a.v_pool, row0(0, tt), q4, vr[tt]);
  }
  float m_run = -INFINITY, l_run = 0.f;  // for head column l16
  f32x4_t acc[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) acc[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // One chunk: S^T, online softmax, O^T += V^T P^T.  The loads of the next
  // chunk are issued between the stages (K after S^T, V after P V); the loop
  // below runs all chunks but the last with `next` set and then the last one
  // without, so every load inside the loop is unconditional and the waits
  // before S^T and before P V cover only the loads they need.
  auto chunk = [&](int c, bool next) {
    const int nvalid = S.blk_nvalid[chunk_block(c)];
    const int tok0 = chunk_tok0(c);
    f32x4_t st[TILES];
#pragma unroll
    for (int tt = 0; tt < TILES; ++tt) {
      st[tt] = st_tile(qf, kr[tt]);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        st[tt][r] = tok0 + 16 * tt + 4 * q4 + r < nvalid ? st[tt][r] * a.qk_scale_log2 : -INFINITY;
    }
    if (next) {
#pragma unroll
      for (int tt = 0; tt < TILES; ++tt) load_row(a.k_pool, row0(c + 1, tt), q4, kr[tt]);
    }
    float mc = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < TILES; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r) mc = fmaxf(mc, st[tt][r]);
    mc = fmaxf(mc, __shfl_xor(mc, 16));
    mc = fmaxf(mc, __shfl_xor(mc, 32));
    const float mn = fmaxf(m_run, mc);
    // a column with nothing visible yet keeps m = -inf; its p are 2^-inf = 0
    const float mu = mn == -INFINITY ? 0.f : mn;
    const float alpha = exp2_raw(m_run - mu);
    float ls = 0.f;
#pragma unroll
    for (int tt = 0; tt < TILES; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        st[tt][r] = exp2_raw(st[tt][r] - mu);
        ls += st[tt][r];
      }
    ls += __shfl_xor(ls, 16);
    ls += __shfl_xor(ls, 32);
    l_run = l_run * alpha + ls;
    m_run = mn;
#pragma unroll
    for (int m = 0; m < 8; ++m) acc[m] *= alpha;
#pragma unroll
    for (int tt = 0; tt < TILES; ++tt)
      mask_row(vr[tt], tok_valid(c, tt));
    if constexpr (kF32) {
#pragma unroll
      for (int m = 0; m < 8; ++m) {
#pragma unroll
        for (int tt = 0; tt < TILES; ++tt) {
          const f32x4_t vt = vt_tile(vr[tt], m, sel_f);
#pragma unroll
          for (int r = 0; r < 4; ++r)
            acc[m] = __builtin_amdgcn_mfma_f32_16x16x4f32(vt[r], st[tt][r], acc[m], 0, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int tp = 0; tp < TILES; tp += 2) {
        const bf16x8_t pb = pack8_rne(st[tp], st[tp + 1]);
        const auto v0 = v_operand(vr[tp]);
        const auto v1 = v_operand(vr[tp + 1]);
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const f32x4_t va = vt_tile(v0, m, sel_bf);
          const f32x4_t vb = vt_tile(v1, m, sel_bf);
          acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pack8_exact(va, vb), pb, acc[m], 0, 0, 0);
        }
      }
    }
    if (next) {
#pragma unroll
      for (int tt = 0; tt < TILES; ++tt) load_row(a.v_pool, row0(c + 1, tt), q4, vr[tt]);
    }
  };
  for (int c = 0; c + 1 < nchunk; ++c) chunk(c, true);
  if (nchunk > 0) chunk(nchunk - 1, false);

  // Merge the waves: lane (l16, q4) holds O^T[16m + 4q4 + r][head l16]
  // (MX-fp6: O^T[fp6_dim_of(m, q4, r)][head l16]), four consecutive dims per
  // m, stored as one 16-byte write.
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const int d0 = kGroupMajor ? fp6_dim_of(m, q4, 0) : 16 * m + 4 * q4;
    *reinterpret_cast<f32x4_t*>(&S.o[w][l16][d0]) = acc[m];
  }
  if (q4 == 0) {
    S.m[w][l16] = m_run;
    S.l[w][l16] = l_run;
  }
  __syncthreads();
  if (tid < 16) {
    float M = S.m[0][tid];
#pragma unroll
    for (int ww = 1; ww < W; ++ww) M = fmaxf(M, S.m[ww][tid]);
    float lsum = 0.f;
#pragma unroll
    for (int ww = 0; ww < W; ++ww) {
      const float sc = S.m[ww][tid] == -INFINITY ? 0.f : exp2f(S.m[ww][tid] - M);
      S.m[ww][tid] = sc;  // becomes the wave's weight
      lsum += S.l[ww][tid] * sc;
    }
    S.m_all[tid] = M;
    S.l_all[tid] = lsum;
  }
  __syncthreads();

  const int64_t part0 =
      ((static_cast<int64_t>(t) * a.hkv + g) * a.nsplit_max + split) * G;
  for (int i = tid; i < G * 128; i += kThreads) {
    const int hh = i / 128;
    const int d = i % 128;
    const float l = S.l_all[hh];
    float o = 0.f;
    if (l > 0.f) {
#pragma unroll
      for (int ww = 0; ww < W; ++ww) o = fmaf(S.o[ww][hh][d], S.m[ww][hh], o);
      o *= a.v_scale / l;
    }
    if (nsplit == 1) {
      store_out(qtag, a.out, (hq0 + hh) * 128 + d, o);
    } else {
      store_shared_f32(a.part_o + (part0 + hh) * 128 + d, o);
    }
  }
  if (tid < G) {
    const float lse = S.l_all[tid] > 0.f ? (S.m_all[tid] + log2f(S.l_all[tid])) * kLn2 : -INFINITY;
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
  if (nsplit <= 8) {
    // One round trip: every thread loads the lse and the partial of each
    // split for its (head, dim) and weights them itself.  Slots past the last
    // split re-read it and get weight 0.
    for (int i = tid; i < G * 128; i += kThreads) {
      const int hh = i / 128;
      const int d = i % 128;
      float ls[8], v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int c = min(u, nsplit - 1);
        ls[u] = load_shared_f32(a.part_lse + base0 + c * G + hh);
        v[u] = load_shared_f32(a.part_o + (base0 + c * G + hh) * 128 + d);
      }
      float mx = -INFINITY;
#pragma unroll
      for (int u = 0; u < 8; ++u) mx = fmaxf(mx, u < nsplit ? ls[u] : -INFINITY);
      float ws = 0.f, o = 0.f;
      if (mx != -INFINITY) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float e = u < nsplit ? __expf(ls[u] - mx) : 0.f;
          ws += e;
          o = fmaf(e, v[u], o);
        }
      }
      store_out(qtag, a.out, (hq0 + hh) * 128 + d, ws > 0.f ? o / ws : 0.f);
      if (d == 0 && a.lse_out != nullptr)
        a.lse_out[hq0 + hh] = ws > 0.f ? mx + __logf(ws) : -INFINITY;
    }
    return;
  }
  // Split weights exp(lse_c - lse) of every head, once, in LDS (the partial
  // lse values are loaded by many threads at once).
  float* w_lds = &S.o[0][0][0];  // reused: nsplit_max * G <= W * 16 * 128 floats
  for (int i = tid; i < nsplit * G; i += kThreads) w_lds[i] = load_shared_f32(a.part_lse + base0 + i);
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
  for (int i = tid; i < G * 128; i += kThreads) {
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
