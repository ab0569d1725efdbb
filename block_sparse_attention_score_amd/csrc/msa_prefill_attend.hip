// Chunked-prefill attention, key-major.
//
// Selection is per query token (sglang page minimax_sparse_backend.py,
// MiniMaxSparseAttnBackend.__init__: one query per selection block), so in a
// prefill chunk every key block j of a sequence is attended by the tokens
// that selected it.  The SM100 prefill page (minimax_sparse.py,
// minimax_sparse_prefill) builds, per (sequence, head, key block), the list of
// those tokens and runs key-major attention tiles over it; this file does the
// same on gfx950:
//   1. k2q CSR: count the selecting tokens of every (b, index head, j), scan
//      the counts into list offsets and 128-row work tiles, fill the lists;
//   2. one workgroup per tile: up to 128 query rows (tokens x GQA heads of one
//      kv head) against block j, staged once in LDS (K as [key][dim], V as
//      [dim][key]); S^T = K Q^T and O^T = V^T P^T on bf16 MFMA, causal mask
//      per row; a normalised partial (o in bf16, lse in f32) per (token, kv
//      head, slot);
//   3. per (token, kv head), the log-sum-exp combine of its partials.
#include "msa_device.h"
#include "msa_internal.h"

namespace msa {

namespace {

constexpr int kRows = 128;       // query rows (token x head) per tile
constexpr int kStride = 136;     // LDS row stride in bf16 elements (128 + 8)
constexpr float kLn2f = 0.69314718055994531f;

struct PfLds {
  uint16_t k[kBlock * kStride];   // K   [key][dim]
  uint16_t vt[kBlock * kStride];  // V^T [dim][key]
  int tok[kRows];                 // token of each token slot of the tile (-1: none)
  int slot[kRows];                // its slot in the token's selection
  int pos[kRows];                 // its position in the sequence
};

__device__ __forceinline__ bf16x8_t lds_b128(const uint16_t* p) {
  bf16x8_t r;
  __builtin_memcpy(&r, p, 16);
  return r;
}

// Eight consecutive K/V elements as bf16, through the caches (a key block is
// read by every tile of its list).
__device__ __forceinline__ bf16x8_t load8_cached(const BF16*, const void* base, int64_t idx) {
  bf16x8_t r;
  __builtin_memcpy(&r, reinterpret_cast<const uint16_t*>(base) + idx, 16);
  return r;
}
__device__ __forceinline__ bf16x8_t load8_cached(const FP8*, const void* base, int64_t idx) {
  uint2 raw;
  __builtin_memcpy(&raw, reinterpret_cast<const uint8_t*>(base) + idx, 8);
  float x[8];
  fp8x4_to_f32(raw.x, x);
  fp8x4_to_f32(raw.y, x + 4);
  uint32_t u[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    u[i] = (__float_as_uint(x[2 * i]) >> 16) | (__float_as_uint(x[2 * i + 1]) & 0xffff0000u);
  bf16x8_t r;
  __builtin_memcpy(&r, u, 16);
  return r;
}

__device__ __forceinline__ uint32_t pack2_rne(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v;
  v[0] = static_cast<__bf16>(lo);
  v[1] = static_cast<__bf16>(hi);
  uint32_t u;
  __builtin_memcpy(&u, &v, 4);
  return u;
}

}  // namespace

// ---------------------------------------------------------------- k2q CSR

// Workgroup (chunk c, sequence b, index head h): the 256 tokens
// cu[b] + 256 c + tid count their selected blocks in an LDS histogram of the
// sequence's max_blocks bins, then add the non-zero bins to the lists' counts
// (the forced blocks are shared by every token: one global atomic per bin).
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
    for (int s = 0; s < n; ++s) {
      const int j = a.sel[static_cast<int64_t>(row) * a.kmax + s];
      if (j >= 0 && j < a.max_blocks) atomicAdd(&hist[j], 1);
    }
  }
  __syncthreads();
  int32_t* c = a.counts + (static_cast<int64_t>(b) * a.hidx + h) * a.max_blocks;
  for (int i = tid; i < a.max_blocks; i += kWgThreads)
    if (hist[i] > 0) atomicAdd(c + i, hist[i]);
}

// One workgroup: exclusive scans of the counts (list offsets) and of the
// tiles per list (work-item offsets), then the work items themselves.
__global__ __launch_bounds__(1024) void k2q_scan_kernel(PrefillAttnArgs a, int n) {
  __shared__ int wsum[16];
  const int tid = threadIdx.x;
  const int per = (n + 1023) / 1024;
  const int i0 = min(tid * per, n);
  const int i1 = min(i0 + per, n);
  int sc = 0, st = 0;
  for (int i = i0; i < i1; ++i) {
    const int c = a.counts[i];
    sc += c;
    st += (c + a.tq - 1) / a.tq;
  }
  int ec = block_incl_scan(sc, wsum) - sc;
  int et = block_incl_scan(st, wsum) - st;
  for (int i = i0; i < i1; ++i) {
    const int c = a.counts[i];
    const int nt = (c + a.tq - 1) / a.tq;
    a.tok_off[i] = ec;
    for (int k = 0; k < nt; ++k)
      if (et + k < a.max_items) a.items[et + k] = make_int4(i, ec + k * a.tq, min(a.tq, c - k * a.tq), 0);
    ec += c;
    et += nt;
  }
  if (tid == 1023) *a.n_items = min(et, a.max_items);
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
  for (int s = 0; s < n; ++s) {
    const int j = a.sel[static_cast<int64_t>(row) * a.kmax + s];
    if (j >= 0 && j < a.max_blocks) atomicAdd(&hist[j], 1);
  }
  __syncthreads();
  const int64_t bh0 = (static_cast<int64_t>(b) * a.hidx + h) * a.max_blocks;
  for (int i = tid; i < a.max_blocks; i += kWgThreads)
    if (hist[i] > 0) hist[i] = a.tok_off[bh0 + i] + atomicAdd(a.cursor + bh0 + i, hist[i]);
  __syncthreads();
  for (int s = 0; s < n; ++s) {
    const int j = a.sel[static_cast<int64_t>(row) * a.kmax + s];
    if (j < 0 || j >= a.max_blocks) continue;
    a.csr[atomicAdd(&hist[j], 1)] = (t << 8) | s;
  }
}

// ------------------------------------------------------------ attention tile

template <class KT, int G>
__global__ __launch_bounds__(kWgThreads, 2) void prefill_attend_kernel(PrefillAttnArgs a) {
  __shared__ PfLds S;
  constexpr int TQ = kRows / G;  // tokens per tile
  const KT* ktag = nullptr;
  // Work item: tiles of one key block are consecutive; spread them so that
  // each XCD (workgroups x, x + 8, ...) takes a contiguous range and its L2
  // serves the block to all of them.
  const int total = *a.n_items;
  const int per = (total + 7) / 8;
  const int x = blockIdx.x;
  if (x / 8 >= per) return;
  const int item = (x % 8) * per + x / 8;
  if (item >= total) return;
  const int4 it = a.items[item];
  const int bhj = it.x;
  const int c0 = it.y;    // first list entry of the tile
  const int ntok = it.z;  // tokens in the tile
  const int j = bhj % a.max_blocks;
  const int bh = bhj / a.max_blocks;
  const int h = bh % a.hidx;
  const int b = bh / a.hidx;
  const int g = h * (a.hkv / a.hidx) + blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int w = tid / kWave;
  const int l16 = lane & 15;
  const int q4 = lane >> 4;

  const int L = a.seq_lens[b];
  const int cu0 = a.cu_seqlens_q[b];
  const int p0 = L - (a.cu_seqlens_q[b + 1] - cu0) - cu0;  // position of token t: p0 + t
  // Query rows of this wave: 32 w + 16 nt + l16 = token slot * G + head.
  // Their loads go out first, to overlap with the staging of the block.
  const int hq_stride = a.hkv * G;
  bf16x8_t qf[2][4];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int r = 32 * w + 16 * nt + l16;
    const int ts = r / G;
    const int hh = r - ts * G;
    const int t = ts < ntok ? (a.csr[c0 + ts] >> 8) : -1;
    const int64_t q0 = (static_cast<int64_t>(t) * hq_stride + g * G + hh) * 128 + 8 * q4;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qf[nt][ks] = t >= 0 ? load8_cached(static_cast<const BF16*>(nullptr), a.q, q0 + 32 * ks)
                          : bf16x8_t{};
  }
  if (tid < TQ) {
    if (tid < ntok) {
      const int e = a.csr[c0 + tid];
      S.tok[tid] = e >> 8;
      S.slot[tid] = e & 255;
      S.pos[tid] = p0 + (e >> 8);
    } else {
      S.tok[tid] = -1;
      S.slot[tid] = 0;
      S.pos[tid] = -1;
    }
  }
  const int page = a.block_table[static_cast<int64_t>(b) * a.max_blocks + j];
  const bool page_ok = page >= 0 && page < a.num_pages;
  // keys at or past the sequence end hold stale bytes: staged as zeros
  const int nvalid = page_ok ? max(0, min(kBlock, L - j * kBlock)) : 0;
  const int64_t head0 = (static_cast<int64_t>(page_ok ? page : 0) * a.hkv + g) * kBlock * 128;

  // K rows: instruction i of thread tid reads key 16 i + tid / 16, dims
  // 8 (tid % 16) .. + 8 (full 256-byte rows per 16 lanes).
  {
    const int kr = tid >> 4;
    const int dc = (tid & 15) * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int key = 16 * i + kr;
      bf16x8_t v = bf16x8_t{};
      if (key < nvalid) v = load8_cached(ktag, a.k_pool, head0 + key * 128 + dc);
      __builtin_memcpy(&S.k[key * kStride + dc], &v, 16);
    }
  }
  // V transposed: thread tid reads keys 64 hf + 4 (tid / 16) + kk, dims
  // 8 (tid % 16) .. + 8, and writes each dim's four consecutive keys at once.
  {
    const int kq = tid >> 4;
    const int dc = (tid & 15) * 8;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      uint16_t v[4][8];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int key = 64 * hf + 4 * kq + kk;
        bf16x8_t x = bf16x8_t{};
        if (key < nvalid) x = load8_cached(ktag, a.v_pool, head0 + key * 128 + dc);
        __builtin_memcpy(&v[kk][0], &x, 16);
      }
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const uint32_t w0 = static_cast<uint32_t>(v[0][d]) | (static_cast<uint32_t>(v[1][d]) << 16);
        const uint32_t w1 = static_cast<uint32_t>(v[2][d]) | (static_cast<uint32_t>(v[3][d]) << 16);
        const u32x2_t pr = {w0, w1};
        __builtin_memcpy(&S.vt[(dc + d) * kStride + 64 * hf + 4 * kq], &pr, 8);
      }
    }
  }
  __syncthreads();

  int rpos[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) rpos[nt] = S.pos[(32 * w + 16 * nt + l16) / G];

  // S^T tiles: keys 16 mt + 4 q4 + r (rows), query rows 16 nt + l16 (columns).
  f32x4_t st[8][2];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) {
    st[mt][0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    st[mt][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8_t kf = lds_b128(&S.k[(16 * mt + l16) * kStride + 32 * ks + 8 * q4]);
      st[mt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[0][ks], st[mt][0], 0, 0, 0);
      st[mt][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[1][ks], st[mt][1], 0, 0, 0);
    }
  }

  // Softmax of each query row over the block's visible keys (base 2).
  const int tok0 = j * kBlock;
  float mrow[2], lrow[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    float m = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = 16 * mt + 4 * q4 + r;
        const bool ok = key < nvalid && tok0 + key <= rpos[nt];
        const float s = ok ? st[mt][nt][r] * a.qk_scale_log2 : -INFINITY;
        st[mt][nt][r] = s;
        m = fmaxf(m, s);
      }
    m = fmaxf(m, __shfl_xor(m, 16));
    m = fmaxf(m, __shfl_xor(m, 32));
    float l = 0.f;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float s = st[mt][nt][r];
        const float e = s == -INFINITY ? 0.f : exp2f(s - m);
        st[mt][nt][r] = e;
        l += e;
      }
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    mrow[nt] = m;
    lrow[nt] = l;
  }

  // O^T = V^T P^T: dims 16 dt + 4 q4 + r (rows), query rows 16 nt + l16.
  // k-slots e of a 32-key step kk: keys 32 kk + 4 q4 + e (e < 4) and
  // 32 kk + 16 + 4 q4 + (e - 4), the keys the S^T tiles 2 kk, 2 kk + 1 hold.
  f32x4_t o[8][2];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    o[dt][0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    o[dt][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
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
      const uint16_t* row = &S.vt[(16 * dt + l16) * kStride + 32 * kk + 4 * q4];
      u32x2_t lo, hi;
      __builtin_memcpy(&lo, row, 8);
      __builtin_memcpy(&hi, row + 16, 8);
      const u32x4_t cat = {lo[0], lo[1], hi[0], hi[1]};
      bf16x8_t vf;
      __builtin_memcpy(&vf, &cat, 16);
      o[dt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb[0], o[dt][0], 0, 0, 0);
      o[dt][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb[1], o[dt][1], 0, 0, 0);
    }
  }

  // Normalised partial and its log-sum-exp (natural log of the scaled logits).
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int r = 32 * w + 16 * nt + l16;
    const int ts = r / G;
    const int hh = r - ts * G;
    const int t = S.tok[ts];
    if (t < 0) continue;
    const float l = lrow[nt];
    const float inv = l > 0.f ? a.v_scale / l : 0.f;
    const int64_t base =
        ((static_cast<int64_t>(t) * a.hkv + g) * a.kmax + S.slot[ts]) * G + hh;
    uint16_t* po = a.part_o + base * 128 + 4 * q4;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const u32x2_t v = {pack2_rne(o[dt][nt][0] * inv, o[dt][nt][1] * inv),
                         pack2_rne(o[dt][nt][2] * inv, o[dt][nt][3] * inv)};
      *reinterpret_cast<u32x2_t*>(po + 16 * dt) = v;
    }
    if (q4 == 0)
      a.part_lse[base] = l > 0.f ? (mrow[nt] + log2f(l)) * kLn2f : -INFINITY;
  }
}

// ---------------------------------------------------------------- combine

// One workgroup per (token, kv head): out = sum_s exp(lse_s - lse) o_s.
template <int G>
__global__ __launch_bounds__(kWgThreads) void prefill_combine_kernel(PrefillAttnArgs a) {
  __shared__ float wgt[kMaxSelect * G];
  const int t = blockIdx.x;
  const int g = blockIdx.y;
  const int h = g / (a.hkv / a.hidx);
  const int tid = threadIdx.x;
  const int n = min(max(a.cnt[t * a.hidx + h], 0), a.kmax);
  const int64_t base = (static_cast<int64_t>(t) * a.hkv + g) * a.kmax * G;  // slot 0, head 0
  const int64_t out0 = (static_cast<int64_t>(t) * a.hkv + g) * G;           // q head row
  for (int i = tid; i < n * G; i += kWgThreads) wgt[i] = a.part_lse[base + i];
  __syncthreads();
  if (tid < G) {
    float mx = -INFINITY;
    for (int s = 0; s < n; ++s) mx = fmaxf(mx, wgt[s * G + tid]);
    float sum = 0.f;
    if (mx != -INFINITY)
      for (int s = 0; s < n; ++s) sum += __expf(wgt[s * G + tid] - mx);
    const float inv = sum > 0.f ? 1.f / sum : 0.f;
    for (int s = 0; s < n; ++s)
      wgt[s * G + tid] = mx != -INFINITY ? __expf(wgt[s * G + tid] - mx) * inv : 0.f;
    if (a.lse_out != nullptr) a.lse_out[out0 + tid] = sum > 0.f ? mx + __logf(sum) : -INFINITY;
  }
  __syncthreads();
  // Thread i: head i / 32, dims 4 (i % 32) .. + 4 (one 8-byte load per slot).
  for (int i = tid; i < G * 32; i += kWgThreads) {
    const int hh = i / 32;
    const int d = 4 * (i - hh * 32);
    const uint16_t* po = a.part_o + (base + hh) * 128 + d;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < n; s0 += 8) {
      // straight-line batch: slots past the last re-read it with weight 0
      u32x2_t v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        v[u] = *reinterpret_cast<const u32x2_t*>(
            po + static_cast<int64_t>(min(s0 + u, n - 1)) * G * 128);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float wv = s0 + u < n ? wgt[(s0 + u) * G + hh] : 0.f;
        acc[0] = fmaf(wv, __uint_as_float(v[u][0] << 16), acc[0]);
        acc[1] = fmaf(wv, __uint_as_float(v[u][0] & 0xffff0000u), acc[1]);
        acc[2] = fmaf(wv, __uint_as_float(v[u][1] << 16), acc[2]);
        acc[3] = fmaf(wv, __uint_as_float(v[u][1] & 0xffff0000u), acc[3]);
      }
    }
    const u32x2_t r = {pack2_rne(acc[0], acc[1]), pack2_rne(acc[2], acc[3])};
    *reinterpret_cast<u32x2_t*>(reinterpret_cast<uint16_t*>(a.out) + (out0 + hh) * 128 + d) = r;
  }
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

template <class KT>
static bool launch_pf_attend_g(const PrefillAttnArgs& a, int group, hipStream_t s) {
  const dim3 grid(a.max_items, a.hkv / a.hidx);
  switch (group) {
    case 1: prefill_attend_kernel<KT, 1><<<grid, kWgThreads, 0, s>>>(a); return true;
    case 2: prefill_attend_kernel<KT, 2><<<grid, kWgThreads, 0, s>>>(a); return true;
    case 4: prefill_attend_kernel<KT, 4><<<grid, kWgThreads, 0, s>>>(a); return true;
    case 8: prefill_attend_kernel<KT, 8><<<grid, kWgThreads, 0, s>>>(a); return true;
    case 16: prefill_attend_kernel<KT, 16><<<grid, kWgThreads, 0, s>>>(a); return true;
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
    if (!ok) return hipErrorInvalidValue;
  }
  const dim3 cgrid(a.num_tokens, a.hkv);
  switch (group) {
    case 1: prefill_combine_kernel<1><<<cgrid, kWgThreads, 0, s>>>(a); break;
    case 2: prefill_combine_kernel<2><<<cgrid, kWgThreads, 0, s>>>(a); break;
    case 4: prefill_combine_kernel<4><<<cgrid, kWgThreads, 0, s>>>(a); break;
    case 8: prefill_combine_kernel<8><<<cgrid, kWgThreads, 0, s>>>(a); break;
    case 16: prefill_combine_kernel<16><<<cgrid, kWgThreads, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace msa
