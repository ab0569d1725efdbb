// Chunked prefill, index-value branch: causal softmax attention of every new
// token's index query over the index keys and index values of its sequence.
//
// The sglang page minimax_sparse_backend.py (forward_extend) hands the
// index-value cache to the prefill op beside the index keys, unless the layer
// disables the value branch, and returns an index output idx_o of
// num_idx_heads * sparse_index_dim values per token; the attention of each
// index query over every visible token's index key and value, with the scale
// 1/sqrt(Di), is the reading taken (the op's body is not on the pages).
//
// Work is split as the index scoring is: a workgroup takes 256 query rows of
// one (sequence, index head) and a run of key blocks, so long prefixes spread
// over many workgroups.  Eight waves own 32 query rows each (index queries in
// registers as B operands); each key block is staged once in LDS (K as
// [key][dim], V transposed to [dim][key], double-buffered) and every wave
// computes S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_16x16x32_bf16 with an
// online softmax (base 2) per query row over the run's blocks.  The run's
// normalised partial (o in f32, lse) is stored per (token, index head, run);
// a second kernel merges a token's runs with the log-sum-exp combine.
#include "msa_device.h"
#include "msa_internal.h"

namespace msa {

namespace {

constexpr int kIvWaves = 8;
constexpr int kIvThreads = kIvWaves * kWave;  // 512
constexpr int kIvRows = 32 * kIvWaves;        // query rows per workgroup
// LDS row strides in bf16 elements, by gfx950's bank rules (64 banks of 4
// bytes): the 8-byte V^T fragment reads of 16 rows are conflict-free at a
// 264-byte row, and the 16-byte K fragment reads of 16 rows at a 288-byte
// row (Di = 128); the transposing V^T stores are conflict-free at 264 bytes
// with the staging map below.
constexpr int kKeyStride = kBlock + 4;  // V^T row stride
template <int DI>
constexpr int kKStride = DI == 128 ? DI + 16 : DI + 8;  // K row stride
constexpr float kLn2v = 0.69314718055994531f;

template <int DI>
struct IvStage {
  alignas(16) uint16_t k[kBlock * kKStride<DI>];  // K   [key][dim]
  alignas(16) uint16_t vt[DI * kKeyStride];   // V^T [dim][key]
};

__device__ __forceinline__ float rows_max_v(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  const auto r2 = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return fmaxf(__uint_as_float(r2[0]), __uint_as_float(r2[1]));
}
__device__ __forceinline__ float rows_sum_v(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  const auto r2 = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __uint_as_float(r2[0]) + __uint_as_float(r2[1]);
}

__device__ __forceinline__ uint32_t pack2_rne_v(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v;
  v[0] = static_cast<__bf16>(lo);
  v[1] = static_cast<__bf16>(hi);
  uint32_t u;
  __builtin_memcpy(&u, &v, 4);
  return u;
}

__device__ __forceinline__ void clear8(u32x4_t& v, bool keep) {
  const uint32_t m = keep ? 0xffffffffu : 0u;
  v.x &= m; v.y &= m; v.z &= m; v.w &= m;
}

}  // namespace

template <int DI>
__global__ __launch_bounds__(kIvThreads, 1) void prefill_value_kernel(PrefillValueArgs a) {
  constexpr int KS = DI / 32;            // 32-dim k-steps of S^T
  constexpr int DT = DI / 16;            // 16-dim row tiles of O^T
  constexpr int LPK = DI / 8;            // staging lanes per key row
  constexpr int KPP = kIvThreads / LPK;  // key rows per staging pass
  constexpr int KPASS = kBlock / KPP;    // K staging loads per thread
  constexpr int VKEYS = kBlock / KPP;    // consecutive V keys per thread
  static_assert(VKEYS == 2 || VKEYS == 4, "V staging covers 2 or 4 keys per thread");
  __shared__ IvStage<DI> S[2];

  // workgroup -> (256-row query tile, sequence, index head, key-block run),
  // query tile outermost (the grid is sized for the longest possible
  // sequence; empty tiles exit at once and are dispatched last)
  const int per_tile = a.num_seqs * a.hidx * a.kchunks;
  const int qt = blockIdx.x / per_tile;
  int rem = blockIdx.x - qt * per_tile;
  const int b = rem / (a.hidx * a.kchunks);
  rem -= b * a.hidx * a.kchunks;
  const int h = rem / a.kchunks;
  const int kc = rem - h * a.kchunks;
  const int cu0 = a.cu_seqlens_q[b];
  const int nq = a.cu_seqlens_q[b + 1] - cu0;
  const int i0 = qt * kIvRows;
  if (i0 >= nq) return;
  const int L = a.seq_lens[b];
  const int prefix = L - nq;
  const int p_last = prefix + min(nq, i0 + kIvRows) - 1;
  if (p_last < 0) return;
  const int nb_tile = min(p_last / kBlock + 1, a.max_blocks);
  const int j0 = kc * a.blocks_per_chunk;
  const int j1 = min(nb_tile, j0 + a.blocks_per_chunk);
  if (j0 >= j1) return;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int w = tid / kWave;
  const int l16 = lane & 15;
  const int q4 = lane >> 4;

  // index queries of this wave's rows 32 w + 16 nt + l16 as B operands
  bf16x8_t qf[2][KS];
  int rpos[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int i = i0 + 32 * w + 16 * nt + l16;
    rpos[nt] = i < nq ? prefix + i : -1;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (i < nq) {
        qf[nt][ks] = *reinterpret_cast<const bf16x8_t*>(
            reinterpret_cast<const uint16_t*>(a.idx_q) +
            (static_cast<int64_t>(cu0 + i) * a.hidx + h) * DI + 32 * ks + 8 * q4);
      } else {
        qf[nt][ks] = bf16x8_t{};
      }
    }
  }

  // staging: K rows KPP * i + kr, dims dc .. dc + 8; V rows VKEYS * kr + kk
  const int kr = tid / LPK;
  const int dc = (tid % LPK) * 8;
  // V: at Di = 128 the lanes of a wave take 8 key groups x 8 dim chunks, so
  // that one transposing store of the wave (rows 8 c + d, 4 keys each) covers
  // every bank exactly twice
  const int kvr = DI == 128 ? (tid % 8) + 8 * (tid / 128) : kr;
  const int vdc = DI == 128 ? ((tid / 8) % 16) * 8 : dc;
  const int* bt_row = a.block_table + static_cast<int64_t>(b) * a.max_blocks;
  u32x4_t kraw[KPASS], vraw[VKEYS];
  int nvalid_next = 0;
  auto fetch = [&](int j) {
    int page = bt_row[j];
    const bool ok = page >= 0 && page < a.num_pages;
    nvalid_next = ok ? max(0, min(kBlock, L - j * kBlock)) : 0;
    if (!ok) page = 0;  // never used: every key of the block is masked
    const int64_t run = (static_cast<int64_t>(page) * a.hidx + h) * kBlock * DI;
    const uint16_t* kp = reinterpret_cast<const uint16_t*>(a.idx_k) + run;
    const uint16_t* vp = reinterpret_cast<const uint16_t*>(a.idx_v) + run;
#pragma unroll
    for (int i = 0; i < KPASS; ++i)
      kraw[i] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4_t*>(kp + (KPP * i + kr) * DI + dc));
#pragma unroll
    for (int kk = 0; kk < VKEYS; ++kk)
      vraw[kk] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4_t*>(vp + (VKEYS * kvr + kk) * DI + vdc));
  };
  auto stage = [&](IvStage<DI>& B, int nvalid) {
#pragma unroll
    for (int i = 0; i < KPASS; ++i)
      *reinterpret_cast<u32x4_t*>(&B.k[(KPP * i + kr) * kKStride<DI> + dc]) = kraw[i];
    // value rows past the sequence end hold stale bytes (possibly NaN):
    // cleared, since 0 * NaN would reach the MFMA sums
#pragma unroll
    for (int kk = 0; kk < VKEYS; ++kk) clear8(vraw[kk], VKEYS * kvr + kk < nvalid);
    uint16_t v[VKEYS][8];
#pragma unroll
    for (int kk = 0; kk < VKEYS; ++kk) __builtin_memcpy(&v[kk][0], &vraw[kk], 16);
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      if constexpr (VKEYS == 4) {
        const u32x2_t pr = {static_cast<uint32_t>(v[0][d]) | (static_cast<uint32_t>(v[1][d]) << 16),
                            static_cast<uint32_t>(v[2][d]) | (static_cast<uint32_t>(v[3][d]) << 16)};
        *reinterpret_cast<u32x2_t*>(&B.vt[(vdc + d) * kKeyStride + 4 * kvr]) = pr;
      } else {
        *reinterpret_cast<uint32_t*>(&B.vt[(vdc + d) * kKeyStride + 2 * kvr]) =
            static_cast<uint32_t>(v[0][d]) | (static_cast<uint32_t>(v[1][d]) << 16);
      }
    }
  };

  float mrow[2] = {-INFINITY, -INFINITY}, lrow[2] = {0.f, 0.f};
  f32x4_t o[DT][2];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    o[dt][0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    o[dt][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  fetch(j0);
  int nvalid_cur = nvalid_next;
  stage(S[0], nvalid_cur);
  __syncthreads();
  int buf = 0;
  for (int j = j0; j < j1; ++j) {
    if (j + 1 < j1) fetch(j + 1);
    const IvStage<DI>& B = S[buf];
    const int tok0 = j * kBlock;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      f32x4_t st[4][2];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        st[mt][0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        st[mt][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(
              &B.k[(64 * kh + 16 * mt + l16) * kKStride<DI> + 32 * ks + 8 * q4]);
          st[mt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[0][ks], st[mt][0], 0, 0, 0);
          st[mt][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[1][ks], st[mt][1], 0, 0, 0);
        }
      }
      // keys past the sequence end or after the row's position: -inf
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = 64 * kh + 16 * mt + 4 * q4 + r;
            const bool ok = key < nvalid_cur && tok0 + key <= rpos[nt];
            st[mt][nt][r] = ok ? st[mt][nt][r] * a.scale_log2 : -INFINITY;
          }
      float alpha[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        float mr = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) mr = fmaxf(mr, st[mt][nt][r]);
        const float mn = fmaxf(mrow[nt], rows_max_v(mr));
        // a row with nothing visible yet keeps m = -inf; its p are 2^-inf = 0
        const float mu = mn == -INFINITY ? 0.f : mn;
        alpha[nt] = __builtin_amdgcn_exp2f(mrow[nt] - mu);
        float l = 0.f;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float e = __builtin_amdgcn_exp2f(st[mt][nt][r] - mu);
            st[mt][nt][r] = e;
            l += e;
          }
        mrow[nt] = mn;
        lrow[nt] = lrow[nt] * alpha[nt] + rows_sum_v(l);
      }
      bf16x8_t pb[2][2];
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const uint32_t u[4] = {pack2_rne_v(st[2 * k2][nt][0], st[2 * k2][nt][1]),
                                 pack2_rne_v(st[2 * k2][nt][2], st[2 * k2][nt][3]),
                                 pack2_rne_v(st[2 * k2 + 1][nt][0], st[2 * k2 + 1][nt][1]),
                                 pack2_rne_v(st[2 * k2 + 1][nt][2], st[2 * k2 + 1][nt][3])};
          __builtin_memcpy(&pb[k2][nt], u, 16);
        }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
          for (int r = 0; r < 4; ++r) o[dt][nt][r] *= alpha[nt];
      // O^T += V^T P^T over the half's two 32-key steps: k-slots of lane group
      // q4 are the keys 32 kk + 4 q4 + e and 32 kk + 16 + 4 q4 + e, where the
      // S^T tiles 2 k2 and 2 k2 + 1 hold them
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        const int kk = 2 * kh + k2;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const uint16_t* vrow = &B.vt[(16 * dt + l16) * kKeyStride + 32 * kk + 4 * q4];
          const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(vrow);
          const u32x2_t hi2 = *reinterpret_cast<const u32x2_t*>(vrow + 16);
          const u32x4_t cat = {lo[0], lo[1], hi2[0], hi2[1]};
          bf16x8_t vf;
          __builtin_memcpy(&vf, &cat, 16);
          o[dt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb[k2][0], o[dt][0], 0, 0, 0);
          o[dt][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb[k2][1], o[dt][1], 0, 0, 0);
        }
      }
    }
    if (j + 1 < j1) {
      nvalid_cur = nvalid_next;
      stage(S[buf ^ 1], nvalid_cur);
    }
    __syncthreads();
    buf ^= 1;
  }

  // the run's normalised partial of each row and its lse (natural log)
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int i = i0 + 32 * w + 16 * nt + l16;
    if (i >= nq) continue;
    const float l = lrow[nt];
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const int64_t prow = (static_cast<int64_t>(cu0 + i) * a.hidx + h) * a.kchunks + kc;
    float* po = a.part_o + prow * DI + 4 * q4;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<f32x4_t*>(po + 16 * dt) = o[dt][nt] * inv;
    if (q4 == 0) a.part_lse[prow] = l > 0.f ? (mrow[nt] + __builtin_amdgcn_logf(l)) * kLn2v : -INFINITY;
  }
}

// out = sum_c exp(lse_c - lse) o_c over the runs c of a token that hold any
// of its visible blocks.  DI / 4 threads per (token, index head) row, four
// dims each.
template <int DI>
__global__ __launch_bounds__(kWgThreads) void prefill_value_combine_kernel(PrefillValueArgs a) {
  constexpr int TPR = DI / 4;                // threads per row
  constexpr int RPW = kWgThreads / TPR;      // rows per workgroup
  const int row = blockIdx.x * RPW + threadIdx.x / TPR;
  if (row >= a.num_tokens * a.hidx) return;
  const int t = row / a.hidx;
  const int d0 = (threadIdx.x % TPR) * 4;
  int lo = 0, hi = a.num_seqs;  // cu[lo] <= t < cu[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) / 2;
    if (a.cu_seqlens_q[mid] <= t) lo = mid; else hi = mid;
  }
  const int n = a.cu_seqlens_q[lo + 1] - a.cu_seqlens_q[lo];
  const int p = a.seq_lens[lo] - n + (t - a.cu_seqlens_q[lo]);
  const int nkc = p >= 0 ? min(p / kBlock, a.max_blocks - 1) / a.blocks_per_chunk + 1 : 0;
  const float* lse = a.part_lse + static_cast<int64_t>(row) * a.kchunks;
  const float* po = a.part_o + static_cast<int64_t>(row) * a.kchunks * DI + d0;
  float m = -INFINITY;
  for (int c = 0; c < nkc; ++c) m = fmaxf(m, lse[c]);
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  float ws = 0.f;
  if (m != -INFINITY) {
    for (int c = 0; c < nkc; ++c) {
      const float wv = __expf(lse[c] - m);
      ws += wv;
      acc += wv * *reinterpret_cast<const f32x4_t*>(po + static_cast<int64_t>(c) * DI);
    }
  }
  const float inv = ws > 0.f ? 1.f / ws : 0.f;
  const int64_t out0 = static_cast<int64_t>(row) * DI + d0;
  if (a.out_f32) {
    *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(a.idx_out) + out0) = acc * inv;
  } else {
    const u32x2_t v = {pack2_rne_v(acc[0] * inv, acc[1] * inv), pack2_rne_v(acc[2] * inv, acc[3] * inv)};
    *reinterpret_cast<u32x2_t*>(reinterpret_cast<uint16_t*>(a.idx_out) + out0) = v;
  }
}

hipError_t launch_prefill_value(const PrefillValueArgs& a, int idx_dim, hipStream_t s) {
  const int grid = a.num_seqs * a.max_tiles * a.hidx * a.kchunks;
  if (grid == 0 || a.num_tokens == 0) return hipSuccess;
  const int rows = a.num_tokens * a.hidx;
  if (idx_dim == 128) {
    prefill_value_kernel<128><<<grid, kIvThreads, 0, s>>>(a);
    prefill_value_combine_kernel<128><<<(rows + 7) / 8, kWgThreads, 0, s>>>(a);
  } else {
    prefill_value_kernel<64><<<grid, kIvThreads, 0, s>>>(a);
    prefill_value_combine_kernel<64><<<(rows + 15) / 16, kWgThreads, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace msa
