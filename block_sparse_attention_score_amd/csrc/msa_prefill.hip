// Chunked prefill: index-head scoring as a causal bf16 GEMM on the matrix
// cores with a block-max epilogue, and a wavefront-per-row top-k selection.
//
// vLLM page sparse_attention_msa.py (MiniMaxM3SparseMSAImpl.forward, prefill
// part): prefill tokens attend causally to the selected 128-token blocks of
// their sequence; sglang page minimax_sparse_backend.py (forward_extend): the
// new tokens of a sequence follow its cached prefix (cu_seqlens over the
// extend lengths, prefix lengths alongside).
//
// Scoring.  For the n_b new tokens of sequence b (positions p_i = L_b - n_b +
// i) and index head h, score[i][j] = max over tokens t <= p_i of block j of
// q_idx[i] . k_idx[t].  A workgroup takes 256 query rows (4 waves x 64) and a
// run of key blocks; the query rows stay in registers as MFMA B operands; each
// key block (128 tokens x Di) is staged once in LDS by direct-to-LDS buffer
// loads (each lane's 16 bytes land at the instruction's LDS base + 16 lane;
// the chunks of a row XOR-swizzled so that fragment reads do not conflict)
// and read by all four waves as A operands of v_mfma_f32_16x16x32_bf16, so
// each result tile is S^T (tokens down, queries across) and a lane folds its
// four tokens per tile into its query's maximum with no cross-lane step until
// the block ends.  With no staging registers the kernel fits 128 VGPRs and one
// 32 KB buffer, so four workgroups share a CU and each one's wait for its
// next block is covered by the others' MFMAs.  Blocks that end before a
// wave's first query skip the causal mask.  The mean and log-sum-exp block
// scores use the same tiles: a lane sums (or exp-accumulates) its tokens and
// the four lanes of a query column combine at the block's end.
#include "msa_device.h"
#include "msa_internal.h"
#include "msa_select.h"

namespace msa {

constexpr int kPrefillRows = 256;  // query rows per scoring workgroup

// (four workgroups per CU need at most 128 VGPRs; the log-sum-exp reducer at
// Di = 128 needs more and runs two per CU instead of spilling)
template <int DI, int ST>
__global__ __launch_bounds__(kWgThreads, (ST == kScoreLse && DI == 128) ? 2 : 4) void
prefill_score_kernel(PrefillScoreArgs a) {
  constexpr int KS = DI / 32;              // 32-dim k-steps
  constexpr int CH = DI * 2 / 16;          // 16-byte chunks per key row
  constexpr int RPI = kWave / CH;          // rows per direct-to-LDS instruction
  constexpr int NI = kBlock / RPI / 4;     // instructions per wave per block
  __shared__ __attribute__((aligned(16))) uint16_t kb[kBlock * DI];
  const int runs = a.num_seqs * a.hidx * a.kchunks;
  const int xl = blockIdx.x >> 3;
  const int qt = xl % a.max_tiles;
  const int run = (xl / a.max_tiles) * 8 + (blockIdx.x & 7);
  if (run >= runs) return;
  int rem = run;
  const int b = rem / (a.hidx * a.kchunks);
  rem -= b * a.hidx * a.kchunks;
  const int h = rem / a.kchunks;
  const int kc = rem - h * a.kchunks;
  const int cu0 = a.cu_seqlens_q[b];
  const int nq = a.cu_seqlens_q[b + 1] - cu0;
  const int i0 = qt * kPrefillRows;
  if (i0 >= nq) return;
  const int L = a.seq_lens[b];
  const int prefix = L - nq;
  const int p_last = prefix + min(nq, i0 + kPrefillRows) - 1;
  if (p_last < 0) return;
  const int nb_tile = min(p_last / kBlock + 1, a.max_blocks);
  const int j0 = kc * kPrefillBlocksPerChunk;
  const int j1 = min(nb_tile, j0 + kPrefillBlocksPerChunk);
  if (j0 >= j1) return;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int l16 = lane & 15;
  const int q4 = lane >> 4;

  bf16x8_t qb[4][KS];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    const int i = i0 + 64 * w + 16 * rt + l16;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if (i < nq) {
        qb[rt][s] = *reinterpret_cast<const bf16x8_t*>(
            reinterpret_cast<const uint16_t*>(a.idx_q) +
            (static_cast<int64_t>(cu0 + i) * a.hidx + h) * DI + 32 * s + 8 * q4);
      } else {
        qb[rt][s] = bf16x8_t{};
      }
    }
  }
  const int pos_w0 = prefix + i0 + 64 * w;
  const __attribute__((address_space(4))) int32_t* bt_row =
      (const __attribute__((address_space(4))) int32_t*)(
          reinterpret_cast<uintptr_t>(a.block_table + static_cast<int64_t>(b) * a.max_blocks));
  const int np32 = static_cast<int>(a.num_pages < 0x7fffffff ? a.num_pages : 0x7fffffff);
  const int rows = min(nq - i0, kPrefillRows);
  const auto srsrc = __builtin_amdgcn_make_buffer_rsrc(
      a.scores + (static_cast<int64_t>(cu0 + i0) * a.hidx + h) * a.max_blocks, 0,
      rows * a.hidx * a.max_blocks * 4, 0x00020000);
  int srow[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) srow[rt] = (64 * w + 16 * rt + l16) * a.hidx * a.max_blocks * 4;
  float sv[4][4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int e = 0; e < 4; ++e) sv[rt][e] = -INFINITY;

  // Chunk c of key row r sits at chunk swz(c, r): 16 rows of a fragment read
  // then hit 16 distinct 16-byte bank groups (Di = 128: 256-byte rows, XOR
  // with r mod 16; Di = 64: 128-byte rows, two per bank group, XOR with
  // (r / 2) mod 8).
  auto swz = [](int c, int r) { return DI == 128 ? (c ^ (r & 15)) : (c ^ ((r >> 1) & 7)); };
  auto tile = [&](int n, f32x4_t (&acc)[4]) {
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) acc[rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const bf16x8_t ka = *reinterpret_cast<const bf16x8_t*>(
          &kb[(16 * n + l16) * DI + 8 * swz(4 * s + q4, 16 * n + l16)]);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
        acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qb[rt][s], acc[rt], 0, 0, 0);
    }
  };

  for (int j = j0; j < j1; ++j) {
    const int pg = bt_row[j];
    const bool page_ok = pg >= 0 && pg < np32;
    {
      // (LDS pointers cast in place: a helper returning an LDS pointer type
      // would not compile for the host side; source offsets from a fresh
      // thread index, so they are not kept live across the loop)
      const auto r = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<char*>(reinterpret_cast<const char*>(a.idx_k)) +
              (static_cast<int64_t>(page_ok ? pg : 0) * a.hidx + h) * kBlock * DI * 2,
          0, page_ok ? kBlock * DI * 2 : 0, 0x00020000);
      int tl = tid;
      asm volatile("" : "+v"(tl));
      const int ln = tl & (kWave - 1);
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int row0 = RPI * (NI * w + i);
        const int row = row0 + ln / CH;
        const int cp = ln % CH;
        // (the offset goes through a local: written into the builtin's
        // argument list, the swizzle call made the host side of the kernel
        // drop its launch stub)
        const int off = row * DI * 2 + 16 * swz(cp, row);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            r, (__attribute__((address_space(3))) void*)(kb + row0 * DI), 16, off, 0, 0, 0);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    float mx[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) mx[rt] = -INFINITY;
    if constexpr (ST != kScoreMax) {
      BlockScore<ST> red[4];
      if (page_ok) {
        const bool full = kBlock * j + kBlock - 1 <= pos_w0;
        for (int n = 0; n < 8; ++n) {
          f32x4_t acc[4];
          tile(n, acc);
          const int tok = kBlock * j + 16 * n + 4 * q4;
#pragma unroll
          for (int rt = 0; rt < 4; ++rt) {
            const int pos = pos_w0 + 16 * rt + l16;
            const float d[4] = {acc[rt][0], acc[rt][1], acc[rt][2], acc[rt][3]};
            const bool ok[4] = {full || tok <= pos, full || tok + 1 <= pos,
                                full || tok + 2 <= pos, full || tok + 3 <= pos};
            red[rt].add(d, ok, true, a.st_scale_log2);
          }
        }
      }
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const int pos = pos_w0 + 16 * rt + l16;
        const int nvis = page_ok ? min(kBlock, max(0, pos + 1 - kBlock * j)) : 0;
        mx[rt] = red[rt].finish_q4(nvis);
      }
    } else if (page_ok && kBlock * j + kBlock - 1 <= pos_w0) {
#pragma unroll 2
      for (int n = 0; n < 8; ++n) {
        f32x4_t acc[4];
        tile(n, acc);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
          mx[rt] = max_nan(max_nan(max_nan(max_nan(mx[rt], acc[rt][0]), acc[rt][1]), acc[rt][2]),
                           acc[rt][3]);
      }
    } else if (page_ok) {
#pragma unroll 2
      for (int n = 0; n < 8; ++n) {
        f32x4_t acc[4];
        tile(n, acc);
        const int tok = kBlock * j + 16 * n + 4 * q4;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          const int pos = pos_w0 + 16 * rt + l16;
#pragma unroll
          for (int r = 0; r < 4; ++r) mx[rt] = max_nan(mx[rt], tok + r <= pos ? acc[rt][r] : -INFINITY);
        }
      }
    }
    if constexpr (ST == kScoreMax) {
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        mx[rt] = max_nan(mx[rt], __shfl_xor(mx[rt], 16));
        mx[rt] = max_nan(mx[rt], __shfl_xor(mx[rt], 32));
      }
    }
    const int jj = j - j0;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int e = 0; e < 4; ++e) sv[rt][e] = jj == 4 * q4 + e ? mx[rt] : sv[rt][e];
    // every wave is done with the buffer before the next block overwrites it
    __syncthreads();
  }
  const int jb = 4 * q4;
  if (j0 + kPrefillBlocksPerChunk <= a.max_blocks) {
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const u32x4_t v = {__float_as_uint(sv[rt][0]), __float_as_uint(sv[rt][1]),
                         __float_as_uint(sv[rt][2]), __float_as_uint(sv[rt][3])};
      __builtin_amdgcn_raw_buffer_store_b128(v, srsrc, srow[rt] + 4 * jb, 4 * j0, 0);
    }
  } else {
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (j0 + jb + e < a.max_blocks)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sv[rt][e]), srsrc,
                                                srow[rt] + 4 * (jb + e), 4 * j0, 0);
  }
}


// One wavefront per (query token, index head) row, for rows of up to 64 * E
// blocks (select_wave).
template <int E>
__global__ __launch_bounds__(kWgThreads) void select_wave_kernel(SelectArgs a) {
  if (a.zero_words != nullptr) clear_words(a);
  const int lane = threadIdx.x & (kWave - 1);
  const int row = blockIdx.x * (kWgThreads / kWave) + threadIdx.x / kWave;
  if (row >= a.num_tokens * a.hidx) return;
  const int t = row / a.hidx;
  // The row's scores are fetched first (their address does not depend on the
  // position), so their loads overlap the position lookup.
  float v[E];
  load_row_scores<E>(a.scores + static_cast<int64_t>(row) * a.max_blocks, a.max_blocks, v);
  int p;
  if (a.cu_seqlens_q == nullptr) {
    p = a.seq_lens[t] - 1;
  } else if (a.num_seqs <= kWave) {
    // lane b reads sequence b's bounds and length in one round trip; token t
    // belongs to the last sequence whose first token is at or before t (the
    // offsets never decrease, so those lanes are a prefix of the wave)
    const int bl = min(lane, a.num_seqs - 1);
    const int cu_l = a.cu_seqlens_q[bl];
    const int cu_n = a.cu_seqlens_q[bl + 1];
    const int len = a.seq_lens[bl];
    const int b = max(__popcll(__builtin_amdgcn_ballot_w64(lane < a.num_seqs && cu_l <= t)) - 1, 0);
    const int first = __builtin_amdgcn_readlane(cu_l, b);
    p = __builtin_amdgcn_readlane(len, b) - (__builtin_amdgcn_readlane(cu_n, b) - first) +
        (t - first);
  } else {
    int lo = 0, hi = a.num_seqs;
    while (hi - lo > 1) {
      const int mid = (lo + hi) / 2;
      if (a.cu_seqlens_q[mid] <= t) lo = mid; else hi = mid;
    }
    p = a.seq_lens[lo] - (a.cu_seqlens_q[lo + 1] - a.cu_seqlens_q[lo]) + (t - a.cu_seqlens_q[lo]);
  }
  const int nb = p >= 0 ? min(p / kBlock + 1, a.max_blocks) : 0;
  int32_t* sel = a.sel + static_cast<int64_t>(row) * a.kmax;
  const int total = select_wave_loaded<E>(v, nb,
                                          topk_beside_forced(a.topk, nb, a.init, a.local,
                                                             a.forced_in_budget),
                                          a.init, a.local,
                                          [&](int pos, int j) { sel[pos] = j; });
  for (int i = total + lane; i < a.kmax; i += kWave) sel[i] = -1;
  if (lane == 0) a.cnt[row] = total;
}

// ------------------------------------------------------------- launchers

template <int ST>
static void launch_prefill_score_st(const PrefillScoreArgs& a, int idx_dim, int grid,
                                    hipStream_t s) {
  if (idx_dim == 128)
    prefill_score_kernel<128, ST><<<grid, kWgThreads, 0, s>>>(a);
  else
    prefill_score_kernel<64, ST><<<grid, kWgThreads, 0, s>>>(a);
}

hipError_t launch_prefill_score(const PrefillScoreArgs& a, int idx_dim, int score_type,
                                hipStream_t s) {
  // runs rounded up to a multiple of 8 (one set per XCD), times the tiles
  const int grid = (a.num_seqs * a.hidx * a.kchunks + 7) / 8 * 8 * a.max_tiles;
  if (grid == 0) return hipSuccess;
  if (score_type == kScoreMean) launch_prefill_score_st<kScoreMean>(a, idx_dim, grid, s);
  else if (score_type == kScoreLse) launch_prefill_score_st<kScoreLse>(a, idx_dim, grid, s);
  else launch_prefill_score_st<kScoreMax>(a, idx_dim, grid, s);
  return hipGetLastError();
}

bool select_wave_fits(int max_blocks) { return max_blocks <= 1024; }

hipError_t launch_select_wave(const SelectArgs& a, hipStream_t s) {
  const int rows = a.num_tokens * a.hidx;
  if (rows == 0) return hipSuccess;
  const int grid = (rows + 3) / 4;
  if (a.max_blocks <= 256)
    select_wave_kernel<4><<<grid, kWgThreads, 0, s>>>(a);
  else
    select_wave_kernel<16><<<grid, kWgThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace msa
