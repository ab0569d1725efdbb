// Per-query block selection on one 256-thread workgroup.
//
// Selection rule (sglang page minimax_sparse_backend.py,
// MiniMaxSparseAttnBackend.__init__: init, local and top-k block counts for a
// per-token selection): for nb visible blocks the forced set is
// F = {0..init-1} U {nb-local..nb-1}; the top-k of the other blocks by
// (score desc, block asc) join F; the result is written in ascending block
// order, -1 padded, with |S| = |F| + min(topk, nb - |F|).
//
// Method: scores become order-preserving 32-bit keys (-0 folded onto +0).  A
// 4-pass, 8-bit radix select over the candidates finds the key T of the k-th
// best candidate and how many candidates with key == T still fit; those are
// taken in ascending block order (ranks from a workgroup scan), which is the
// lower-index tie rule.  Each thread owns a contiguous run of blocks, so one
// more scan gives every selected block its output slot.
#pragma once

#include "msa_device.h"

namespace msa {

struct SelectLds {
  int hist[256];
  int wsum[16];
  int digit;
  int need;
};

// Number of forced blocks among nb visible ones.
__device__ __forceinline__ int forced_count(int nb, int init, int local) {
  const int a = min(init, nb);
  const int lo = max(0, nb - local);
  return a + (nb - lo) - max(0, a - lo);
}

// Candidates to take beside the forced blocks of a row of nb visible blocks:
// topk, or, when the forced blocks count inside the budget, what is left of
// it (max(topk - |F|, 0)).  The selection routines below take this count.
__device__ __forceinline__ int topk_beside_forced(int topk, int nb, int init, int local,
                                                  int forced_in_budget) {
  return forced_in_budget ? max(topk - forced_count(nb, init, local), 0) : topk;
}

// s: nb scores of one (query, index head) row.  MAXPER >= ceil(nb / NT).
// Must be called by all NT (256 .. 1024) threads of the workgroup.  Calls
// emit(pos, j) for every selected block j, pos being its slot in ascending
// block order, and returns the selection size.  No barrier after the last
// emit.
template <int MAXPER, int NT = kWgThreads, class Emit>
__device__ int select_core(const float* __restrict__ s, int nb, int topk, int init, int local,
                           SelectLds& L, Emit emit) {
  static_assert(NT >= 256 && NT <= 1024, "one histogram bin per thread of the first 256");
  const int tid = threadIdx.x;
  const int per = div_up(nb, NT);
  const int j0 = tid * per;
  const int lo_init = min(init, nb);       // j <  lo_init  -> forced (init)
  const int hi_local = max(0, nb - local);  // j >= hi_local -> forced (local)
  const int nforced = forced_count(nb, init, local);
  const int ncand = nb - nforced;
  const int keff = min(topk, ncand);
  const bool take_all = keff == ncand;

  // Straight-line loads (slots past the row re-read its last score and are
  // discarded), so that all of a thread's loads are in flight at once.
  uint32_t key[MAXPER];
  if (nb > 0) {
    float v[MAXPER];
#pragma unroll
    for (int i = 0; i < MAXPER; ++i) {
      const int j = min(j0 + i, nb - 1);
      v[i] = s[j];
    }
#pragma unroll
    for (int i = 0; i < MAXPER; ++i) key[i] = (i < per && j0 + i < nb) ? score_key(v[i]) : 0u;
  } else {
#pragma unroll
    for (int i = 0; i < MAXPER; ++i) key[i] = 0u;
  }
  auto is_cand = [&](int j) { return j < nb && j >= lo_init && j < hi_local; };

  uint32_t T = 0u;
  int need = 0;
  if (!take_all && keff == 0) {
    // no candidate joins the forced blocks: no key lies above T = max, none
    // of those equal to it is needed
    T = 0xFFFFFFFFu;
  } else if (!take_all) {
    uint32_t prefix = 0u;
    need = keff;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      const uint32_t hi_mask = pass == 0 ? 0u : (0xFFFFFFFFu << (shift + 8));
      if (tid < 256) L.hist[tid] = 0;
      __syncthreads();
#pragma unroll
      for (int i = 0; i < MAXPER; ++i) {
        const int j = j0 + i;
        if (i < per && is_cand(j) && (key[i] & hi_mask) == prefix)
          atomicAdd(&L.hist[(key[i] >> shift) & 0xFF], 1);
      }
      __syncthreads();
      // Thread tid looks at digit 255 - tid: an inclusive scan counts the
      // candidates whose digit is >= that one.
      const int d = 255 - tid;
      const int c = tid < 256 ? L.hist[d] : 0;
      const int incl = block_incl_scan(c, L.wsum);
      const int excl = incl - c;
      if (excl < need && need <= incl) {
        L.digit = d;
        L.need = need - excl;
      }
      __syncthreads();
      prefix |= static_cast<uint32_t>(L.digit) << shift;
      need = L.need;
      __syncthreads();
    }
    T = prefix;
  }

  // Rank of each key == T candidate among equals, in block order.
  int eq_local = 0;
  if (!take_all) {
#pragma unroll
    for (int i = 0; i < MAXPER; ++i) {
      const int j = j0 + i;
      eq_local += (i < per && is_cand(j) && key[i] == T) ? 1 : 0;
    }
  }
  int r = block_incl_scan(eq_local, L.wsum) - eq_local;

  bool flag[MAXPER];
  int sel_local = 0;
#pragma unroll
  for (int i = 0; i < MAXPER; ++i) {
    const int j = j0 + i;
    bool f = false;
    if (i < per && j < nb) {
      if (!is_cand(j) || take_all) {
        f = true;
      } else if (key[i] > T) {
        f = true;
      } else if (key[i] == T) {
        f = r < need;
        ++r;
      }
    }
    flag[i] = f;
    sel_local += f ? 1 : 0;
  }
  int pos = block_incl_scan(sel_local, L.wsum) - sel_local;
#pragma unroll
  for (int i = 0; i < MAXPER; ++i) {
    if (flag[i]) {
      emit(pos, j0 + i);
      ++pos;
    }
  }
  return nforced + keff;
}

// The same selection on one wave (no barrier, no LDS): block j sits in lane
// j % 64, slot j / 64, with E >= ceil(nb / 64).  T, the key of the k-th best
// candidate, is found bit by bit with ballot counts, from the highest bit in
// which the candidates' keys differ (the wave's largest and smallest key give
// it; the bits above are common to all candidates and so to T); candidates
// above T are taken, and of those equal to T the first ones in block order
// (ranks from ballot prefix counts), which is the lower-index tie rule.
// Output slots come from the same prefix counts, so the list is ascending.
// Calls emit(pos, j) from the lane owning block j; returns the selection size.
// select_wave_loaded takes the row already in registers: v[e] holds block
// lane + 64 e for every such block below nb (other slots are ignored).
template <int E>
__device__ __forceinline__ void load_row_scores(const float* __restrict__ s, int n,
                                                float (&v)[E]) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int e = 0; e < E; ++e) v[e] = s[min(lane + kWave * e, max(n - 1, 0))];
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xF, 0xF, false));
}

// Maximum of an unsigned value over the wavefront (all lanes active), as a
// uniform value: DPP maxima within each row of 16 lanes, then the four rows.
__device__ __forceinline__ uint32_t wave_umax_uniform(uint32_t v) {
  v = max(v, dpp_u<kDppXor1>(v));
  v = max(v, dpp_u<kDppXor2>(v));
  v = max(v, dpp_u<kDppHalfMirror>(v));
  v = max(v, dpp_u<kDppMirror>(v));
  const uint32_t r0 = __builtin_amdgcn_readlane(static_cast<int>(v), 0);
  const uint32_t r1 = __builtin_amdgcn_readlane(static_cast<int>(v), 16);
  const uint32_t r2 = __builtin_amdgcn_readlane(static_cast<int>(v), 32);
  const uint32_t r3 = __builtin_amdgcn_readlane(static_cast<int>(v), 48);
  return max(max(r0, r1), max(r2, r3));
}

template <int E, class Emit>
__device__ int select_wave_loaded(const float (&v)[E], int nb, int topk, int init, int local,
                                  Emit emit) {
  const int lane = threadIdx.x & (kWave - 1);
  const int lo_init = min(init, nb);
  const int hi_local = max(0, nb - local);
  const int nforced = forced_count(nb, init, local);
  const int ncand = nb - nforced;
  const int keff = min(topk, ncand);
  const bool take_all = keff == ncand;

  uint32_t key[E];
  bool cand[E], valid[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = lane + kWave * e;
    valid[e] = j < nb;
    cand[e] = valid[e] && j >= lo_init && j < hi_local;
    key[e] = cand[e] ? score_key(v[e]) : 0u;
  }
  // Non-candidates carry key 0, and every probe c below is >= 1, so the bit
  // loop needs no candidate mask.
  auto count = [](bool x) { return __popcll(__builtin_amdgcn_ballot_w64(x)); };
  uint32_t T = 0u;
  int need = 0;
  if (!take_all && keff == 0) {
    T = 0xFFFFFFFFu;  // no candidate joins the forced blocks
  } else if (!take_all) {
    // Bits above the highest one in which the candidates' keys differ are
    // the same in every candidate, hence in T: the search starts below them
    // (for those bits every probe would count all candidates or none).
    uint32_t hi = 0u, lo_inv = 0u;  // max key, ~min key over the candidates
#pragma unroll
    for (int e = 0; e < E; ++e) {
      hi = max(hi, cand[e] ? key[e] : 0u);
      lo_inv = max(lo_inv, cand[e] ? ~key[e] : 0u);
    }
    hi = wave_umax_uniform(hi);
    const uint32_t diff = hi ^ ~wave_umax_uniform(lo_inv);
    int top = -1;
    if (diff == 0u) {
      T = hi;  // all candidates equal: T is their key
    } else {
      top = 31 - __builtin_clz(diff);
      T = hi & ~((2u << top) - 1u);
    }
    for (int bit = top; bit >= 0; --bit) {
      const uint32_t c = T | (1u << bit);
      // all masks first, then their counts: each compare writes a mask of
      // its own, so the compares do not wait for one another's counts
      uint64_t bm[E];
#pragma unroll
      for (int e = 0; e < E; ++e) bm[e] = __builtin_amdgcn_ballot_w64(key[e] >= c);
      int n = 0;
#pragma unroll
      for (int e = 0; e < E; ++e) n += __popcll(bm[e]);
      if (n == keff) {
        // exactly the selection: it is {key > c - 1}, with no tie to break
        T = c - 1;
        break;
      }
      if (n > keff) T = c;
    }
    int above = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) above += count(cand[e] && key[e] > T);
    need = keff - above;
  }
  auto below = [&](uint64_t m) {  // set bits of m in lanes below this one
    return static_cast<int>(__builtin_amdgcn_mbcnt_hi(
        static_cast<uint32_t>(m >> 32), __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u)));
  };
  int eq_before = 0, pos_before = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const bool is_eq = !take_all && cand[e] && key[e] == T;
    const uint64_t eqm = __builtin_amdgcn_ballot_w64(is_eq);
    const int rank = eq_before + below(eqm);
    const bool pick = valid[e] && (!cand[e] || take_all || key[e] > T || (is_eq && rank < need));
    const uint64_t pm = __builtin_amdgcn_ballot_w64(pick);
    if (pick) emit(pos_before + below(pm), lane + kWave * e);
    eq_before += __popcll(eqm);
    pos_before += __popcll(pm);
  }
  return nforced + keff;
}

template <int E, class Emit>
__device__ int select_wave(const float* __restrict__ s, int nb, int topk, int init, int local,
                           Emit emit) {
  float v[E];
  load_row_scores<E>(s, nb, v);
  return select_wave_loaded<E>(v, nb, topk, init, local, emit);
}

// select_core writing the selection to sel[0..kmax) (-1 padded) and its size
// to *cnt, ending with a barrier.
template <int MAXPER>
__device__ void select_row(const float* __restrict__ s, int nb, int topk,
                           int init, int local, int kmax,
                           int32_t* __restrict__ sel, int32_t* __restrict__ cnt,
                           SelectLds& L) {
  const int tid = threadIdx.x;
  const int total =
      select_core<MAXPER>(s, nb, topk, init, local, L, [&](int pos, int j) { sel[pos] = j; });
  for (int i = total + tid; i < kmax; i += kWgThreads) sel[i] = -1;
  if (tid == 0) *cnt = total;
  __syncthreads();
}

}  // namespace msa
