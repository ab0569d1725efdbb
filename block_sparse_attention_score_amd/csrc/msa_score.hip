// Standalone kernels: decode block scoring (step 1 alone), per-row selection
// (step 2 alone), the decode work planner, and fp8 dequantisation.
#include "msa_score.h"

namespace msa {

// One workgroup per (pair, chunk); scores only.
template <class IT, int DI>
__global__ __launch_bounds__(kWgThreads) void decode_score_kernel(ScoreArgs a) {
  __shared__ SelectLds sl;
  __shared__ int flag;
  if (blockIdx.x == 0 && a.zero_words != nullptr)
    for (int i = threadIdx.x; i < a.zero_count; i += kWgThreads) a.zero_words[i] = 0u;
  const int pair = blockIdx.x / a.chunks_per_pair;
  score_chunk<IT, DI, 4, false>(a, pair, blockIdx.x - pair * a.chunks_per_pair, sl, &flag);
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

// Workgroup-wide inclusive scan over 1024 threads (16 waves).
__device__ __forceinline__ int block1024_incl_scan(int v, int* wsum) {
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int n = __shfl_up(v, o);
    if (lane >= o) v += n;
  }
  if (lane == kWave - 1) wsum[w] = v;
  __syncthreads();
  int add = 0;
  for (int i = 0; i < w; ++i) add += wsum[i];
  __syncthreads();
  return v + add;
}

// Decode planner (one workgroup).  Zeroes the hand-off words and writes the
// order in which the persistent decode kernel claims its work: the score
// items (pair, chunk) of every (sequence, index head) pair, pair-major, with
// the attention splits of a pair's kv heads placed `lag` score items after
// the pair's last score item (or at the end), so that they are claimed about
// when the pair's selection is done.  A pair with no tokens gets one score
// item, which publishes its empty selection.  Every attention item follows
// all score items of its pair, which is what keeps the kernel's waits finite.
__global__ __launch_bounds__(1024) void decode_plan_kernel(PlanArgs a) {
  __shared__ int wsum[16];
  __shared__ int carry;
  __shared__ int s_end[kMaxPairs];  // inclusive end of each pair's score items
  for (int64_t i = threadIdx.x; i < a.zero_count; i += 1024) a.zero_begin[i] = 0u;
  if (threadIdx.x == 0) carry = 0;
  __syncthreads();
  const int npairs = a.num_seqs * a.hidx;
  for (int base = 0; base < npairs; base += 1024) {
    const int pair = base + static_cast<int>(threadIdx.x);
    int n = 0;
    if (pair < npairs) {
      const int L = a.seq_lens[pair / a.hidx];
      const int nb = L > 0 ? min((L - 1) / kBlock + 1, a.max_blocks) : 0;
      n = max(1, div_up(nb, a.pages_per_item));
    }
    const int incl = block1024_incl_scan(n, wsum);
    if (pair < npairs) s_end[pair] = carry + incl;
    __syncthreads();
    if (threadIdx.x == 1023) carry += incl;
    __syncthreads();
  }
  const int n_score = carry;
  const int per_pair = a.kv_per_idx * a.nsplit_max;  // attention items of a pair
  // number of pairs q with s_end[q] <= v (s_end is increasing)
  auto count_le = [&](int v) {
    int lo = 0, hi = npairs;
    while (lo < hi) {
      const int mid = (lo + hi) / 2;
      if (s_end[mid] <= v) lo = mid + 1; else hi = mid;
    }
    return lo;
  };
  // attention items: pair p's group sits before score item min(n_score, end + lag)
  for (int i = threadIdx.x; i < per_pair * npairs; i += 1024) {
    const int pair = i / per_pair;
    const int r = i - pair * per_pair;
    const int ins = min(n_score, s_end[pair] + a.lag);
    const int unit = pair * a.kv_per_idx + r / a.nsplit_max;
    a.items[ins + per_pair * pair + r] = make_int2(-1 - unit, r % a.nsplit_max);
  }
  // score item k follows the attention groups of every pair q with
  // end(q) + lag <= k
  for (int k = threadIdx.x; k < n_score; k += 1024) {
    const int pair = count_le(k);  // first pair whose end exceeds k
    const int start = pair > 0 ? s_end[pair - 1] : 0;
    a.items[k + per_pair * count_le(k - a.lag)] = make_int2(pair, k - start);
  }
  if (threadIdx.x == 0) *a.n_items = n_score + per_pair * npairs;
}

__global__ void fill_f32_kernel(float* p, int64_t n, float value) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[i] = value;
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

hipError_t launch_fill_f32(float* p, int64_t n, float value, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  fill_f32_kernel<<<static_cast<int>(blocks < 2048 ? blocks : 2048), 256, 0, s>>>(p, n, value);
  return hipGetLastError();
}

hipError_t launch_decode_plan(const PlanArgs& a, hipStream_t s) {
  decode_plan_kernel<<<1, 1024, 0, s>>>(a);
  return hipGetLastError();
}

template <class IT, int DI>
static void launch_score_t(const ScoreArgs& a, hipStream_t s) {
  const int grid = a.num_seqs * a.hidx * a.chunks_per_pair;
  decode_score_kernel<IT, DI><<<grid, kWgThreads, 0, s>>>(a);
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
