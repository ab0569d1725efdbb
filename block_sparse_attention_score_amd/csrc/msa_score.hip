// Standalone kernels: decode block scoring, per-row selection (step 2 alone),
// fills and fp8 dequantisation.
#include "msa_score.h"
#include "msa_select.h"

namespace msa {

// One workgroup per (pair, chunk); scores only.
template <class IT, int DI, int ST>
__global__ __launch_bounds__(kWgThreads) void decode_score_kernel(ScoreArgs a) {
  if (blockIdx.x == 0 && a.zero_words != nullptr)
    for (int i = threadIdx.x; i < a.zero_count; i += kWgThreads) a.zero_words[i] = 0u;
  const int pair = blockIdx.x / a.chunks_per_pair;
  score_chunk<IT, DI, ST>(a, pair, blockIdx.x - pair * a.chunks_per_pair);
}

// The same grid with the index-value branch on: scores and value partials.
template <class IT, int DI, int ST>
__global__ __launch_bounds__(kWgThreads) void decode_score_value_kernel(ScoreArgs a) {
  __shared__ IvLds<DI> lds;
  if (blockIdx.x == 0 && a.zero_words != nullptr)
    for (int i = threadIdx.x; i < a.zero_count; i += kWgThreads) a.zero_words[i] = 0u;
  const int pair = blockIdx.x / a.chunks_per_pair;
  score_value_chunk<IT, DI, ST>(a, pair, blockIdx.x - pair * a.chunks_per_pair, lds);
}

// Short chunks: one workgroup per (pair, chunk), every query of the pair's
// sequence.
template <class IT, int DI, int ST>
__global__ __launch_bounds__(kWgThreads) void multi_score_kernel(ScoreArgs a) {
  const int pair = blockIdx.x / a.chunks_per_pair;
  score_chunk_multi<IT, DI, 4, ST>(a, pair, blockIdx.x - pair * a.chunks_per_pair);
}

// One workgroup per (query token, index head) row.
template <int MAXPER>
__global__ __launch_bounds__(kWgThreads) void select_kernel(SelectArgs a) {
  __shared__ SelectLds sl;
  if (a.zero_words != nullptr) clear_words(a);
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
  select_row<MAXPER>(a.scores + static_cast<int64_t>(rowi) * a.max_blocks, nb,
                     topk_beside_forced(a.topk, nb, a.init, a.local, a.forced_in_budget),
                     a.init, a.local, a.kmax, a.sel + static_cast<int64_t>(rowi) * a.kmax,
                     a.cnt + rowi, sl);
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

// fp8 codes -> float32, through the same packed conversions to bf16 the
// attention loaders use (exact for both formats), widened exactly to float32
// and multiplied by the scale.
template <class K8>
__global__ void fp8_dequant_kernel(const uint8_t* in, float* out, int64_t n, float scale) {
  const int64_t i = (blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x) * 8;
  if (i >= n) return;
  uint32_t w[2] = {0u, 0u};
  for (int k = 0; k < 8 && i + k < n; ++k) w[k / 4] |= static_cast<uint32_t>(in[i + k]) << (8 * (k % 4));
  const bf16x8_t v = __is_same(K8, BF8) ? bf8x8_to_bf16x8(w[0], w[1]) : fp8x8_to_bf16x8(w[0], w[1]);
  for (int k = 0; k < 8 && i + k < n; ++k) out[i + k] = static_cast<float>(v[k]) * scale;
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


template <class IT, int DI, int ST>
static void launch_score_t(const ScoreArgs& a, hipStream_t s) {
  const int grid = a.num_seqs * a.hidx * a.chunks_per_pair;
  if (a.idx_v != nullptr)
    decode_score_value_kernel<IT, DI, ST><<<grid, kWgThreads, 0, s>>>(a);
  else
    decode_score_kernel<IT, DI, ST><<<grid, kWgThreads, 0, s>>>(a);
}

template <int ST>
static void launch_score_st(const ScoreArgs& a, int idx_dtype, int idx_dim, hipStream_t s) {
  const bool f32 = idx_dtype == 1;
  if (idx_dim == 128) {
    if (f32) launch_score_t<F32, 128, ST>(a, s); else launch_score_t<BF16, 128, ST>(a, s);
  } else {
    if (f32) launch_score_t<F32, 64, ST>(a, s); else launch_score_t<BF16, 64, ST>(a, s);
  }
}

hipError_t launch_decode_score(const ScoreArgs& a, int idx_dtype, int idx_dim, int score_type,
                               hipStream_t s) {
  if (a.num_seqs * a.hidx * a.chunks_per_pair == 0) return hipSuccess;
  if (score_type == kScoreMean) launch_score_st<kScoreMean>(a, idx_dtype, idx_dim, s);
  else if (score_type == kScoreLse) launch_score_st<kScoreLse>(a, idx_dtype, idx_dim, s);
  else launch_score_st<kScoreMax>(a, idx_dtype, idx_dim, s);
  return hipGetLastError();
}

template <int ST>
static void launch_multi_st(const ScoreArgs& a, int idx_dim, int grid, hipStream_t s) {
  if (idx_dim == 128) multi_score_kernel<BF16, 128, ST><<<grid, kWgThreads, 0, s>>>(a);
  else multi_score_kernel<BF16, 64, ST><<<grid, kWgThreads, 0, s>>>(a);
}

hipError_t launch_multi_score(const ScoreArgs& a, int idx_dim, int score_type, hipStream_t s) {
  const int grid = a.num_seqs * a.hidx * a.chunks_per_pair;
  if (grid == 0) return hipSuccess;
  if (score_type == kScoreMean) launch_multi_st<kScoreMean>(a, idx_dim, grid, s);
  else if (score_type == kScoreLse) launch_multi_st<kScoreLse>(a, idx_dim, grid, s);
  else launch_multi_st<kScoreMax>(a, idx_dim, grid, s);
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

// MX-fp4: n / 2 code bytes, then n / 32 scale bytes; 8 elements per thread.
__global__ void fp4_dequant_kernel(const uint8_t* in, float* out, int64_t n, float scale) {
  const int64_t i = (blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x) * 8;
  if (i >= n) return;
  const uint32_t w = *reinterpret_cast<const uint32_t*>(in + i / 2);
  const bf16x8_t v = fp4x8_to_bf16x8(w, e8m0_to_f32(in[n / 2 + i / 32]));
  for (int k = 0; k < 8; ++k) out[i + k] = static_cast<float>(v[k]) * scale;
}

// MX-fp6: 3 n / 4 code bytes, then n / 32 scale bytes; one 32-element group
// per thread (byte copies: the buffer's alignment is not known).
__global__ void fp6_dequant_kernel(const uint8_t* in, float* out, int64_t n, float scale) {
  const int64_t grp = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
  if (grp * 32 >= n) return;
  uint32_t w[6];
  __builtin_memcpy(w, in + grp * 24, 24);
  const bf16x32_t v = fp6x32_to_bf16x32(w, e8m0_to_f32(in[n / 32 * 24 + grp]));
  for (int k = 0; k < 32; ++k) out[grp * 32 + k] = static_cast<float>(v[k]) * scale;
}

hipError_t launch_fp8_dequant(const uint8_t* in, float* out, int64_t n, float scale, int dtype,
                              hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t threads = (n + 7) / 8;
  const int64_t blocks = (threads + 255) / 256;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (dtype == 5) {
    const int64_t groups = n / 32;
    const int64_t gblocks = (groups + 255) / 256;
    if (gblocks > 0) fp6_dequant_kernel<<<static_cast<unsigned>(gblocks), 256, 0, s>>>(in, out, n, scale);
  } else if (dtype == 4)
    fp4_dequant_kernel<<<static_cast<unsigned>(blocks), 256, 0, s>>>(in, out, n, scale);
  else if (dtype == 3)
    fp8_dequant_kernel<BF8><<<static_cast<unsigned>(blocks), 256, 0, s>>>(in, out, n, scale);
  else
    fp8_dequant_kernel<FP8><<<static_cast<unsigned>(blocks), 256, 0, s>>>(in, out, n, scale);
  return hipGetLastError();
}

}  // namespace msa
