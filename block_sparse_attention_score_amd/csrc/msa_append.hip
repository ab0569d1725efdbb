// Paged append: the new tokens' K, V and index keys (and, with the
// index-value branch, index values) written into the pools at their token
// slots (the sglang page minimax_sparse_backend.py stores the
// new tokens into its pool at out_cache_loc before it attends; slot s is
// page s / 128, offset s % 128 of the head-major pages here).  fp8 pools
// receive the e4m3 (or e5m2) code of x / scale (per-tensor k_scale / v_scale,
// the vLLM page's fp8 cache scales): float32 division, clamp to the format's
// largest finite value (448 / 57344), round to nearest even by the gfx950
// conversion instruction.
//
// One thread moves 8 consecutive elements of one row (16-byte bf16 loads):
// the grid is flat over (token, 8-element vector of the token's Hkv K rows,
// Hkv V rows and Hidx index rows), so consecutive threads write consecutive
// 16-byte pieces of a row and no thread idles.  Memory-bound and tiny: one
// decode step appends B tokens.
#include "msa_device.h"
#include "msa_internal.h"

namespace msa {

template <class T>
struct Pack8;
template <>
struct Pack8<BF16> {
  uint4 v;
};
template <>
struct Pack8<F32> {
  float4 a, b;
};
template <>
struct Pack8<FP8> {
  uint2 v;
};

__device__ __forceinline__ void load8_plain(const BF16*, const void* p, int64_t i, float (&x)[8]) {
  const uint4 u = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(p) + i);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    x[2 * k] = __uint_as_float(w[k] << 16);
    x[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8_plain(const F32*, const void* p, int64_t i, float (&x)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p) + i);
  const float4 b = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p) + i + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

// Same storage type: the bytes are copied.
__device__ __forceinline__ void copy8(const BF16*, const void* s, int64_t si, void* d, int64_t di) {
  *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(d) + di) =
      *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(s) + si);
}
__device__ __forceinline__ void copy8(const F32*, const void* s, int64_t si, void* d, int64_t di) {
  const float4* sp = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(s) + si);
  float4* dp = reinterpret_cast<float4*>(reinterpret_cast<float*>(d) + di);
  dp[0] = sp[0];
  dp[1] = sp[1];
}

// e4m3 code of x / scale: float32 division (correctly rounded), clamp to the
// largest finite magnitude (NaN passes), round to nearest even.
__device__ __forceinline__ float fp8_prescale(float x, float scale) {
  const float y = x / scale;
  return y > 448.f ? 448.f : (y < -448.f ? -448.f : y);
}
__device__ __forceinline__ uint2 quant8(const FP8*, const float (&x)[8], float scale) {
  float y[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) y[k] = fp8_prescale(x[k], scale);
  int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
  w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w0, true);
  int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
  w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], w1, true);
  return uint2{static_cast<uint32_t>(w0), static_cast<uint32_t>(w1)};
}
// e5m2: clamp to its largest finite magnitude, 57344 (the code saturates
// rather than becoming inf), then round to nearest even.
__device__ __forceinline__ uint2 quant8(const BF8*, const float (&x)[8], float scale) {
  float y[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float v = x[k] / scale;
    y[k] = v > 57344.f ? 57344.f : (v < -57344.f ? -57344.f : v);
  }
  int w0 = __builtin_amdgcn_cvt_pk_bf8_f32(y[0], y[1], 0, false);
  w0 = __builtin_amdgcn_cvt_pk_bf8_f32(y[2], y[3], w0, true);
  int w1 = __builtin_amdgcn_cvt_pk_bf8_f32(y[4], y[5], 0, false);
  w1 = __builtin_amdgcn_cvt_pk_bf8_f32(y[6], y[7], w1, true);
  return uint2{static_cast<uint32_t>(w0), static_cast<uint32_t>(w1)};
}

// E2M1 code of y (already divided by its group's power-of-two scale): the
// nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6 (clamped at 6), an exact tie going to
// the even code; the sign is kept.  The count of midpoints below |y| is the
// magnitude code, each midpoint compared so that a tie lands on the even
// neighbour.
__device__ __forceinline__ uint32_t e2m1_code(float y) {
  const float m = fabsf(y);
  const uint32_t c = (m > 0.25f) + (m >= 0.75f) + (m > 1.25f) + (m >= 1.75f) + (m > 2.5f) +
                     (m >= 3.5f) + (m > 5.0f);
  return c | (__float_as_uint(y) >> 31 << 3);
}

// One 32-element group of an MX-fp4 row: y = x / tensor scale (float32
// division); the group's E8M0 scale is 2^(floor(log2 max|y|) - 2) (2 being
// E2M1's largest exponent), clamped to the code range (an all-zero group
// takes code 0); each element stores the E2M1 code of y / 2^(scale - 127);
// a group holding a NaN stores the NaN scale code and zero codes.
template <class KS>
__device__ void quant_group_fp4(const void* src, int64_t si, float tscale, uint8_t* codes16,
                                uint8_t* scale_byte) {
  float y[32];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float x[8];
    load8_plain(static_cast<const KS*>(nullptr), src, si + 8 * q, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) y[8 * q + e] = x[e] / tscale;
  }
  float amax = 0.f;
  bool nan = false;
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    nan |= y[e] != y[e];
    amax = fmaxf(amax, fabsf(y[e]));
  }
  const int k = amax > 0.f ? __builtin_amdgcn_frexp_expf(amax) - 3 : -127;
  const int sc = min(max(k + 127, 0), 254);
  uint32_t w[4] = {0u, 0u, 0u, 0u};
  if (!nan) {
#pragma unroll
    for (int e = 0; e < 32; ++e) w[e / 8] |= e2m1_code(ldexpf(y[e], 127 - sc)) << (4 * (e % 8));
  }
  *reinterpret_cast<uint4*>(codes16) = uint4{w[0], w[1], w[2], w[3]};
  *scale_byte = static_cast<uint8_t>(nan ? 255 : sc);
}

// E2M3 code of y (already divided by its group's power-of-two scale): the
// nearest of the 32 magnitudes (k / 8 below 2, k / 4 in [2, 4), k / 2 from 4
// to 7.5; clamped at 7.5), an exact tie going to the even code; the sign is
// kept.  Within each range the value times its code density is rounded to
// the nearest integer, ties to even (a power-of-two product, so exact), and
// the code is that integer plus the range's offset (0, 8, 16), which keeps
// the parity.
__device__ __forceinline__ uint32_t e2m3_code(float y) {
  const float m = fminf(fabsf(y), 7.5f);
  const float dens = m < 2.f ? 8.f : (m < 4.f ? 4.f : 2.f);
  const uint32_t off = m < 2.f ? 0u : (m < 4.f ? 8u : 16u);
  const uint32_t c = static_cast<uint32_t>(__builtin_rintf(m * dens)) + off;
  return c | (__float_as_uint(y) >> 31 << 5);
}

// One 32-element group of an MX-fp6 row, by the rule of quant_group_fp4 with
// E2M3 codes (2 is also E2M3's largest exponent): 24 code bytes (element e at
// bits 6 e of their little-endian value) and the scale byte.
template <class KS>
__device__ void quant_group_fp6(const void* src, int64_t si, float tscale, uint8_t* codes24,
                                uint8_t* scale_byte) {
  float y[32];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float x[8];
    load8_plain(static_cast<const KS*>(nullptr), src, si + 8 * q, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) y[8 * q + e] = x[e] / tscale;
  }
  float amax = 0.f;
  bool nan = false;
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    nan |= y[e] != y[e];
    amax = fmaxf(amax, fabsf(y[e]));
  }
  const int k = amax > 0.f ? __builtin_amdgcn_frexp_expf(amax) - 3 : -127;
  const int sc = min(max(k + 127, 0), 254);
  uint64_t w[3] = {0u, 0u, 0u};
  if (!nan) {
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const uint64_t c = e2m3_code(ldexpf(y[e], 127 - sc));
      const int pos = 6 * e;
      w[pos / 64] |= c << (pos % 64);
      if (pos % 64 > 58) w[pos / 64 + 1] |= c >> (64 - pos % 64);
    }
  }
#pragma unroll
  for (int i = 0; i < 3; ++i) reinterpret_cast<uint64_t*>(codes24)[i] = w[i];
  *scale_byte = static_cast<uint8_t>(nan ? 255 : sc);
}

// KS: storage of the new K/V rows; KP: of the K/V pools; IT: of the index
// keys (new rows and pool alike).  A K/V piece is 8 elements, or, for MX
// pools, one 32-element scale group.
template <class KS, class KP, class IT>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  constexpr int kPiece = __is_same(KP, FP4) || __is_same(KP, FP6) ? 32 : 8;
  const int vd = a.head_dim / kPiece;   // pieces per K/V row
  const int vi = a.idx_dim / 8;    // per index row
  const int n_kv = a.hkv * vd;
  const int n_iv = a.idx_v_pool != nullptr ? a.hidx * vi : 0;  // index-value pieces
  const int per_token = 2 * n_kv + a.hidx * vi + n_iv;
  const int64_t gi = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gi >= static_cast<int64_t>(a.num_tokens) * per_token) return;
  const int t = static_cast<int>(gi / per_token);
  const int i = static_cast<int>(gi - static_cast<int64_t>(t) * per_token);
  const int64_t slot = a.slots[t];
  if (slot < 0 || slot >= a.num_pages * kBlock) return;
  const int64_t page = slot / kBlock;
  const int off = static_cast<int>(slot - page * kBlock);
  if (i < 2 * n_kv) {
    const bool is_v = i >= n_kv;
    const int r = is_v ? i - n_kv : i;
    const int h = r / vd;
    const int c = r - h * vd;
    const void* src = is_v ? a.v_new : a.k_new;
    void* pool = is_v ? a.v_pool : a.k_pool;
    const int64_t si = (static_cast<int64_t>(t) * a.hkv + h) * a.head_dim + c * 8;
    const int64_t di = ((page * a.hkv + h) * kBlock + off) * a.head_dim + c * 8;
    if constexpr (__is_same(KP, FP4)) {
      uint8_t* run = reinterpret_cast<uint8_t*>(pool) + (page * a.hkv + h) * kFp4Run;
      quant_group_fp4<KS>(src, (static_cast<int64_t>(t) * a.hkv + h) * a.head_dim + c * 32,
                          is_v ? a.v_scale : a.k_scale, run + off * 64 + c * 16,
                          run + kFp4Codes + off * 4 + c);
    } else if constexpr (__is_same(KP, FP6)) {
      uint8_t* run = reinterpret_cast<uint8_t*>(pool) + (page * a.hkv + h) * kFp6Run;
      quant_group_fp6<KS>(src, (static_cast<int64_t>(t) * a.hkv + h) * a.head_dim + c * 32,
                          is_v ? a.v_scale : a.k_scale, run + off * 96 + c * 24,
                          run + kFp6Codes + off * 4 + c);
    } else if constexpr (__is_same(KP, FP8) || __is_same(KP, BF8)) {
      float x[8];
      load8_plain(static_cast<const KS*>(nullptr), src, si, x);
      *reinterpret_cast<uint2*>(reinterpret_cast<uint8_t*>(pool) + di) =
          quant8(static_cast<const KP*>(nullptr), x, is_v ? a.v_scale : a.k_scale);
    } else {
      copy8(static_cast<const KS*>(nullptr), src, si, pool, di);
    }
  } else {
    // index keys, then (index-value branch) index values
    int r = i - 2 * n_kv;
    const bool is_iv = r >= a.hidx * vi;
    if (is_iv) r -= a.hidx * vi;
    const int h = r / vi;
    const int c = r - h * vi;
    const int64_t si = (static_cast<int64_t>(t) * a.hidx + h) * a.idx_dim + c * 8;
    const int64_t di = ((page * a.hidx + h) * kBlock + off) * a.idx_dim + c * 8;
    copy8(static_cast<const IT*>(nullptr), is_iv ? a.idx_v_new : a.idx_k_new, si,
          is_iv ? a.idx_v_pool : a.idx_k_pool, di);
  }
}

template <class KS, class KP>
static void launch_append_i(const AppendArgs& a, int idx_dtype, dim3 grid, hipStream_t s) {
  if (idx_dtype == 1) append_kernel<KS, KP, F32><<<grid, 256, 0, s>>>(a);
  else append_kernel<KS, KP, BF16><<<grid, 256, 0, s>>>(a);
}

hipError_t launch_append(const AppendArgs& a, int kv_dtype, int idx_dtype, hipStream_t s) {
  if (a.num_tokens == 0) return hipSuccess;
  const int64_t per_token = 2 * a.hkv * (a.head_dim / (kv_dtype == 4 || kv_dtype == 5 ? 32 : 8)) +
                            (a.idx_v_pool != nullptr ? 2 : 1) * a.hidx * (a.idx_dim / 8);
  const int64_t blocks = (static_cast<int64_t>(a.num_tokens) * per_token + 255) / 256;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(blocks));
  if (kv_dtype == 0) launch_append_i<BF16, BF16>(a, idx_dtype, grid, s);
  else if (kv_dtype == 2) launch_append_i<BF16, FP8>(a, idx_dtype, grid, s);
  else if (kv_dtype == 3) launch_append_i<BF16, BF8>(a, idx_dtype, grid, s);
  else if (kv_dtype == 4) launch_append_i<BF16, FP4>(a, idx_dtype, grid, s);
  else if (kv_dtype == 5) launch_append_i<BF16, FP6>(a, idx_dtype, grid, s);
  else launch_append_i<F32, F32>(a, idx_dtype, grid, s);
  return hipGetLastError();
}

}  // namespace msa
