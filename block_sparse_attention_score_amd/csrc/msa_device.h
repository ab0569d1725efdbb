// Device helpers for the gfx950 kernels of libmsa: storage-type unpacking,
// wavefront reductions over 16-lane DPP rows, order-preserving score keys and
// 256-thread workgroup scans.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

constexpr int kBlock = 128;      // tokens per block == tokens per page
constexpr int kWave = 64;        // CDNA wavefront width
constexpr int kWgThreads = 256;  // 4 waves per workgroup

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Storage tags.
struct BF16 {};
struct F32 {};
struct FP8 {};   // OCP fp8 E4M3 ("e4m3fn") codes
struct BF8 {};   // OCP fp8 E5M2 codes
struct FP4 {};   // OCP MX-fp4: E2M1 codes with an E8M0 scale per 32 elements
struct FP6 {};   // OCP MX-fp6: E2M3 codes with an E8M0 scale per 32 elements

// MX-fp4 pools hold, per (page, head), the 128 x 128 / 2 code bytes (element
// 2i of a row in the low nibble of byte i) and then the 128 x 4 scale bytes.
constexpr int kFp4Codes = 128 * 128 / 2;
constexpr int kFp4Run = kFp4Codes + 128 * 4;
// MX-fp6 pools: per (page, head) the 128 x 96 code bytes (a 32-element group
// in 24 bytes, element i at bits 6 i .. 6 i + 5 of their little-endian value)
// and then the 128 x 4 scale bytes.
constexpr int kFp6Codes = 128 * 128 * 3 / 4;
constexpr int kFp6Run = kFp6Codes + 128 * 4;

// ---------------------------------------------------------------- loads

// Raw storage of eight consecutive elements, loaded with one (fp8, bf16) or
// two (f32) vector loads and widened to float only when used.
template <class T>
struct Raw8;
template <>
struct Raw8<BF16> {
  uint4 v;
};
template <>
struct Raw8<F32> {
  float4 a, b;
};
template <>
struct Raw8<FP8> {
  uint2 v;
};
template <>
struct Raw8<BF8> {
  uint2 v;
};

// Pages of the pools are streamed once per call: their loads are
// non-temporal, so they do not displace (or force the write-back of) lines
// that other work keeps in the L2 and the Infinity Cache.  On MI355X this
// about doubles the achieved read bandwidth of the page scans when the caches
// hold dirty data.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4v_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ Raw8<BF16> load_raw(const BF16*, const void* base,
                                               int64_t idx) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(
      reinterpret_cast<const uint16_t*>(base) + idx));
  return {uint4{v.x, v.y, v.z, v.w}};
}
__device__ __forceinline__ Raw8<F32> load_raw(const F32*, const void* base,
                                              int64_t idx) {
  const f32x4v_t* p = reinterpret_cast<const f32x4v_t*>(
      reinterpret_cast<const float*>(base) + idx);
  const f32x4v_t a = __builtin_nontemporal_load(p);
  const f32x4v_t b = __builtin_nontemporal_load(p + 1);
  return {float4{a.x, a.y, a.z, a.w}, float4{b.x, b.y, b.z, b.w}};
}
__device__ __forceinline__ Raw8<FP8> load_raw(const FP8*, const void* base,
                                              int64_t idx) {
  const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(
      reinterpret_cast<const uint8_t*>(base) + idx));
  return {uint2{v.x, v.y}};
}

__device__ __forceinline__ void unpack(const Raw8<BF16>& r, float (&x)[8]) {
  const uint32_t u[4] = {r.v.x, r.v.y, r.v.z, r.v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(u[i] << 16);
    x[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void unpack(const Raw8<F32>& r, float (&x)[8]) {
  x[0] = r.a.x; x[1] = r.a.y; x[2] = r.a.z; x[3] = r.a.w;
  x[4] = r.b.x; x[5] = r.b.y; x[6] = r.b.z; x[7] = r.b.w;
}

// OCP e4m3 codes -> float with the gfx950 conversion instruction (two codes
// per instruction, selected by word).
__device__ __forceinline__ void fp8x4_to_f32(uint32_t w, float* x) {
  const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), false);
  const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), true);
  x[0] = lo[0]; x[1] = lo[1]; x[2] = hi[0]; x[3] = hi[1];
}
__device__ __forceinline__ void unpack(const Raw8<FP8>& r, float (&x)[8]) {
  fp8x4_to_f32(r.v.x, x);
  fp8x4_to_f32(r.v.y, x + 4);
}
__device__ __forceinline__ Raw8<BF8> load_raw(const BF8*, const void* base, int64_t idx) {
  const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(
      reinterpret_cast<const uint8_t*>(base) + idx));
  return {uint2{v.x, v.y}};
}
// OCP e5m2 codes -> float (gfx950 conversion, two codes per instruction).
__device__ __forceinline__ void bf8x4_to_f32(uint32_t w, float* x) {
  const auto lo = __builtin_amdgcn_cvt_pk_f32_bf8(static_cast<int>(w), false);
  const auto hi = __builtin_amdgcn_cvt_pk_f32_bf8(static_cast<int>(w), true);
  x[0] = lo[0]; x[1] = lo[1]; x[2] = hi[0]; x[3] = hi[1];
}
__device__ __forceinline__ void unpack(const Raw8<BF8>& r, float (&x)[8]) {
  bf8x4_to_f32(r.v.x, x);
  bf8x4_to_f32(r.v.y, x + 4);
}

template <class T>
__device__ __forceinline__ void load8(const T* tag, const void* base, int64_t idx,
                                      float (&x)[8]) {
  unpack(load_raw(tag, base, idx), x);
}

// Four consecutive elements (8-, 4- or 16-byte non-temporal loads).
template <class T>
struct Raw4;
template <>
struct Raw4<BF16> {
  uint2 v;
};
template <>
struct Raw4<F32> {
  float4 v;
};
template <>
struct Raw4<FP8> {
  uint32_t v;
};

__device__ __forceinline__ Raw4<BF16> load_raw4(const BF16*, const void* base, int64_t idx) {
  const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(
      reinterpret_cast<const uint16_t*>(base) + idx));
  return {uint2{v.x, v.y}};
}
__device__ __forceinline__ Raw4<F32> load_raw4(const F32*, const void* base, int64_t idx) {
  const f32x4v_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4v_t*>(
      reinterpret_cast<const float*>(base) + idx));
  return {float4{v.x, v.y, v.z, v.w}};
}
__device__ __forceinline__ Raw4<FP8> load_raw4(const FP8*, const void* base, int64_t idx) {
  return {__builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(
      reinterpret_cast<const uint8_t*>(base) + idx))};
}

__device__ __forceinline__ void unpack4(const Raw4<BF16>& r, float (&x)[4]) {
  x[0] = __uint_as_float(r.v.x << 16);
  x[1] = __uint_as_float(r.v.x & 0xffff0000u);
  x[2] = __uint_as_float(r.v.y << 16);
  x[3] = __uint_as_float(r.v.y & 0xffff0000u);
}
__device__ __forceinline__ void unpack4(const Raw4<F32>& r, float (&x)[4]) {
  x[0] = r.v.x; x[1] = r.v.y; x[2] = r.v.z; x[3] = r.v.w;
}
__device__ __forceinline__ void unpack4(const Raw4<FP8>& r, float (&x)[4]) {
  fp8x4_to_f32(r.v, x);
}

// Eight fp8-e4m3 codes (two little-endian words) to bf16, exactly (every
// e4m3 value is a bf16 value; the scale operand is 1): the gfx950 packed
// conversion, one instruction per two codes.
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
  const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
  const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
  const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
  return bf16x8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Eight fp8-e5m2 codes to bf16, exactly (every e5m2 value, subnormals and
// infinities included, is a bf16 value): the gfx950 packed conversion.
__device__ __forceinline__ bf16x8_t bf8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w0, 1.0f, false);
  const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w0, 1.0f, true);
  const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w1, 1.0f, false);
  const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w1, 1.0f, true);
  return bf16x8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// E8M0 scale code -> float: 2^(code - 127) (code 0 is the float32 subnormal
// 2^-127), 0xFF -> NaN.
__device__ __forceinline__ float e8m0_to_f32(uint32_t code) {
  return code == 255u ? __uint_as_float(0x7fc00000u)
                      : (code == 0u ? __uint_as_float(0x00400000u) : __uint_as_float(code << 23));
}

// Eight E2M1 codes (one little-endian word, element 2i in the low nibble of
// byte i) times a scale, to bf16: the gfx950 scaled conversion, two codes per
// instruction (exact while the products are bf16 values: every E2M1 value
// times a power of two in bf16's range is one).
__device__ __forceinline__ bf16x8_t fp4x8_to_bf16x8(uint32_t w, float scale) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0);
  const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1);
  const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2);
  const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3);
  return bf16x8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// One 32-element E2M3 group (its 24 bytes in the low six words) times a
// scale, to bf16, in one gfx950 scaled conversion (exact for the same reason
// as E2M1: every E2M3 value times a power of two in bf16's range is a bf16
// value).
typedef int i32x6_t __attribute__((ext_vector_type(6)));
typedef __bf16 bf16x32_t __attribute__((ext_vector_type(32)));
__device__ __forceinline__ bf16x32_t fp6x32_to_bf16x32(const uint32_t (&w)[6], float scale) {
  const i32x6_t v = {static_cast<int>(w[0]), static_cast<int>(w[1]), static_cast<int>(w[2]),
                     static_cast<int>(w[3]), static_cast<int>(w[4]), static_cast<int>(w[5])};
  return __builtin_amdgcn_cvt_scalef32_pk32_bf16_fp6(v, scale);
}
// Elements 8 c .. 8 c + 7 of a converted group.
__device__ __forceinline__ bf16x8_t bf16x32_part(const bf16x32_t& v, int c) {
  return bf16x8_t{v[8 * c], v[8 * c + 1], v[8 * c + 2], v[8 * c + 3],
                  v[8 * c + 4], v[8 * c + 5], v[8 * c + 6], v[8 * c + 7]};
}

// Eight consecutive elements packed as bf16 for an MFMA operand.  fp8 codes
// convert exactly (every e4m3 value is a bf16 value).
__device__ __forceinline__ bf16x8_t load8_bf16(const BF16*, const void* base,
                                               int64_t idx) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(
      reinterpret_cast<const uint16_t*>(base) + idx));
  bf16x8_t r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}


// float -> bf16 bits, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40);
  return static_cast<uint16_t>((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// ------------------------------------------------------------ DPP rows

// DPP control words (GFX9 encoding).
constexpr int kDppXor1 = 0xB1;          // quad_perm(1,0,3,2)
constexpr int kDppXor2 = 0x4E;          // quad_perm(2,3,0,1)
constexpr int kDppHalfMirror = 0x141;   // lane i <- lane 7-i within 8
constexpr int kDppMirror = 0x140;       // lane i <- lane 15-i within 16

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over groups of N consecutive lanes (N in {8, 16}); every lane of the
// group receives the group's sum.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  v += dpp_f<kDppXor1>(v);
  v += dpp_f<kDppXor2>(v);
  v += dpp_f<kDppHalfMirror>(v);
  if constexpr (N == 16) v += dpp_f<kDppMirror>(v);
  return v;
}

template <int N>
__device__ __forceinline__ float group_max(float v) {
  v = fmaxf(v, dpp_f<kDppXor1>(v));
  v = fmaxf(v, dpp_f<kDppXor2>(v));
  v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
  if constexpr (N == 16) v = fmaxf(v, dpp_f<kDppMirror>(v));
  return v;
}

// Max over the whole wavefront, result in every lane.
__device__ __forceinline__ float wave_max(float v) {
  v = group_max<16>(v);
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}

// Sum over the whole wavefront, result in every lane.
__device__ __forceinline__ float wave_sum(float v) {
  v = group_sum<16>(v);
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

// ------------------------------------------------------- block scores
//
// A block's score from the index dots of its visible tokens, by score type:
// 0 max (the reading the spec fixes), 1 the mean, 2 the log-sum-exp of the
// dots times 1/sqrt(Di) (kept in base 2 while accumulating: c = log2(e) /
// sqrt(Di) scales the dots, the result is converted back).  A wave feeds each
// token's dot from every lane of its row; for the mean and the log-sum-exp
// only the row's owner lane counts it.
constexpr int kScoreMax = 0;
constexpr int kScoreMean = 1;
constexpr int kScoreLse = 2;
constexpr float kLn2d = 0.69314718055994531f;

template <int ST>
struct BlockScore;
template <>
struct BlockScore<kScoreMax> {
  float m = -INFINITY;
  template <int N>
  __device__ __forceinline__ void add(const float (&d)[N], const bool (&ok)[N], bool, float) {
#pragma unroll
    for (int i = 0; i < N; ++i) m = fmaxf(m, ok[i] ? d[i] : -INFINITY);
  }
  __device__ __forceinline__ float finish(int) { return wave_max(m); }
};
template <>
struct BlockScore<kScoreMean> {
  float s = 0.f;
  template <int N>
  __device__ __forceinline__ void add(const float (&d)[N], const bool (&ok)[N], bool owner, float) {
#pragma unroll
    for (int i = 0; i < N; ++i) s += (ok[i] && owner) ? d[i] : 0.f;
  }
  // nvalid: visible tokens of the block (none: the block is not visible)
  __device__ __forceinline__ float finish(int nvalid) {
    const float t = wave_sum(s);
    return nvalid > 0 ? t / static_cast<float>(nvalid) : -INFINITY;
  }
  // the same over the four lanes 16 apart that share a column of an MFMA
  // result tile (every lane counts its own tokens)
  __device__ __forceinline__ float finish_q4(int nvalid) {
    float t = s + __shfl_xor(s, 16);
    t += __shfl_xor(t, 32);
    return nvalid > 0 ? t / static_cast<float>(nvalid) : -INFINITY;
  }
};
template <>
struct BlockScore<kScoreLse> {
  float m = -INFINITY, e = 0.f;
  template <int N>
  __device__ __forceinline__ void add(const float (&d)[N], const bool (&ok)[N], bool owner,
                                      float c) {
    float z[N];
    float mb = m;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      z[i] = (ok[i] && owner) ? d[i] * c : -INFINITY;
      mb = fmaxf(mb, z[i]);
    }
    const float mu = mb == -INFINITY ? 0.f : mb;
    e *= __builtin_amdgcn_exp2f(m - mu);
#pragma unroll
    for (int i = 0; i < N; ++i) e += __builtin_amdgcn_exp2f(z[i] - mu);
    m = mb;
  }
  __device__ __forceinline__ float finish(int) {
    const float M = wave_max(m);
    const float mu = M == -INFINITY ? 0.f : M;
    const float E = wave_sum(e * __builtin_amdgcn_exp2f(m - mu));
    return E > 0.f ? (mu + __builtin_amdgcn_logf(E)) * kLn2d : -INFINITY;
  }
  __device__ __forceinline__ float finish_q4(int) {
    float M = fmaxf(m, __shfl_xor(m, 16));
    M = fmaxf(M, __shfl_xor(M, 32));
    const float mu = M == -INFINITY ? 0.f : M;
    float E = e * __builtin_amdgcn_exp2f(m - mu);
    E += __shfl_xor(E, 16);
    E += __shfl_xor(E, 32);
    return E > 0.f ? (mu + __builtin_amdgcn_logf(E)) * kLn2d : -INFINITY;
  }
};

// --------------------------------------------------------- score keys

// Order-preserving map float -> uint32 (larger float, larger key); -0 and +0
// map to the same key so that they tie.
__device__ __forceinline__ uint32_t score_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ------------------------------------------------------- block scans

// Inclusive prefix sum over the threads of a workgroup (up to 1024).  `wsum`
// is LDS scratch of one int per wave.  Contains barriers: every thread must
// call it.
__device__ __forceinline__ int block_incl_scan(int v, int* wsum) {
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

__host__ __device__ constexpr int div_up(int a, int b) { return (a + b - 1) / b; }

// max(a, b) that propagates NaN (v_maximum_f32 / v_maximum3_f32 on gfx950).
// fmaxf must first quiet a signalling NaN, so every MFMA result it takes
// costs one more VALU instruction; the maxima below only ever see finite
// scores or -inf (masked entries are replaced before the max).
__device__ __forceinline__ float max_nan(float a, float b) {
  return __builtin_elementwise_maximum(a, b);
}

// ------------------------------------------- cross-workgroup hand-off
//
// Workgroups of one launch hand results to the workgroup that finishes a unit
// last (atomic ticket).  The data travels only through relaxed device-scope
// atomic loads and stores, which the gfx950 memory model makes coherent across
// the XCDs' separate L2 caches by themselves (no whole-cache write-back or
// invalidate, which agent-scope fences would issue per wave).  A writer waits
// for its stores to complete before it takes a ticket; the last taker reads
// only after its ticket returned.

__device__ __forceinline__ void store_shared_f32(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_shared_f32(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// All of this wave's memory operations have completed.
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0); }

// Ticket of a unit of `parts` workgroups; returns true in every thread of the
// workgroup that took the last ticket.  Every thread must call it after its
// last hand-off store.
__device__ __forceinline__ bool take_last_ticket(uint32_t* ticket, int parts, int* lds_flag) {
  wait_stores();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev =
        __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *lds_flag = prev == static_cast<uint32_t>(parts - 1);
  }
  __syncthreads();
  return *lds_flag != 0;
}

}  // namespace msa
