// Decode attention over a given selection (step 3 on its own): one
// workgroup per (split, kv head, sequence).
#include "msa_attend.h"

namespace msa {

// Eight waves per workgroup: with one workgroup per CU (the split sizing
// aims at that), two waves per SIMD stream blocks.
constexpr int kAttendWaves = 8;

// Workgroup i runs on XCD i % 8; each XCD takes a contiguous run of
// (token, kv head, split) units (`per` of them), so the splits of a row and
// the neighbouring tokens of a sequence share one L2.
template <class QT, class KT, int G>
__global__ __launch_bounds__(kWave * kAttendWaves, 1) void decode_attend_kernel(AttendArgs a,
                                                                                int per) {
  __shared__ AttendLds<G, kAttendWaves> lds;
  const int u = static_cast<int>(blockIdx.x % 8) * per + static_cast<int>(blockIdx.x / 8);
  const int per_tok = a.nsplit_max * a.hkv;
  if (u >= per_tok * a.num_tokens) return;
  const int t = u / per_tok;
  const int r = u - t * per_tok;
  attend_split<QT, KT, G, kAttendWaves>(a, r % a.nsplit_max, r / a.nsplit_max, t, lds);
}

// ------------------------------------------------------------ launcher

template <class QT, class KT, int G>
static void launch_attend_t(const AttendArgs& a, hipStream_t s) {
  const int units = a.nsplit_max * a.hkv * a.num_tokens;
  const int per = (units + 7) / 8;
  decode_attend_kernel<QT, KT, G><<<8 * per, kWave * kAttendWaves, 0, s>>>(a, per);
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
  if (a.num_tokens == 0) return hipSuccess;
  // the 1-D grid holds all units rounded up to a multiple of 8, in 32 bits
  if (int64_t(a.nsplit_max) * a.hkv * a.num_tokens > int64_t(0x7fffffff) - 7)
    return hipErrorInvalidValue;
  bool ok = false;
  if (q_dtype == 0 && kv_dtype == 0) ok = launch_attend_g<BF16, BF16>(a, group, s);
  else if (q_dtype == 0 && kv_dtype == 2) ok = launch_attend_g<BF16, FP8>(a, group, s);
  else if (q_dtype == 0 && kv_dtype == 3) ok = launch_attend_g<BF16, BF8>(a, group, s);
  else if (q_dtype == 0 && kv_dtype == 4) ok = launch_attend_g<BF16, FP4>(a, group, s);
  else if (q_dtype == 0 && kv_dtype == 5) ok = launch_attend_g<BF16, FP6>(a, group, s);
  else if (q_dtype == 1 && kv_dtype == 1) ok = launch_attend_g<F32, F32>(a, group, s);
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace msa
