// The decode path in one persistent launch: score every block, select, and
// attend over the selection, with the attention of a (sequence, kv head)
// unit starting as soon as its index head's selection is done.
//
// Work items are claimed in order from one atomic counter: first the score
// items of the planner's list (pair-major, so pairs complete early and in
// turn), then the attention splits of every unit.  A split waits for its
// pair's ready flag before it reads the selection.  The wait always ends: a
// split is claimed only after every score item has been claimed by a
// workgroup that is already running, and score items never wait on anything,
// so every pair's selection is published.  The wait is still bounded (the
// workgroup proceeds after about 0.2 s), so a broken invariant cannot hang
// the device.
#include "msa_attend.h"
#include "msa_score.h"

namespace msa {

constexpr int kSpinLimit = 1 << 22;

__device__ __forceinline__ void wait_ready(const uint32_t* flag, int* lds_flag) {
  if (threadIdx.x == 0) {
    int seen = 0;
    for (int it = 0; it < kSpinLimit; ++it) {
      if (__hip_atomic_load(const_cast<uint32_t*>(flag), __ATOMIC_RELAXED,
                            __HIP_MEMORY_SCOPE_AGENT) != 0u) {
        seen = 1;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    *lds_flag = seen;
  }
  __syncthreads();
}

template <class IT, int DI, class QT, class KT, int G>
__global__ __launch_bounds__(kWgThreads, 2) void decode_fused_kernel(ScoreArgs sa, AttendArgs aa,
                                                                  FusedArgs fa) {
  __shared__ union Lds {
    SelectLds sel;
    AttendLds<G> att;
  } lds;
  __shared__ int x_s, y_s, flag;
  const int total = *fa.n_items;
  for (;;) {
    if (threadIdx.x == 0) {
      const int it = static_cast<int>(
          __hip_atomic_fetch_add(fa.counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
      if (it < total) {
        const int2 xy = fa.items[it];
        x_s = xy.x;
        y_s = xy.y;
      } else {
        x_s = INT32_MIN;
      }
    }
    __syncthreads();
    const int x = x_s;
    const int y = y_s;
    if (x == INT32_MIN) return;
    if (x >= 0) {
      score_chunk<IT, DI, 32, true>(sa, x, y, lds.sel, &flag);
    } else {
      const int unit = -1 - x;
      const int b = unit / aa.hkv;
      const int g = unit - b * aa.hkv;
      wait_ready(sa.ready + b * aa.hidx + g / (aa.hkv / aa.hidx), &flag);
      attend_split<QT, KT, G, true>(aa, y, g, b, lds.att);
    }
    __syncthreads();
  }
}

// Resident workgroups of `kernel` on the current device.
static int resident_grid(const void* kernel) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kWgThreads, 0) != hipSuccess ||
      cus <= 0 || per_cu <= 0)
    return 256;
  return cus * per_cu;
}

template <class IT, int DI, class QT, class KT, int G>
static int fused_grid() {
  static int grid = 0;  // per instantiation; every device here is the same part
  if (grid == 0) grid = resident_grid(reinterpret_cast<const void*>(decode_fused_kernel<IT, DI, QT, KT, G>));
  return grid;
}

template <class IT, int DI, class QT, class KT, int G>
static void launch_fused_t(const ScoreArgs& sa, const AttendArgs& aa, const FusedArgs& fa,
                           hipStream_t s) {
  decode_fused_kernel<IT, DI, QT, KT, G><<<fused_grid<IT, DI, QT, KT, G>(), kWgThreads, 0, s>>>(
      sa, aa, fa);
}

// Calls f.run<IT, DI, QT, KT, G>() for the kernel instantiation of a call.
template <class F, class IT, int DI, class QT, class KT>
static bool dispatch_g(int group, F& f) {
  switch (group) {
    case 1: f.template run<IT, DI, QT, KT, 1>(); return true;
    case 2: f.template run<IT, DI, QT, KT, 2>(); return true;
    case 4: f.template run<IT, DI, QT, KT, 4>(); return true;
    case 8: f.template run<IT, DI, QT, KT, 8>(); return true;
    case 16: f.template run<IT, DI, QT, KT, 16>(); return true;
    default: return false;
  }
}

template <class F, class IT, int DI>
static bool dispatch_qkv(int q_dtype, int kv_dtype, int group, F& f) {
  if (q_dtype == 0 && kv_dtype == 0) return dispatch_g<F, IT, DI, BF16, BF16>(group, f);
  if (q_dtype == 0 && kv_dtype == 2) return dispatch_g<F, IT, DI, BF16, FP8>(group, f);
  if (q_dtype == 1 && kv_dtype == 1) return dispatch_g<F, IT, DI, F32, F32>(group, f);
  return false;
}

template <class F>
static bool dispatch(int idx_dtype, int idx_dim, int q_dtype, int kv_dtype, int group, F& f) {
  if (idx_dim == 128)
    return idx_dtype == 1 ? dispatch_qkv<F, F32, 128>(q_dtype, kv_dtype, group, f)
                          : dispatch_qkv<F, BF16, 128>(q_dtype, kv_dtype, group, f);
  return idx_dtype == 1 ? dispatch_qkv<F, F32, 64>(q_dtype, kv_dtype, group, f)
                        : dispatch_qkv<F, BF16, 64>(q_dtype, kv_dtype, group, f);
}

struct GridQuery {
  int grid = 0;
  template <class IT, int DI, class QT, class KT, int G>
  void run() {
    grid = fused_grid<IT, DI, QT, KT, G>();
  }
};

struct Launcher {
  const ScoreArgs& sa;
  const AttendArgs& aa;
  const FusedArgs& fa;
  hipStream_t s;
  template <class IT, int DI, class QT, class KT, int G>
  void run() {
    launch_fused_t<IT, DI, QT, KT, G>(sa, aa, fa, s);
  }
};

int decode_fused_grid(int idx_dtype, int idx_dim, int q_dtype, int kv_dtype, int group) {
  GridQuery q;
  return dispatch(idx_dtype, idx_dim, q_dtype, kv_dtype, group, q) ? q.grid : 0;
}

hipError_t launch_decode_fused(const ScoreArgs& sa, const AttendArgs& aa, const FusedArgs& fa,
                               int idx_dtype, int idx_dim, int q_dtype, int kv_dtype, int group,
                               hipStream_t s) {
  Launcher l{sa, aa, fa, s};
  if (!dispatch(idx_dtype, idx_dim, q_dtype, kv_dtype, group, l)) return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace msa
