// dsa_check_indices: a debug validator of index arrays (the structure the
// top-k guarantees, checked on the device without the scores): for query r
// with n = q_pos[r] + 1 candidates and k_eff = min(k, n), the first k_eff
// entries are distinct positions in [0, n) and the rest are -1.
#include <stdint.h>

#include "dsa.h"
#include "dsa_common.hpp"
#include "dsa_internal.hpp"

namespace dsa {
namespace {

constexpr int kCheckThreads = 256;

// One workgroup per row: the row's first k_eff entries sorted in LDS
// (bitonic, ascending, padded with INT_MAX), then every thread counts the
// out-of-range entries, the equal neighbours and the bad padding in its
// share; the row's count is added to *n_bad.
__global__ __launch_bounds__(kCheckThreads) void check_indices_kernel(const int32_t* idx, const int32_t* q_pos,
                                                                      int k, int32_t* n_bad) {
  __shared__ int32_t s[DSA_MAX_TOPK];
  __shared__ int32_t s_cnt[kCheckThreads / 64];
  const int r = blockIdx.x;
  const int t = threadIdx.x;
  const int64_t n = int64_t(q_pos[r]) + 1;
  const int k_eff = n <= 0 ? 0 : (n < k ? int(n) : k);
  const int32_t* row = idx + int64_t(r) * k;
  int P = 1;
  while (P < k_eff) P <<= 1;
  int bad = 0;
  for (int j = t; j < P; j += kCheckThreads) {
    int32_t v = 0x7FFFFFFF;
    if (j < k_eff) {
      v = row[j];
      bad += (v < 0 || int64_t(v) >= n) ? 1 : 0;
    }
    s[j] = v;
  }
  for (int j = k_eff + t; j < k; j += kCheckThreads) bad += row[j] != -1 ? 1 : 0;
  __syncthreads();
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = t; i < P / 2; i += kCheckThreads) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool up = (lo & size) == 0;
        const int32_t a = s[lo], b = s[hi];
        if ((a > b) == up) {
          s[lo] = b;
          s[hi] = a;
        }
      }
      __syncthreads();
    }
  }
  // repeats of valid positions (out-of-range ones are counted above)
  for (int j = t + 1; j < k_eff; j += kCheckThreads) bad += (s[j] == s[j - 1] && s[j] >= 0 && int64_t(s[j]) < n) ? 1 : 0;
  // workgroup sum, then one atomic per row
  for (int d = 32; d > 0; d >>= 1) bad += __shfl_xor(bad, d, 64);
  if ((t & 63) == 0) s_cnt[t >> 6] = bad;
  __syncthreads();
  if (t == 0) {
    int total = 0;
    for (int w = 0; w < kCheckThreads / 64; ++w) total += s_cnt[w];
    if (total) atomicAdd(n_bad, total);
  }
}

}  // namespace
}  // namespace dsa

extern "C" dsa_status dsa_check_indices(const int32_t* idx, const int32_t* q_pos, int32_t R, int32_t k,
                                        int32_t* n_bad, void* stream) {
  if (!n_bad || (R > 0 && (!idx || !q_pos))) return DSA_ERR_NULL;
  if (R < 0) return DSA_ERR_SHAPE;
  if (k < 1 || k > DSA_MAX_TOPK) return DSA_ERR_UNSUPPORTED;
  if (R == 0) return DSA_OK;
  dsa::check_indices_kernel<<<dim3(unsigned(R)), dsa::kCheckThreads, 0, static_cast<hipStream_t>(stream)>>>(
      idx, q_pos, k, n_bad);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? DSA_OK : static_cast<dsa_status>(dsa::record_hip_error(e));
}
