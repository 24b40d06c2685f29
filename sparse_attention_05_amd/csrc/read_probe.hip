// dsa_read_probe: a plain streaming read of a device buffer, the reference
// rate for a kernel that reads its operand once from HBM (the indexer's key
// stream, which is nearly all of a decode step's bytes). No part of the
// method: it sets the attainable read rate beside the published peak.
#include <stdint.h>

#include "dsa.h"
#include "dsa_common.hpp"
#include "dsa_internal.hpp"

namespace dsa {
namespace {

constexpr int kProbeThreads = 512;

// One workgroup per CU; thread t of the grid reads the 16-byte pieces
// t, t + G, t + 2G, ... (G threads in the grid) four at a time, so every
// load of the grid is one contiguous sweep; each workgroup writes the sum
// of the floats it read (the loads cannot be dropped).
__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const float4* __restrict__ p, int64_t n16,
                                                                   float* out) {
  __shared__ float s_w[kProbeThreads / 64];
  const int64_t stride = int64_t(gridDim.x) * kProbeThreads;
  int64_t i = int64_t(blockIdx.x) * kProbeThreads + threadIdx.x;
  float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const float4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
    s0 += (a.x + a.y) + (a.z + a.w);
    s1 += (b.x + b.y) + (b.z + b.w);
    s2 += (c.x + c.y) + (c.z + c.w);
    s3 += (d.x + d.y) + (d.z + d.w);
  }
  for (; i < n16; i += stride) {
    const float4 a = p[i];
    s0 += (a.x + a.y) + (a.z + a.w);
  }
  float s = (s0 + s1) + (s2 + s3);
  for (int d = 32; d > 0; d >>= 1) s += __shfl_xor(s, d, 64);
  if ((threadIdx.x & 63) == 0) s_w[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.f;
    for (int w = 0; w < kProbeThreads / 64; ++w) t += s_w[w];
    out[blockIdx.x] = t;
  }
}

}  // namespace
}  // namespace dsa

extern "C" int32_t dsa_read_probe_blocks(void) { return dsa::device_cu_count(); }

extern "C" dsa_status dsa_read_probe(const void* buf, uint64_t bytes, float* out, int32_t out_len, void* stream) {
  if (!buf || !out) return DSA_ERR_NULL;
  if (bytes == 0 || bytes % 16 != 0) return DSA_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(buf) & 15u) != 0 || (reinterpret_cast<uintptr_t>(out) & 3u) != 0)
    return DSA_ERR_ALIGN;
  const int G = dsa::device_cu_count();
  if (out_len < G) return DSA_ERR_SHAPE;
  dsa::read_probe_kernel<<<dim3(unsigned(G)), dsa::kProbeThreads, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const float4*>(buf), int64_t(bytes / 16), out);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? DSA_OK : static_cast<dsa_status>(dsa::record_hip_error(e));
}
