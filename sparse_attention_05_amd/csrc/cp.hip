// Context parallelism over key ranges, rehearsed on one device: each shard
// holds keys [lo, hi) of every sequence, selects its local top-k, and the
// shards' (score, key) lists are merged into the global selection; each shard
// attends over the global winners it holds and the partial attentions are
// merged by their log-sum-exp ("GLM-5: from Vibe Coding to Agentic
// Engineering", section 2.4.2: context-parallel groups for long sequences).
// The selection order (score descending, lower key first, -0 == +0) is total
// and shards hold disjoint keys, so the merged selection equals the unsharded
// one exactly; the output merge runs in shard order, so it is deterministic
// for a fixed shard count.
#include "dsa.h"
#include "dsa_common.hpp"
#include "dsa_internal.hpp"

namespace dsa {
namespace {

constexpr int kMergeThreads = 512;
constexpr int kMergeMaxWords = 16384;  // P * k words of 8 bytes in LDS
constexpr int kMaxShards = 8;

// pair_score[r, j] = scores[r, idx[r, j]], pair_idx[r, j] = idx[r, j] + offset
// (-inf and -1 where idx is -1).
__global__ __launch_bounds__(256) void topk_pairs_kernel(const float* scores, int64_t ld, const int32_t* idx,
                                                         int R, int k, int offset, float* ps, int32_t* pi) {
  const int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (e >= int64_t(R) * k) return;
  const int64_t r = e / k;
  const int i = idx[e];
  ps[e] = i >= 0 ? scores[r * ld + i] : -INFINITY;
  pi[e] = i >= 0 ? i + offset : -1;
}

// Global top-k of P lists of k (score, key) pairs per row, each list in rank
// order with its empty entries (key -1) last: candidate j of list p, as the
// word key(score) << 32 | ~key, has global rank j + sum over the other lists
// of their words above it (binary searches in LDS, the P of a candidate
// interleaved). Workgroup (row, part) ranks part `part` of the row's
// candidates; workgroup part 0 also writes -1 past the last valid rank.
__global__ __launch_bounds__(kMergeThreads) void topk_merge_kernel(const float* ps, const int32_t* pi, int P, int R,
                                                                   int k, int parts, int32_t* out) {
  __shared__ unsigned long long w[kMergeMaxWords];
  __shared__ int s_valid[8];
  const int r = blockIdx.x / parts;
  const int part = blockIdx.x % parts;
  const int m = P * k;
  int valid = 0;
  // the words, 8 per thread per batch with all their loads in flight
  for (int e0 = 0; e0 < m; e0 += 8 * kMergeThreads) {
    int iv[8];
    float sv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = e0 + u * kMergeThreads + threadIdx.x;
      const int p = e / k;
      const int64_t g = (int64_t(p) * R + r) * k + (e - p * k);
      iv[u] = e < m ? pi[g] : -1;
      sv[u] = e < m ? ps[g] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = e0 + u * kMergeThreads + threadIdx.x;
      if (e < m)
        w[e] = iv[u] >= 0 ? (static_cast<unsigned long long>(order_key(sv[u])) << 32) | static_cast<uint32_t>(~iv[u])
                          : 0ull;
      valid += iv[u] >= 0;
    }
  }
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) valid += __shfl_xor(valid, d, 64);
  if ((threadIdx.x & 63) == 0) s_valid[threadIdx.x >> 6] = valid;
  __syncthreads();
  int32_t* row = out + int64_t(r) * k;
  if (part == 0) {
    int n = 0;
    for (int i = 0; i < kMergeThreads / 64; ++i) n += s_valid[i];
    for (int j = (n < k ? n : k) + threadIdx.x; j < k; j += kMergeThreads) row[j] = -1;
  }
  const int per = (m + parts - 1) / parts;
  const int e0 = part * per;
  const int e1 = e0 + per < m ? e0 + per : m;
  int steps = 0;  // binary-search steps over a list of k
  while ((1 << steps) < k + 1) ++steps;
  for (int e = e0 + threadIdx.x; e < e1; e += kMergeThreads) {
    const unsigned long long x = w[e];
    if (x == 0ull) continue;
    const int p = e / k;
    // lo[q]: count of list q's words above x (they form a prefix)
    int lo[8], hi[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      lo[q] = 0;
      hi[q] = q < P && q != p ? k : 0;
    }
    for (int s = 0; s < steps; ++s) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if (lo[q] < hi[q]) {
          const int mid = (lo[q] + hi[q]) >> 1;
          if (w[q * k + mid] > x) lo[q] = mid + 1;
          else hi[q] = mid;
        }
      }
    }
    int rank = e - p * k;
#pragma unroll
    for (int q = 0; q < 8; ++q) rank += lo[q];
    if (rank < k) row[rank] = static_cast<int32_t>(~static_cast<uint32_t>(x));
  }
}

// idx_local[r, j] = idx[r, j] - lo where lo <= idx[r, j] < hi, else -1.
__global__ __launch_bounds__(256) void shard_indices_kernel(const int32_t* idx, int64_t n, int lo, int hi,
                                                            int32_t* out) {
  const int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (e >= n) return;
  const int i = idx[e];
  out[e] = i >= lo && i < hi ? i - lo : -1;
}

// One thread per (row, head, 4 output dims): the P partial outputs weighted
// by exp(LSE_p - max), in shard order; parts with no key (LSE -inf) add
// nothing.
__global__ __launch_bounds__(256) void attn_merge_kernel(const float* o_parts, const float* lse_parts, int P, int R,
                                                         int H, float* out, float* lse) {
  const int64_t gid = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int64_t total = int64_t(R) * H * (kValueDim / 4);
  if (gid >= total) return;
  const int64_t rh = gid / (kValueDim / 4);
  const int v4 = int(gid % (kValueDim / 4));
  const int64_t RH = int64_t(R) * H;
  // all shards' values loaded together (P <= kMaxShards), then summed in shard order
  float l[kMaxShards];
  float4 o[kMaxShards];
#pragma unroll
  for (int p = 0; p < kMaxShards; ++p) {
    l[p] = p < P ? lse_parts[p * RH + rh] : -INFINITY;
    o[p] = p < P ? reinterpret_cast<const float4*>(o_parts + (p * RH + rh) * kValueDim)[v4]
                 : float4{0.f, 0.f, 0.f, 0.f};
  }
  float M = -INFINITY;
#pragma unroll
  for (int p = 0; p < kMaxShards; ++p) M = fmaxf(M, l[p]);
  float L = 0.f;
  float4 acc{0.f, 0.f, 0.f, 0.f};
  if (M != -INFINITY) {
#pragma unroll
    for (int p = 0; p < kMaxShards; ++p) {
      if (l[p] == -INFINITY) continue;
      const float wgt = expf(l[p] - M);
      L += wgt;
      acc.x += wgt * o[p].x;
      acc.y += wgt * o[p].y;
      acc.z += wgt * o[p].z;
      acc.w += wgt * o[p].w;
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  reinterpret_cast<float4*>(out + rh * kValueDim)[v4] = float4{acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv};
  if (lse && v4 == 0) lse[rh] = L > 0.f ? M + logf(L) : -INFINITY;
}

bool aligned(const void* p, unsigned a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

dsa_status launched() {
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? DSA_OK : static_cast<dsa_status>(record_hip_error(e));
}

}  // namespace
}  // namespace dsa

using namespace dsa;

extern "C" {

dsa_status dsa_topk_pairs(const float* scores, int64_t ld_scores, const int32_t* idx, int32_t R, int32_t k,
                          int32_t key_offset, float* pair_score, int32_t* pair_idx, void* stream) {
  if (!scores || !idx || !pair_score || !pair_idx) return DSA_ERR_NULL;
  if (R < 0 || k < 1 || k > DSA_MAX_TOPK || ld_scores < 1 || key_offset < 0) return DSA_ERR_SHAPE;
  const int64_t n = int64_t(R) * k;
  if (n == 0) return DSA_OK;
  topk_pairs_kernel<<<dim3(unsigned((n + 255) / 256)), 256, 0, static_cast<hipStream_t>(stream)>>>(
      scores, ld_scores, idx, R, k, key_offset, pair_score, pair_idx);
  return launched();
}

dsa_status dsa_topk_merge(const float* pair_score, const int32_t* pair_idx, int32_t P, int32_t R, int32_t k,
                          int32_t* idx_out, void* stream) {
  if (!pair_score || !pair_idx || !idx_out) return DSA_ERR_NULL;
  if (R < 0 || k < 1 || k > DSA_MAX_TOPK) return DSA_ERR_SHAPE;
  if (P < 1 || P > kMaxShards || P * k > kMergeMaxWords) return DSA_ERR_UNSUPPORTED;
  if (R == 0) return DSA_OK;
  // enough workgroups per row to cover the CUs, each ranking at least 512 candidates
  const int cus = device_cu_count();
  int parts = (cus + R - 1) / R;
  const int most = (P * k + kMergeThreads - 1) / kMergeThreads;
  if (parts > most) parts = most;
  if (parts < 1) parts = 1;
  topk_merge_kernel<<<dim3(unsigned(R) * unsigned(parts)), kMergeThreads, 0, static_cast<hipStream_t>(stream)>>>(
      pair_score, pair_idx, P, R, k, parts, idx_out);
  return launched();
}

dsa_status dsa_shard_indices(const int32_t* idx, int32_t R, int32_t k, int32_t lo, int32_t hi, int32_t* idx_local,
                             void* stream) {
  if (!idx || !idx_local) return DSA_ERR_NULL;
  if (R < 0 || k < 1 || lo < 0 || hi < lo) return DSA_ERR_SHAPE;
  const int64_t n = int64_t(R) * k;
  if (n == 0) return DSA_OK;
  shard_indices_kernel<<<dim3(unsigned((n + 255) / 256)), 256, 0, static_cast<hipStream_t>(stream)>>>(idx, n, lo, hi,
                                                                                                      idx_local);
  return launched();
}

dsa_status dsa_attn_merge(const float* o_parts, const float* lse_parts, int32_t P, int32_t R, int32_t H, float* out,
                          float* lse, void* stream) {
  if (!o_parts || !lse_parts || !out) return DSA_ERR_NULL;
  if (R < 0 || H < 1) return DSA_ERR_SHAPE;
  if (P < 1 || P > kMaxShards) return DSA_ERR_UNSUPPORTED;
  if (!aligned(o_parts, 16) || !aligned(out, 16)) return DSA_ERR_ALIGN;
  const int64_t threads = int64_t(R) * H * (kValueDim / 4);
  if (threads == 0) return DSA_OK;
  attn_merge_kernel<<<dim3(unsigned((threads + 255) / 256)), 256, 0, static_cast<hipStream_t>(stream)>>>(
      o_parts, lse_parts, P, R, H, out, lse);
  return launched();
}

}  // extern "C"
