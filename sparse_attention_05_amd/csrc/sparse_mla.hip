// Absorbed (MQA-form) sparse MLA attention over the top-k selected keys.
//
// For query r and head h over the selected positions j (idx[r, j] >= 0):
//   l_j = scale * q[r, h, :] . C[row_j, :]        (576-dim dots)
//   O[r, h, :] = sum_j softmax(l)_j * C[row_j, :512],  LSE[r, h] = log sum_j exp(l_j)
// One latent row per token serves every head as key (all 576 dims) and, in
// its first 512 dims, as value ("GLM-5: from Vibe Coding to Agentic
// Engineering", section 2.1: 576-dim latent KV cache, 576-dim dot products in
// decoding, and the plan to serve MLA in MQA form; section 3.2: attention is
// computed sparsely on the retrieved subset).
//
// Decomposition. A workgroup of 4 waves owns (query r, 16 heads, a range of
// selected positions). The range is walked in chunks of 64 keys:
//  * gather: the 64 latent rows go from HBM straight into LDS with 16-byte
//    direct-to-LDS loads (no register staging). Rows are stored key-major,
//    1152 bytes each, with the 16-byte chunks of row r XOR-permuted inside
//    aligned groups of 8 by f(r) = 2(r mod 4) + (r/4 mod 2); this keeps both
//    operand reads below free of LDS bank conflicts. Wave w loads exactly
//    rows 16w..16w+15, the rows of its own q.c tile;
//  * q.c on MFMA, split over the waves by key: wave w forms
//    S^T[16 keys][16 heads] = C[16 x 576] . Q^T, the query fragments staying
//    in registers for the whole range;
//  * online softmax (exp2 domain) with the chunk maximum exchanged through
//    LDS, so all waves apply the same running maximum; P^T goes to LDS in
//    bf16 (the row sums add the same rounded p that enters the MFMA);
//  * p.c on MFMA, split over the waves by value dimension: wave w forms
//    O^T[128w..128w+127][16 heads] += C^T . P^T over all 64 keys, its value
//    operand read from the key-major rows with the transposing LDS read
//    (ds_read_b64_tr_b16), so no second, value-major copy is needed.
// When a row's keys are split over several workgroups, each writes the
// unnormalised O, its max and its sum; the combine kernel merges the splits
// in ascending split order. The split plan depends only on (R, H, k) and the
// device, so the same indices always give the same bits (index replay).
// The workgroups sharing (query, key range) are placed on one XCD, so three
// of every four gathers of a latent row hit that XCD's L2.
#include "attn_core.hpp"

namespace dsa {
namespace {

using namespace attn;

template <bool F32>
__global__ __launch_bounds__(kAttnThreads) void sparse_mla_kernel(AttnArgs a, int splits, int kps) {
  __shared__ Smem<F32> sm;
  __shared__ int s_idx[kMaxTopk];  // raw indices of the range; wave w owns entries 64c + 16w + (0..15)
  const int HG = (a.H + kGroupHeads - 1) / kGroupHeads;
  int r, split, hg;
  map_block(blockIdx.x, a.R, splits, HG, r, split, hg);
  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int lane = t & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int h = hg * kGroupHeads + col;  // this lane's head (MFMA column)
  const int j_beg = split * kps;
  const int j_end = (j_beg + kps < a.k) ? j_beg + kps : a.k;
  const int nchunks = j_end > j_beg ? (j_end - j_beg + kChunkKeys - 1) / kChunkKeys : 0;

  const int64_t base = seq_base(a, r);
  // This wave's indices for every chunk, fetched once (one wait) before the
  // query loads, so that no later wait on them also waits for other loads.
  for (int q = lane; q < 16 * nchunks; q += 64) {
    const int e = kChunkKeys * (q >> 4) + 16 * wave + (q & 15);
    const int j = j_beg + e;
    s_idx[e] = j < j_end ? a.idx[int64_t(r) * a.k + j] : -1;
  }
  QFrag<F32> qf[18];
  load_q<F32>(a, r, h, grp, qf);
  attend<F32>(a, r, split, splits, hg, j_beg, j_end, base, s_idx, qf, sm);
}

// Merge key splits: O = sum_s e_s O_s / sum_s e_s l_s, e_s = 2^(m_s - max m),
// splits with an empty sum skipped. P adjacent lanes share one output float4,
// each lane loading and summing its SPL consecutive splits (all loads issued
// together), then the P partial sums are added in lane order. Every order is
// fixed, so the result is bitwise reproducible.
template <int P, int SPL>
__global__ __launch_bounds__(256) void combine_kernel(AttnArgs a, int splits) {
  const int64_t gid = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int64_t o4 = gid / P;            // output float4 index over [R, H, 128]
  const int part = int(gid % P);
  const int64_t total = int64_t(a.R) * a.H * (kValueDim / 4);
  const bool live = o4 < total;
  const int64_t rh = live ? o4 / (kValueDim / 4) : 0;
  const int v4 = int(o4 % (kValueDim / 4));
  const int r = int(rh / a.H), h = int(rh % a.H);
  const float* ws = static_cast<const float*>(a.ws);
  const float* ml = ws + int64_t(a.R) * splits * a.H * kValueDim;
  const int s0 = part * SPL;
  float4 o[SPL];
  float2 w[SPL];
#pragma unroll
  for (int i = 0; i < SPL; ++i) {
    const int s = s0 + i;
    if (live && s < splits) {
      const int64_t slot = (int64_t(r) * splits + s) * a.H + h;
      o[i] = reinterpret_cast<const float4*>(ws + slot * kValueDim)[v4];
      w[i] = *reinterpret_cast<const float2*>(ml + 2 * slot);
    } else {
      o[i] = float4{0.f, 0.f, 0.f, 0.f};
      w[i] = float2{-INFINITY, 0.f};
    }
  }
  float M = -INFINITY;
#pragma unroll
  for (int i = 0; i < SPL; ++i)
    if (w[i].y > 0.f) M = fmaxf(M, w[i].x);
#pragma unroll
  for (int d = 1; d < P; d <<= 1) M = fmaxf(M, __shfl_xor(M, d, 64));
  float L = 0.f;
  float4 acc{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < SPL; ++i) {
    if (w[i].y > 0.f) {
      const float e = exp2f(w[i].x - M);
      L += e * w[i].y;
      acc.x += e * o[i].x;
      acc.y += e * o[i].y;
      acc.z += e * o[i].z;
      acc.w += e * o[i].w;
    }
  }
  // add the P partial sums in lane order (lane 0 of the group holds the total)
#pragma unroll
  for (int d = 1; d < P; d <<= 1) {
    const float Lo = __shfl_down(L, d, 64);
    const float x = __shfl_down(acc.x, d, 64), y = __shfl_down(acc.y, d, 64);
    const float z = __shfl_down(acc.z, d, 64), ww = __shfl_down(acc.w, d, 64);
    if ((part & (2 * d - 1)) == 0) {
      L += Lo;
      acc.x += x;
      acc.y += y;
      acc.z += z;
      acc.w += ww;
    }
  }
  if (!live || part != 0) return;
  const float inv = L > 0.f ? 1.f / L : 0.f;
  reinterpret_cast<float4*>(a.out + rh * kValueDim)[v4] = float4{acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv};
  if (a.lse && v4 == 0) a.lse[rh] = L > 0.f ? (M + __log2f(L)) * kLn2 : -INFINITY;
}

}  // namespace

using attn::kChunkKeys;
using attn::kGroupHeads;

AttnPlan plan_attention(int R, int H, int k) {
  AttnPlan p{};
  p.head_groups = (H + kGroupHeads - 1) / kGroupHeads;
  const int base = (R > 0 ? R : 1) * p.head_groups;
  const int target = device_cu_count();  // one workgroup (147 KiB of LDS) per CU
  int splits = (target + base - 1) / base;
  int max_splits = (k + kChunkKeys - 1) / kChunkKeys;
  if (max_splits > 64) max_splits = 64;  // the combine covers up to 16 lanes x 4 splits
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  int kps = (k + splits - 1) / splits;
  kps = ((kps + kChunkKeys - 1) / kChunkKeys) * kChunkKeys;
  splits = (k + kps - 1) / kps;
  p.splits = splits;
  p.keys_per_split = kps;
  p.ws_bytes = splits > 1 ? size_t(R) * splits * H * (kValueDim + 2) * sizeof(float) : 0;
  p.ws_bytes = (p.ws_bytes + 255) / 256 * 256;
  return p;
}

hipError_t launch_sparse_mla(const AttnArgs& a, const AttnPlan& plan, hipStream_t stream) {
  if (a.R == 0) return hipSuccess;
  const dim3 grid(unsigned(a.R) * unsigned(plan.splits) * unsigned(plan.head_groups));
  if (a.dtype == kF32) sparse_mla_kernel<true><<<grid, kAttnThreads, 0, stream>>>(a, plan.splits, plan.keys_per_split);
  else sparse_mla_kernel<false><<<grid, kAttnThreads, 0, stream>>>(a, plan.splits, plan.keys_per_split);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_attn_combine(a, plan, stream);
}

hipError_t launch_attn_combine(const AttnArgs& a, const AttnPlan& plan, hipStream_t stream) {
  if (a.R == 0 || plan.splits == 1) return hipSuccess;
  // 4 splits per lane: up to 16 lanes per output float4 (splits <= 64)
  const int P = plan.splits <= 4 ? 1 : plan.splits <= 8 ? 2 : plan.splits <= 16 ? 4 : plan.splits <= 32 ? 8 : 16;
  const int64_t threads = int64_t(a.R) * a.H * (kValueDim / 4) * P;
  const dim3 cgrid(unsigned((threads + 255) / 256));
  if (P == 1) combine_kernel<1, 4><<<cgrid, 256, 0, stream>>>(a, plan.splits);
  else if (P == 2) combine_kernel<2, 4><<<cgrid, 256, 0, stream>>>(a, plan.splits);
  else if (P == 4) combine_kernel<4, 4><<<cgrid, 256, 0, stream>>>(a, plan.splits);
  else if (P == 8) combine_kernel<8, 4><<<cgrid, 256, 0, stream>>>(a, plan.splits);
  else combine_kernel<16, 4><<<cgrid, 256, 0, stream>>>(a, plan.splits);
  return hipGetLastError();
}

}  // namespace dsa
