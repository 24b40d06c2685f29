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
// Decomposition. A workgroup owns (query r, a range of selected positions,
// up to 64 heads); each of its waves owns 16 heads for all 512 value dims.
// Per chunk of KC selected keys (32 for bf16, 16 for fp32):
//  * gather: every latent row is read from HBM once per workgroup with
//    16-byte coalesced loads and written to LDS twice: key-major (for q.c,
//    contraction over dims) and value-major (for p.c, contraction over keys)
//    -- the value-major copy is a 4x8 register transpose, so no LDS
//    transpose pass is needed;
//  * q.c on MFMA: S^T[key][head] = C[KC x 576] . Q^T[576 x 16], the query
//    fragments stay in registers for the whole range;
//  * online softmax in registers (exp2 domain; max via two lane shuffles;
//    the row sums add the same bf16-rounded p that enters the MFMA, so
//    numerator and denominator agree);
//  * p.c on MFMA: O^T[v][head] += C^T[512 x KC] . P^T[KC x 16], P^T taken
//    straight from the q.c accumulators (the K-slot order is chosen to
//    match), O^T in 128 accumulator registers per lane.
// When a row's keys are split over several workgroups, each writes the
// unnormalised O, its max and its sum; a combine kernel merges splits in
// ascending split order. The split plan depends only on (R, H, k) and the
// device, so the same indices always give the same bits (index replay).
#include "dsa_common.hpp"
#include "dsa_internal.hpp"

namespace dsa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <bool F32>
struct AttnCfg {
  static constexpr int KC = F32 ? 16 : 32;            // keys per chunk
  static constexpr int ESZ = F32 ? 4 : 2;             // bytes per element
  static constexpr int CK_STRIDE = kLatentDim + (F32 ? 4 : 8);   // elements per key row (16-B multiple)
  static constexpr int CV_STRIDE = F32 ? (KC + 4) : (KC + 4);    // elements per value-dim row
  static constexpr int CK_BYTES = KC * CK_STRIDE * ESZ;
  static constexpr int CV_BYTES = kValueDim * CV_STRIDE * ESZ;
  static constexpr int TILES = KC / 16;               // 16-key MFMA tiles per chunk
};

template <bool F32>
using QFrag = typename std::conditional<F32, f32x8, bf16x8>::type;

template <bool F32>
__global__ __launch_bounds__(256) void sparse_mla_kernel(AttnArgs a, int splits, int kps) {
  using Cfg = AttnCfg<F32>;
  constexpr int KC = Cfg::KC;
  __shared__ __attribute__((aligned(16))) char smem[Cfg::CK_BYTES + Cfg::CV_BYTES];
  __shared__ int s_valid[KC];
  __shared__ int64_t s_row[KC];

  const int split = blockIdx.x % splits;
  const int r = blockIdx.x / splits;
  const int hb = blockIdx.y;
  const int nthreads = blockDim.x;
  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int h0 = hb * 64 + wave * 16;
  const bool has_heads = h0 < a.H;

  int b = a.q_seq ? a.q_seq[r] : r;
  b = b < 0 ? 0 : (b >= a.B ? a.B - 1 : b);
  const int64_t base = a.row_off[b];
  const int j_beg = split * kps;
  const int j_end = (j_beg + kps < a.k) ? j_beg + kps : a.k;

  // Query fragments (B operand of q.c): head h0 + col, dims 32*ks + 8*grp .. +8.
  QFrag<F32> qf[18];
  {
    const int h = h0 + col;
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
      if (h < a.H) {
        const int64_t off = (int64_t(r) * a.H + h) * kLatentDim + 32 * ks + 8 * grp;
        if constexpr (F32) {
          const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(a.q) + off);
          const float4 x = p[0], y = p[1];
          qf[ks] = f32x8{{x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w}};
        } else {
          qf[ks] = *reinterpret_cast<const bf16x8*>(static_cast<const uint16_t*>(a.q) + off);
        }
      } else {
        if constexpr (F32) qf[ks] = f32x8{{0, 0, 0, 0, 0, 0, 0, 0}};
        else qf[ks] = bf16x8{};
      }
    }
  }

  f32x4 acc_o[32];
#pragma unroll
  for (int mv = 0; mv < 32; ++mv) acc_o[mv] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;  // running max (log2 domain) of this lane's head
  float l_part = 0.f;       // this lane's share of the running sum
  const float scale2 = a.scale * kLog2e;

  char* ck = smem;
  char* cv = smem + Cfg::CK_BYTES;

  for (int j0 = j_beg; j0 < j_end; j0 += KC) {
    // ---- indices of this chunk -------------------------------------------------
    if (t < KC) {
      const int j = j0 + t;
      const int s = j < j_end ? a.idx[int64_t(r) * a.k + j] : -1;
      const int64_t row = base + s;
      const bool ok = s >= 0 && base >= 0 && row < a.cache_rows;
      s_valid[t] = ok;
      s_row[t] = ok ? row : 0;
    }
    __syncthreads();

    // ---- gather into LDS (key-major and value-major) ---------------------------
    if constexpr (!F32) {
      const uint16_t* lat = static_cast<const uint16_t*>(a.latent);
      for (int item = t; item < 768; item += nthreads) {
        if (item < 512) {
          const int kq = item >> 6, dc = item & 63;  // 4 keys x 8 dims
          uint4 v[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int key = 4 * kq + q;
            v[q] = s_valid[key] ? *reinterpret_cast<const uint4*>(lat + s_row[key] * kLatentDim + 8 * dc)
                                : uint4{0u, 0u, 0u, 0u};
            *reinterpret_cast<uint4*>(ck + (key * Cfg::CK_STRIDE + 8 * dc) * 2) = v[q];
          }
          const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&v[0]);
          const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&v[1]);
          const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&v[2]);
          const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&v[3]);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int wi = e >> 1;
            uint32_t lo, hi;
            if (e & 1) {
              lo = (w0[wi] >> 16) | (w1[wi] & 0xFFFF0000u);
              hi = (w2[wi] >> 16) | (w3[wi] & 0xFFFF0000u);
            } else {
              lo = (w0[wi] & 0xFFFFu) | (w1[wi] << 16);
              hi = (w2[wi] & 0xFFFFu) | (w3[wi] << 16);
            }
            *reinterpret_cast<uint2*>(cv + ((8 * dc + e) * Cfg::CV_STRIDE + 4 * kq) * 2) = uint2{lo, hi};
          }
        } else {
          const int it = item - 512;
          const int key = it >> 3, dc = 64 + (it & 7);  // RoPE dims: key-major only
          const uint4 v = s_valid[key] ? *reinterpret_cast<const uint4*>(lat + s_row[key] * kLatentDim + 8 * dc)
                                       : uint4{0u, 0u, 0u, 0u};
          *reinterpret_cast<uint4*>(ck + (key * Cfg::CK_STRIDE + 8 * dc) * 2) = v;
        }
      }
    } else {
      const float* lat = static_cast<const float*>(a.latent);
      for (int item = t; item < 768; item += nthreads) {
        if (item < 512) {
          const int kq = item >> 7, dc = item & 127;  // 4 keys x 4 dims
          float4 v[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int key = 4 * kq + q;
            v[q] = s_valid[key] ? *reinterpret_cast<const float4*>(lat + s_row[key] * kLatentDim + 4 * dc)
                                : float4{0.f, 0.f, 0.f, 0.f};
            *reinterpret_cast<float4*>(ck + (key * Cfg::CK_STRIDE + 4 * dc) * 4) = v[q];
          }
          *reinterpret_cast<float4*>(cv + ((4 * dc + 0) * Cfg::CV_STRIDE + 4 * kq) * 4) = float4{v[0].x, v[1].x, v[2].x, v[3].x};
          *reinterpret_cast<float4*>(cv + ((4 * dc + 1) * Cfg::CV_STRIDE + 4 * kq) * 4) = float4{v[0].y, v[1].y, v[2].y, v[3].y};
          *reinterpret_cast<float4*>(cv + ((4 * dc + 2) * Cfg::CV_STRIDE + 4 * kq) * 4) = float4{v[0].z, v[1].z, v[2].z, v[3].z};
          *reinterpret_cast<float4*>(cv + ((4 * dc + 3) * Cfg::CV_STRIDE + 4 * kq) * 4) = float4{v[0].w, v[1].w, v[2].w, v[3].w};
        } else {
          const int it = item - 512;
          const int key = it >> 4, dc = 128 + (it & 15);
          const float4 v = s_valid[key] ? *reinterpret_cast<const float4*>(lat + s_row[key] * kLatentDim + 4 * dc)
                                        : float4{0.f, 0.f, 0.f, 0.f};
          *reinterpret_cast<float4*>(ck + (key * Cfg::CK_STRIDE + 4 * dc) * 4) = v;
        }
      }
    }
    __syncthreads();

    if (has_heads) {
      // ---- logits: S^T[key][head] = C . Q^T ------------------------------------
      f32x4 sacc[Cfg::TILES];
#pragma unroll
      for (int mt = 0; mt < Cfg::TILES; ++mt) {
        sacc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        const char* rowp = ck + ((16 * mt + col) * Cfg::CK_STRIDE + 8 * grp) * Cfg::ESZ;
#pragma unroll
        for (int ks = 0; ks < 18; ++ks) {
          if constexpr (F32) {
            const float4* p = reinterpret_cast<const float4*>(rowp + 32 * ks * 4);
            const float4 x = p[0], y = p[1];
            const f32x8 af{{x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w}};
            sacc[mt] = mfma_k32(af, qf[ks], sacc[mt]);
          } else {
            const bf16x8 af = *reinterpret_cast<const bf16x8*>(rowp + 32 * ks * 2);
            sacc[mt] = mfma_k32(af, qf[ks], sacc[mt]);
          }
        }
      }

      // ---- online softmax -------------------------------------------------------
      float x[Cfg::TILES][4];
      float cmax = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < Cfg::TILES; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = 16 * mt + 4 * grp + i;
          x[mt][i] = s_valid[key] ? sacc[mt][i] * scale2 : -INFINITY;
          cmax = fmaxf(cmax, x[mt][i]);
        }
      cmax = fmaxf(cmax, wave_shfl_xor(cmax, 16));
      cmax = fmaxf(cmax, wave_shfl_xor(cmax, 32));
      const float m_new = fmaxf(m_run, cmax);
      if (m_new != -INFINITY) {  // wave-uniform: validity is per key, shared by heads
        const float alpha = exp2f(m_run - m_new);
        float p[Cfg::TILES][4];
        float psum = 0.f;
#pragma unroll
        for (int mt = 0; mt < Cfg::TILES; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float pv = exp2f(x[mt][i] - m_new);
            if constexpr (!F32) pv = static_cast<float>(static_cast<__bf16>(pv));
            p[mt][i] = pv;
            psum += pv;
          }
        l_part = l_part * alpha + psum;
        if (__ballot(alpha != 1.f)) {
#pragma unroll
          for (int mv = 0; mv < 32; ++mv) acc_o[mv] *= alpha;
        }
        m_run = m_new;

        // ---- O^T += C^T . P^T --------------------------------------------------------
        if constexpr (F32) {
#pragma unroll
          for (int mv = 0; mv < 32; ++mv) {
            const float4 cvv = *reinterpret_cast<const float4*>(cv + ((16 * mv + col) * Cfg::CV_STRIDE + 4 * grp) * 4);
            acc_o[mv] = __builtin_amdgcn_mfma_f32_16x16x4f32(cvv.x, p[0][0], acc_o[mv], 0, 0, 0);
            acc_o[mv] = __builtin_amdgcn_mfma_f32_16x16x4f32(cvv.y, p[0][1], acc_o[mv], 0, 0, 0);
            acc_o[mv] = __builtin_amdgcn_mfma_f32_16x16x4f32(cvv.z, p[0][2], acc_o[mv], 0, 0, 0);
            acc_o[mv] = __builtin_amdgcn_mfma_f32_16x16x4f32(cvv.w, p[0][3], acc_o[mv], 0, 0, 0);
          }
        } else {
          // K-slot 8*grp + i <-> key 4*grp + i (i < 4) and 16 + 4*grp + (i - 4) (i >= 4)
          const bf16x8 pf{static_cast<__bf16>(p[0][0]), static_cast<__bf16>(p[0][1]),
                          static_cast<__bf16>(p[0][2]), static_cast<__bf16>(p[0][3]),
                          static_cast<__bf16>(p[1][0]), static_cast<__bf16>(p[1][1]),
                          static_cast<__bf16>(p[1][2]), static_cast<__bf16>(p[1][3])};
#pragma unroll
          for (int mv = 0; mv < 32; ++mv) {
            const char* vrow = cv + ((16 * mv + col) * Cfg::CV_STRIDE) * 2;
            const uint2 lo = *reinterpret_cast<const uint2*>(vrow + 8 * grp);
            const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 32 + 8 * grp);
            const bf16x8 af = __builtin_bit_cast(bf16x8, uint4{lo.x, lo.y, hi.x, hi.y});
            acc_o[mv] = mfma_k32(af, pf, acc_o[mv]);
          }
        }
      }
    }
    __syncthreads();  // LDS is rewritten by the next chunk
  }

  if (!has_heads) return;
  float l_tot = l_part + wave_shfl_xor(l_part, 16);
  l_tot += wave_shfl_xor(l_tot, 32);
  const int h = h0 + col;
  if (h >= a.H) return;
  const int64_t rh = int64_t(r) * a.H + h;
  if (splits == 1) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    float* o = a.out + rh * kValueDim;
#pragma unroll
    for (int mv = 0; mv < 32; ++mv)
      *reinterpret_cast<float4*>(o + 16 * mv + 4 * grp) =
          float4{acc_o[mv][0] * inv, acc_o[mv][1] * inv, acc_o[mv][2] * inv, acc_o[mv][3] * inv};
    if (a.lse && grp == 0) a.lse[rh] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  } else {
    float* ws = static_cast<float*>(a.ws);
    const int64_t slot = (int64_t(r) * splits + split) * a.H + h;
    float* o = ws + slot * kValueDim;
#pragma unroll
    for (int mv = 0; mv < 32; ++mv)
      *reinterpret_cast<float4*>(o + 16 * mv + 4 * grp) =
          float4{acc_o[mv][0], acc_o[mv][1], acc_o[mv][2], acc_o[mv][3]};
    float* ml = ws + int64_t(a.R) * splits * a.H * kValueDim;
    if (grp == 0) {
      ml[2 * slot] = m_run;
      ml[2 * slot + 1] = l_tot;
    }
  }
}

// Merge key splits in ascending split order: O = sum_s e_s O_s / sum_s e_s l_s,
// e_s = 2^(m_s - max m). One workgroup of 128 threads per (row, head).
__global__ __launch_bounds__(128) void combine_kernel(AttnArgs a, int splits) {
  const int64_t rh = blockIdx.x;
  const int r = int(rh / a.H), h = int(rh % a.H);
  const float* ws = static_cast<const float*>(a.ws);
  const float* ml = ws + int64_t(a.R) * splits * a.H * kValueDim;
  float M = -INFINITY;
  for (int s = 0; s < splits; ++s) {
    const int64_t slot = (int64_t(r) * splits + s) * a.H + h;
    if (ml[2 * slot + 1] > 0.f) M = fmaxf(M, ml[2 * slot]);
  }
  float L = 0.f;
  float4 acc{0.f, 0.f, 0.f, 0.f};
  const int v = 4 * threadIdx.x;
  for (int s = 0; s < splits; ++s) {
    const int64_t slot = (int64_t(r) * splits + s) * a.H + h;
    const float ls = ml[2 * slot + 1];
    if (!(ls > 0.f)) continue;
    const float e = exp2f(ml[2 * slot] - M);
    L += e * ls;
    const float4 o = *reinterpret_cast<const float4*>(ws + slot * kValueDim + v);
    acc.x += e * o.x;
    acc.y += e * o.y;
    acc.z += e * o.z;
    acc.w += e * o.w;
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  *reinterpret_cast<float4*>(a.out + rh * kValueDim + v) = float4{acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv};
  if (a.lse && threadIdx.x == 0) a.lse[rh] = L > 0.f ? (M + __log2f(L)) * kLn2 : -INFINITY;
}

}  // namespace

AttnPlan plan_attention(int R, int H, int k) {
  AttnPlan p{};
  p.head_blocks = (H + 63) / 64;
  const int heads_in_block = H < 64 ? H : 64;
  p.waves = (heads_in_block + 15) / 16;
  const int base = (R > 0 ? R : 1) * p.head_blocks;
  const int target = 2 * device_cu_count();
  int splits = (target + base - 1) / base;
  const int min_keys = 64;
  const int max_splits = (k + min_keys - 1) / min_keys;
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  int kps = (k + splits - 1) / splits;
  kps = ((kps + 31) / 32) * 32;
  splits = (k + kps - 1) / kps;
  p.splits = splits;
  p.keys_per_split = kps;
  p.ws_bytes = splits > 1 ? size_t(R) * splits * H * (kValueDim + 2) * sizeof(float) : 0;
  p.ws_bytes = (p.ws_bytes + 255) / 256 * 256;
  return p;
}

hipError_t launch_sparse_mla(const AttnArgs& a, const AttnPlan& plan, hipStream_t stream) {
  if (a.R == 0) return hipSuccess;
  dim3 grid(unsigned(a.R) * unsigned(plan.splits), unsigned(plan.head_blocks));
  const int threads = 64 * plan.waves;
  if (a.dtype == kF32) sparse_mla_kernel<true><<<grid, threads, 0, stream>>>(a, plan.splits, plan.keys_per_split);
  else sparse_mla_kernel<false><<<grid, threads, 0, stream>>>(a, plan.splits, plan.keys_per_split);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || plan.splits == 1) return e;
  combine_kernel<<<dim3(unsigned(int64_t(a.R) * a.H)), 128, 0, stream>>>(a, plan.splits);
  return hipGetLastError();
}

}  // namespace dsa
