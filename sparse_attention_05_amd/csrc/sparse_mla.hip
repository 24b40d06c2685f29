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
// Decomposition. A workgroup (4 waves) owns (query r, a range of selected
// positions, up to 64 heads); each wave owns 16 heads for all 512 value
// dims. Per chunk of KC selected keys (32 for bf16, 16 for fp32):
//  * gather: every latent row is read from HBM once per workgroup with
//    16-byte loads (a wave covers 1 KiB of one row per instruction) and
//    written to LDS twice: key-major (for q.c, contraction over dims) and
//    value-major (for p.c, contraction over keys). The value-major copy comes
//    from a 4x8 register transpose and uses an XOR-swizzled slot layout that
//    keeps both its writes and its MFMA operand reads free of LDS bank
//    conflicts. The loads of chunk c+1 are issued before chunk c is
//    computed, into the other LDS buffer;
//  * q.c on MFMA: S^T[key][head] = C[KC x 576] . Q^T[576 x 16], the query
//    fragments stay in registers for the whole range;
//  * online softmax in registers (exp2 domain; the row sums add the same
//    bf16-rounded p that enters the MFMA, so numerator and denominator agree);
//  * p.c on MFMA: O^T[v][head] += C^T[512 x KC] . P^T[KC x 16], P^T taken
//    straight from the q.c accumulators (the K-slot order is chosen to
//    match), O^T in 128 accumulator registers per lane.
// When a row's keys are split over several workgroups, each writes the
// unnormalised O, its max and its sum; the combine kernel merges the splits
// in ascending split order. The split plan depends only on (R, H, k) and the
// device, so the same indices always give the same bits (index replay).
#include "dsa_common.hpp"
#include "dsa_internal.hpp"

namespace dsa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kAttnThreads = 256;

template <bool F32>
struct AttnCfg {
  static constexpr int KC = F32 ? 16 : 32;               // keys per chunk
  static constexpr int ESZ = F32 ? 4 : 2;                // bytes per element
  static constexpr int EPC = 16 / ESZ;                   // elements per 16-byte chunk
  static constexpr int CK_STRIDE = kLatentDim + EPC;     // elements per key row (keeps 16-B alignment)
  static constexpr int CV_STRIDE = F32 ? KC + 4 : KC;    // elements per value-dim row
  static constexpr int CK_ELEMS = KC * CK_STRIDE;
  static constexpr int CV_ELEMS = kValueDim * CV_STRIDE;
  static constexpr int BUF_BYTES = (CK_ELEMS + CV_ELEMS) * ESZ;
  static constexpr int NBUF = F32 ? 1 : 2;
  static constexpr int TILES = KC / 16;                  // 16-key MFMA tiles per chunk
  static constexpr int BLOCK_KEYS_SHIFT = F32 ? 7 : 6;   // block item -> (key quad, dim chunk)
  static constexpr int ROPE_SHIFT = F32 ? 4 : 3;         // rope item -> (key, chunk)
  static constexpr int ROPE_CHUNK0 = kValueDim / EPC;    // first 16-byte chunk of the RoPE part
};

// Element offset of (value dim v, key column c, c % 4 == 0) in the
// value-major copy. bf16 rows are 64 bytes = eight 8-byte slots of 4 keys,
// slot c/4 stored at (c/4) ^ phi(v) with phi(v) = ((v >> 1) ^ (v >> 4)) & 7:
// the MFMA operand reads (16 consecutive rows, one slot each) and the
// transposed writes (rows 8 apart, alternating parity) both land on 16
// distinct 8-byte slots of every 128-byte bank window.
template <bool F32>
__device__ __forceinline__ int cv_off(int v, int c) {
  using Cfg = AttnCfg<F32>;
  if constexpr (F32) return v * Cfg::CV_STRIDE + c;
  else return v * Cfg::CV_STRIDE + 4 * ((c >> 2) ^ (((v >> 1) ^ (v >> 4)) & 7));
}

template <bool F32>
using QFrag = typename std::conditional<F32, f32x8, bf16x8>::type;

// Gathered data of one chunk held by one thread between the load and the
// LDS write: two 4-key x 16-byte transpose blocks and one RoPE chunk.
struct Stage {
  uint4 blk[2][4];
  uint4 rope;
  int ok_rope;
};

template <bool F32>
__device__ __forceinline__ void gather(Stage& st, const AttnArgs& a, int r, int64_t base, int j0, int j_end) {
  using Cfg = AttnCfg<F32>;
  const int t = threadIdx.x;
  const char* lat = static_cast<const char*>(a.latent);
  auto row_of = [&](int key, bool& ok) -> int64_t {
    const int j = j0 + key;
    const int s = j < j_end ? a.idx[int64_t(r) * a.k + j] : -1;
    const int64_t row = base + s;
    ok = s >= 0 && base >= 0 && row < a.cache_rows;
    return ok ? row : 0;
  };
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int item = t + h * kAttnThreads;  // 0..511
    const int kq = item >> Cfg::BLOCK_KEYS_SHIFT;
    const int dc = item & ((1 << Cfg::BLOCK_KEYS_SHIFT) - 1);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      bool ok;
      const int64_t row = row_of(4 * kq + q, ok);
      st.blk[h][q] = ok ? *reinterpret_cast<const uint4*>(lat + row * (kLatentDim * Cfg::ESZ) + 16 * dc)
                        : uint4{0u, 0u, 0u, 0u};
    }
  }
  {
    const int it = t;  // rope item 0..255
    const int key = it >> Cfg::ROPE_SHIFT;
    const int ch = Cfg::ROPE_CHUNK0 + (it & ((1 << Cfg::ROPE_SHIFT) - 1));
    bool ok;
    const int64_t row = row_of(key, ok);
    st.rope = ok ? *reinterpret_cast<const uint4*>(lat + row * (kLatentDim * Cfg::ESZ) + 16 * ch)
                 : uint4{0u, 0u, 0u, 0u};
    st.ok_rope = ok;
  }
}

template <bool F32>
__device__ __forceinline__ void stage_to_lds(const Stage& st, char* buf, int* valid) {
  using Cfg = AttnCfg<F32>;
  const int t = threadIdx.x;
  char* ck = buf;
  char* cv = buf + Cfg::CK_ELEMS * Cfg::ESZ;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int item = t + h * kAttnThreads;
    const int kq = item >> Cfg::BLOCK_KEYS_SHIFT;
    const int dc = item & ((1 << Cfg::BLOCK_KEYS_SHIFT) - 1);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<uint4*>(ck + ((4 * kq + q) * Cfg::CK_STRIDE + Cfg::EPC * dc) * Cfg::ESZ) = st.blk[h][q];
    if constexpr (F32) {
      // 4 keys x 4 dims -> 4 value rows of 4 keys
      const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&st.blk[h][0]);
      const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&st.blk[h][1]);
      const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&st.blk[h][2]);
      const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&st.blk[h][3]);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        *reinterpret_cast<uint4*>(cv + cv_off<F32>(4 * dc + e, 4 * kq) * 4) = uint4{w0[e], w1[e], w2[e], w3[e]};
    } else {
      // 4 keys x 8 dims -> 8 value rows of 4 keys (two bf16 per word)
      const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&st.blk[h][0]);
      const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&st.blk[h][1]);
      const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&st.blk[h][2]);
      const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&st.blk[h][3]);
      // Step s writes row 8*dc + (s ^ odd): lanes of odd dc take the other row
      // of each pair, so neighbouring lanes write rows of different parity.
      const int odd = dc & 1;
#pragma unroll
      for (int sp = 0; sp < 8; sp += 2) {
        const int wi = sp >> 1;
        const uint32_t lo_e = (w0[wi] & 0xFFFFu) | (w1[wi] << 16);
        const uint32_t hi_e = (w2[wi] & 0xFFFFu) | (w3[wi] << 16);
        const uint32_t lo_o = (w0[wi] >> 16) | (w1[wi] & 0xFFFF0000u);
        const uint32_t hi_o = (w2[wi] >> 16) | (w3[wi] & 0xFFFF0000u);
        const int e0 = sp + odd, e1 = sp + (odd ^ 1);
        *reinterpret_cast<uint2*>(cv + cv_off<F32>(8 * dc + e0, 4 * kq) * 2) =
            odd ? uint2{lo_o, hi_o} : uint2{lo_e, hi_e};
        *reinterpret_cast<uint2*>(cv + cv_off<F32>(8 * dc + e1, 4 * kq) * 2) =
            odd ? uint2{lo_e, hi_e} : uint2{lo_o, hi_o};
      }
    }
  }
  {
    const int it = t;
    const int key = it >> Cfg::ROPE_SHIFT;
    const int sub = it & ((1 << Cfg::ROPE_SHIFT) - 1);
    *reinterpret_cast<uint4*>(ck + (key * Cfg::CK_STRIDE + Cfg::EPC * (Cfg::ROPE_CHUNK0 + sub)) * Cfg::ESZ) = st.rope;
    if (sub == 0) valid[key] = st.ok_rope;
  }
}

template <bool F32>
__global__ __launch_bounds__(kAttnThreads) void sparse_mla_kernel(AttnArgs a, int splits, int kps) {
  using Cfg = AttnCfg<F32>;
  constexpr int KC = Cfg::KC;
  // chunk buffers, reused by the epilogue for O as [64 heads][512] floats
  constexpr int kOutBytes = 64 * (kValueDim + 4) * 4;
  constexpr int kSmem = Cfg::NBUF * Cfg::BUF_BYTES > kOutBytes ? Cfg::NBUF * Cfg::BUF_BYTES : kOutBytes;
  __shared__ __attribute__((aligned(16))) char smem[kSmem];
  __shared__ int s_valid[Cfg::NBUF][KC];

  const int split = blockIdx.x % splits;
  const int r = blockIdx.x / splits;
  const int hb = blockIdx.y;
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
  const int nchunks = j_end > j_beg ? (j_end - j_beg + KC - 1) / KC : 0;

  Stage st;
  if (nchunks > 0) gather<F32>(st, a, r, base, j_beg, j_end);

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

  for (int c = 0; c < nchunks; ++c) {
    const int bi = Cfg::NBUF == 2 ? (c & 1) : 0;
    char* buf = smem + bi * Cfg::BUF_BYTES;
    if (Cfg::NBUF == 1 && c > 0) __syncthreads();  // single buffer: previous chunk consumed
    stage_to_lds<F32>(st, buf, s_valid[bi]);
    if (Cfg::NBUF == 2 && c + 1 < nchunks) gather<F32>(st, a, r, base, j_beg + (c + 1) * KC, j_end);
    __syncthreads();  // this chunk is in LDS; the other buffer is free for the next write
    if (Cfg::NBUF == 1 && c + 1 < nchunks) gather<F32>(st, a, r, base, j_beg + (c + 1) * KC, j_end);

    if (has_heads) {
      const char* ck = buf;
      const char* cv = buf + Cfg::CK_ELEMS * Cfg::ESZ;
      // ---- logits: S^T[key][head] = C . Q^T ------------------------------------
      // Four independent accumulator chains per tile (K-steps ks mod 4), summed
      // in a fixed order, so the matrix cores are not serialised on one chain.
      f32x4 sacc[Cfg::TILES];
#pragma unroll
      for (int mt = 0; mt < Cfg::TILES; ++mt) {
        f32x4 part[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) part[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        const char* rowp = ck + ((16 * mt + col) * Cfg::CK_STRIDE + 8 * grp) * Cfg::ESZ;
#pragma unroll
        for (int ks = 0; ks < 18; ++ks) {
          if constexpr (F32) {
            const float4* p = reinterpret_cast<const float4*>(rowp + 32 * ks * 4);
            const float4 x = p[0], y = p[1];
            const f32x8 af{{x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w}};
            part[ks & 3] = mfma_k32(af, qf[ks], part[ks & 3]);
          } else {
            const bf16x8 af = *reinterpret_cast<const bf16x8*>(rowp + 32 * ks * 2);
            part[ks & 3] = mfma_k32(af, qf[ks], part[ks & 3]);
          }
        }
        sacc[mt] = (part[0] + part[1]) + (part[2] + part[3]);
      }

      // ---- online softmax -------------------------------------------------------
      float x[Cfg::TILES][4];
      float cmax = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < Cfg::TILES; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = 16 * mt + 4 * grp + i;
          x[mt][i] = s_valid[bi][key] ? sacc[mt][i] * scale2 : -INFINITY;
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
            const float4 cvv = *reinterpret_cast<const float4*>(cv + cv_off<F32>(16 * mv + col, 4 * grp) * 4);
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
            const int v = 16 * mv + col;
            const uint2 lo = *reinterpret_cast<const uint2*>(cv + cv_off<F32>(v, 4 * grp) * 2);
            const uint2 hi = *reinterpret_cast<const uint2*>(cv + cv_off<F32>(v, 16 + 4 * grp) * 2);
            const bf16x8 af = __builtin_bit_cast(bf16x8, uint4{lo.x, lo.y, hi.x, hi.y});
            acc_o[mv] = mfma_k32(af, pf, acc_o[mv]);
          }
        }
      }
    }
  }

  // ---- epilogue: finish the row sums, stage O in LDS as [head][512], then
  // write whole 2-KiB head rows with contiguous 16-byte stores ----------------
  float l_tot = l_part + wave_shfl_xor(l_part, 16);
  l_tot += wave_shfl_xor(l_tot, 32);
  const bool final_out = splits == 1;
  __syncthreads();  // every wave is done with the chunk buffers
  // 4 waves x 16 heads x (512 + 4) floats: the 16-byte pad per head row
  // spreads the 16 heads of a store over the LDS banks
  constexpr int kORow = kValueDim + 4;
  float* o_lds = reinterpret_cast<float*>(smem);
  if (has_heads) {
    const float inv = final_out ? (l_tot > 0.f ? 1.f / l_tot : 0.f) : 1.f;
    float* orow = o_lds + (wave * 16 + col) * kORow;
#pragma unroll
    for (int mv = 0; mv < 32; ++mv)
      *reinterpret_cast<float4*>(orow + 16 * mv + 4 * grp) =
          float4{acc_o[mv][0] * inv, acc_o[mv][1] * inv, acc_o[mv][2] * inv, acc_o[mv][3] * inv};
    const int h = h0 + col;
    if (h < a.H && grp == 0) {
      const int64_t rh = int64_t(r) * a.H + h;
      if (final_out) {
        if (a.lse) a.lse[rh] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
      } else {
        float* ml = static_cast<float*>(a.ws) + int64_t(a.R) * splits * a.H * kValueDim;
        const int64_t slot = (int64_t(r) * splits + split) * a.H + h;
        *reinterpret_cast<float2*>(ml + 2 * slot) = float2{m_run, l_tot};
      }
    }
  }
  __syncthreads();
  const int hcount = (a.H - hb * 64) < 64 ? (a.H - hb * 64) : 64;  // heads of this block
  float* dst = final_out ? a.out + (int64_t(r) * a.H + hb * 64) * kValueDim
                         : static_cast<float*>(a.ws) + ((int64_t(r) * splits + split) * a.H + hb * 64) * kValueDim;
  for (int i = t; i < hcount * (kValueDim / 4); i += kAttnThreads) {
    const int hh = i / (kValueDim / 4), v4 = i % (kValueDim / 4);
    reinterpret_cast<float4*>(dst)[i] = *reinterpret_cast<const float4*>(o_lds + hh * kORow + 4 * v4);
  }
}

// Merge key splits: O = sum_s e_s O_s / sum_s e_s l_s, e_s = 2^(m_s - max m),
// splits with an empty sum skipped. P = ceil(splits / 16) adjacent lanes share
// one output float4, each lane loading and summing its <= 16 splits (all loads
// issued together), then the P partial sums are added in lane order. Every
// order is fixed, so the result is bitwise reproducible.
template <int P>
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
  const int s0 = part * 16;
  float4 o[16];
  float2 w[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
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
  for (int i = 0; i < 16; ++i)
    if (w[i].y > 0.f) M = fmaxf(M, w[i].x);
#pragma unroll
  for (int d = 1; d < P; d <<= 1) M = fmaxf(M, __shfl_xor(M, d, 64));
  float L = 0.f;
  float4 acc{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 16; ++i) {
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

AttnPlan plan_attention(int R, int H, int k) {
  AttnPlan p{};
  p.head_blocks = (H + 63) / 64;
  p.waves = 4;
  const int base = (R > 0 ? R : 1) * p.head_blocks;
  const int target = device_cu_count();  // one 4-wave workgroup fills a CU
  int splits = (target + base - 1) / base;
  const int min_keys = 64;  // at least two chunks, so loads overlap compute
  int max_splits = (k + min_keys - 1) / min_keys;
  if (max_splits > 64) max_splits = 64;  // the combine holds one split per lane
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
  if (a.dtype == kF32) sparse_mla_kernel<true><<<grid, kAttnThreads, 0, stream>>>(a, plan.splits, plan.keys_per_split);
  else sparse_mla_kernel<false><<<grid, kAttnThreads, 0, stream>>>(a, plan.splits, plan.keys_per_split);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || plan.splits == 1) return e;
  const int P = plan.splits <= 16 ? 1 : (plan.splits <= 32 ? 2 : 4);
  const int64_t threads = int64_t(a.R) * a.H * (kValueDim / 4) * P;
  const dim3 cgrid(unsigned((threads + 255) / 256));
  if (P == 1) combine_kernel<1><<<cgrid, 256, 0, stream>>>(a, plan.splits);
  else if (P == 2) combine_kernel<2><<<cgrid, 256, 0, stream>>>(a, plan.splits);
  else combine_kernel<4><<<cgrid, 256, 0, stream>>>(a, plan.splits);
  return hipGetLastError();
}

}  // namespace dsa
