// Lightning-indexer scores on gfx950 MFMA.
//
//   scores[r, s] = sum_h w[r, h] * ReLU(q[r, h, :] . key[row_off[b] + s, :]),  s = 0..q_pos[r]
//
// The indexer ("GLM-5: from Vibe Coding to Agentic Engineering", section 2.1.2
// and section 3.2; shape 32 x 128 in "Zhipu AI / GLM", section 9.1) is, per
// query, a [H_I x D_I] x [D_I x n] product with a ReLU and a head-weighted
// sum as epilogue. In decode every key is read once and used by one query's
// H_I heads (2*H_I*D_I flops per D_I-element key: 64 flop/B in bf16), so the
// kernel is a key stream bound by HBM; it still needs the matrix cores,
// because 64 flop/B at 8 TB/s is 512 TFLOP/s, three times the fp32 vector peak.
//
// Work split: one wave owns `keys_per_wave` consecutive keys of one query
// and walks them 64 at a time (4 MFMA column tiles of 16 keys). The query's
// head tile(s) stay in registers as the A operand (heads on M); each lane
// loads the B operand straight from HBM: key n = lane % 16, 8 consecutive
// dims per K-step, 16-byte loads. The next 64 keys are loaded while the
// current ones are multiplied. Epilogue per lane: ReLU, multiply by the head
// weight, sum over the lane's 16 heads; a 3-shuffle butterfly then leaves
// lane l with the full score of key s0 + l, so the 64 scores go out as one
// coalesced 256-byte store. Every sum has a fixed order: the scores are
// bitwise reproducible.
#include "dsa_common.hpp"
#include "dsa_internal.hpp"

namespace dsa {
namespace {

constexpr int kWaves = 4;

// Storage modes of (query, key): 0 = fp32/fp32, 1 = bf16/bf16, 2 = bf16/fp8-e4m3.
template <int QK>
struct Frag {
  using type = bf16x8;
};
template <>
struct Frag<0> {
  using type = f32x8;
};

__device__ __forceinline__ void zero(bf16x8& f) {
  f = bf16x8{};
}
__device__ __forceinline__ void zero(f32x8& f) {
#pragma unroll
  for (int j = 0; j < 8; ++j) f.v[j] = 0.f;
}

// 8 consecutive elements starting at element offset `off` of a row array.
template <int QK>
__device__ __forceinline__ void load_q(typename Frag<QK>::type& f, const void* base, int64_t off) {
  if constexpr (QK == 0) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
    float4 x = p[0], y = p[1];
    f.v[0] = x.x; f.v[1] = x.y; f.v[2] = x.z; f.v[3] = x.w;
    f.v[4] = y.x; f.v[5] = y.y; f.v[6] = y.z; f.v[7] = y.w;
  } else {
    f = *reinterpret_cast<const bf16x8*>(static_cast<const uint16_t*>(base) + off);
  }
}

// OCP e4m3 -> bf16 is exact (3 mantissa bits fit in 7, every e4m3 exponent
// fits bf16's range); v_cvt_scalef32_pk_bf16_fp8 converts two codes per call.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint2 c) {
  bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.x, 1.0f, false);
  bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.x, 1.0f, true);
  bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.y, 1.0f, false);
  bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.y, 1.0f, true);
  return bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

template <int QK>
struct KeyRaw {
  uint4 v[QK == 0 ? 2 : 1];  // fp32: 32 B, bf16: 16 B, fp8: low 8 B used
};

template <int QK>
__device__ __forceinline__ void load_key(KeyRaw<QK>& k, const void* keys, int64_t elem_off) {
  if constexpr (QK == 0) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const float*>(keys) + elem_off);
    k.v[0] = p[0];
    k.v[1] = p[1];
  } else if constexpr (QK == 1) {
    k.v[0] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(keys) + elem_off);
  } else {
    uint2 c = *reinterpret_cast<const uint2*>(static_cast<const uint8_t*>(keys) + elem_off);
    k.v[0] = uint4{c.x, c.y, 0u, 0u};
  }
}

template <int QK>
__device__ __forceinline__ typename Frag<QK>::type key_frag(const KeyRaw<QK>& k) {
  typename Frag<QK>::type f;
  if constexpr (QK == 0) {
    const uint32_t* u = reinterpret_cast<const uint32_t*>(&k.v[0]);
#pragma unroll
    for (int j = 0; j < 8; ++j) f.v[j] = __uint_as_float(u[j]);
  } else if constexpr (QK == 1) {
    f = __builtin_bit_cast(bf16x8, k.v[0]);
  } else {
    f = fp8x8_to_bf16(uint2{k.v[0].x, k.v[0].y});
  }
  return f;
}

template <int QK, int MT, int DI>
__global__ __launch_bounds__(kWaves * 64) void index_scores_kernel(IndexArgs a, int keys_per_wave) {
  constexpr int NKS = DI / 32;  // K-steps of 32 dims
  using F = typename Frag<QK>::type;

  const int r = blockIdx.x;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int col = lane & 15;  // MFMA column: key within a 16-key tile
  const int grp = lane >> 4;  // K-slot group / C-row group

  int b = a.q_seq ? a.q_seq[r] : r;
  b = b < 0 ? 0 : (b >= a.B ? a.B - 1 : b);
  const int qpos = a.q_pos ? a.q_pos[r] : a.seq_len[b] - 1;
  int64_t n = qpos + 1 < a.max_n ? qpos + 1 : a.max_n;
  const int64_t base = a.row_off[b];
  if (base < 0 || base >= a.cache_rows) n = 0;
  else if (n > a.cache_rows - base) n = a.cache_rows - base;

  const int64_t s_beg = (int64_t(blockIdx.y) * kWaves + wave) * keys_per_wave;
  const int64_t s_end = s_beg + keys_per_wave < n ? s_beg + keys_per_wave : n;
  if (s_beg >= s_end) return;

  // Issue the first key group before the query loads so both are in flight.
  KeyRaw<QK> cur[4][NKS];
  auto load_group = [&](KeyRaw<QK> (&dst)[4][NKS], int64_t s0) {
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
      const int64_t s = s0 + 16 * blk + col;
      const bool ok = s < s_end;
      const int64_t off = (base + (ok ? s : 0)) * DI + 8 * grp;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        if (ok) load_key<QK>(dst[blk][ks], a.keys, off + 32 * ks);
        else {
#pragma unroll
          for (int j = 0; j < (QK == 0 ? 2 : 1); ++j) dst[blk][ks].v[j] = uint4{0u, 0u, 0u, 0u};
        }
      }
    }
  };
  load_group(cur, s_beg);

  // A operand: head 16*mt + col, dims 32*ks + 8*grp .. +8. Padded heads are zero.
  F qa[MT][NKS];
  float wr[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int h = 16 * mt + col;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      if (h < a.H_I) load_q<QK>(qa[mt][ks], a.q, (int64_t(r) * a.H_I + h) * DI + 32 * ks + 8 * grp);
      else zero(qa[mt][ks]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hw = 16 * mt + 4 * grp + i;  // C row held by this lane
      wr[mt][i] = hw < a.H_I ? a.w[int64_t(r) * a.H_I + hw] : 0.f;
    }
  }

  float* out = a.scores + int64_t(r) * a.ld;
  for (int64_t s0 = s_beg; s0 < s_end; s0 += 64) {
    KeyRaw<QK> nxt[4][NKS];
    const bool more = s0 + 64 < s_end;
    if (more) load_group(nxt, s0 + 64);

    float part[4];
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
      f32x4 acc[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const F kb = key_frag<QK>(cur[blk][ks]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt] = mfma_k32(qa[mt][ks], kb, acc[mt]);
      }
      float sc = 1.f;
      if constexpr (QK == 2) {
        const int64_t s = s0 + 16 * blk + col;
        sc = s < s_end ? bf16_bits_to_f32(a.k_scale[base + s]) : 1.f;
      }
      float p = 0.f;
      if (QK == 2 && sc < 0.f) {
        // relu(sc*z) with a negative row scale: scale each dot first.
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) p += wr[mt][i] * fmaxf(sc * acc[mt][i], 0.f);
      } else {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) p += wr[mt][i] * fmaxf(acc[mt][i], 0.f);
      }
      part[blk] = p;
    }

    // Butterfly reduce-scatter over the 4 lane groups of each column:
    // afterwards lane l holds the score of key s0 + l.
    const bool hi5 = lane & 32, hi4 = lane & 16;
    const float r0 = wave_shfl_xor(hi5 ? part[0] : part[2], 32);
    const float r1 = wave_shfl_xor(hi5 ? part[1] : part[3], 32);
    const float k0 = (hi5 ? part[2] : part[0]) + r0;
    const float k1 = (hi5 ? part[3] : part[1]) + r1;
    const float rv = wave_shfl_xor(hi4 ? k0 : k1, 16);
    float v = (hi4 ? k1 : k0) + rv;

    const int64_t s = s0 + lane;
    if (s < s_end) {
      if constexpr (QK == 2) {
        // Non-negative row scale: relu(sc*z) = sc*relu(z), applied once per key.
        const float sc = bf16_bits_to_f32(a.k_scale[base + s]);
        if (!(sc < 0.f)) v *= sc;
      }
      out[s] = v;
    }

    if (more) {
#pragma unroll
      for (int blk = 0; blk < 4; ++blk)
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) cur[blk][ks] = nxt[blk][ks];
    }
  }
}

template <int QK, int MT, int DI>
hipError_t launch_t(const IndexArgs& a, int kpw, hipStream_t stream) {
  const int64_t per_wg = int64_t(kWaves) * kpw;
  const unsigned chunks = unsigned((a.max_n + per_wg - 1) / per_wg);
  dim3 grid(unsigned(a.R), chunks);
  index_scores_kernel<QK, MT, DI><<<grid, kWaves * 64, 0, stream>>>(a, kpw);
  return hipGetLastError();
}

template <int QK, int MT>
hipError_t launch_d(const IndexArgs& a, int kpw, hipStream_t stream) {
  return a.D_I == 64 ? launch_t<QK, MT, 64>(a, kpw, stream) : launch_t<QK, MT, 128>(a, kpw, stream);
}

template <int QK>
hipError_t launch_m(const IndexArgs& a, int kpw, hipStream_t stream) {
  if (a.H_I <= 16) return launch_d<QK, 1>(a, kpw, stream);
  if (a.H_I <= 32) return launch_d<QK, 2>(a, kpw, stream);
  return launch_d<QK, 4>(a, kpw, stream);
}

}  // namespace

hipError_t launch_index_scores(const IndexArgs& a, hipStream_t stream) {
  if (a.R == 0) return hipSuccess;
  // Keys per wave: enough waves to cover the chip several times over, at
  // least one 64-key group each.
  const int64_t total = int64_t(a.R) * a.max_n;
  const int64_t target_waves = int64_t(device_cu_count()) * 16;
  int64_t kpw = (total + target_waves - 1) / target_waves;
  kpw = ((kpw + 63) / 64) * 64;
  if (kpw < 64) kpw = 64;
  if (kpw > 1024) kpw = 1024;
  const int mode = a.q_dtype == kF32 ? 0 : (a.k_dtype == kFP8 ? 2 : 1);
  if (mode == 0) return launch_m<0>(a, int(kpw), stream);
  if (mode == 1) return launch_m<1>(a, int(kpw), stream);
  return launch_m<2>(a, int(kpw), stream);
}

}  // namespace dsa
