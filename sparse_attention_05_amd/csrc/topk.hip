// Deterministic top-k of each score row (k <= 2048).
//
// The pages require the DSA selection to be reproducible bit for bit: a
// non-deterministic large-k top-k desynchronised rollout and training and
// collapsed RL ("GLM-5: from Vibe Coding to Agentic Engineering", section
// 3.2; "Zhipu AI / GLM", section 9.3; "GLM-5 Notes", Replay). Here the result
// is *unique by definition* -- the first k of the stable descending sort,
// ties to the lower key index -- and the kernel computes that unique array
// with integer work only, so no schedule can change it:
//
//  1. each score becomes a 32-bit order-preserving key (-0 folded onto +0);
//  2. radix select over the keys' range [min, max]: each pass histograms the
//     keys that can still hold the k-th largest into <= 2048 bins (integer
//     LDS atomics, 4 copies per bin so equal keys in one wave spread over
//     banks), a block-wide suffix scan finds the bin that holds it, and the
//     range narrows to that bin; <= 3 passes reach the threshold key T, the
//     count `above` of keys > T, and how many keys equal T;
//  3. winners: every key > T, plus the lowest-index `k - above` keys equal to
//     T (index-order ranks from wave ballots; skipped when all of them fit);
//  4. the <= 2048 winners, as 64-bit (key, ~index) words, are sorted
//     descending by a bitonic network in LDS and written out as indices.
//
// One workgroup of 1024 threads per row. Rows of up to 32K scores stay in
// registers between passes; longer rows are re-read from global memory
// (they were just written by the indexer and sit in L2/MALL).
#include "dsa_common.hpp"
#include "dsa_internal.hpp"

namespace dsa {
namespace {

constexpr int kThreads = 1024;
constexpr int kWavesPerBlock = kThreads / 64;
constexpr int kTile = 4 * kThreads;  // elements per coalesced sweep (float4 per thread)
constexpr int kBins = 2048;
constexpr int kCopies = 4;
constexpr int kMaxTiles = 256;       // rows of up to 2^20 scores

struct TopkShared {
  uint32_t hist[kBins * kCopies];
  unsigned long long comp[kMaxTopk];
  uint32_t tie_cnt[kMaxTiles * kWavesPerBlock];
  uint32_t red[2 * kWavesPerBlock];
  uint32_t sel_bin, sel_above, sel_cnt;
  uint32_t wcount;
};

__device__ __forceinline__ int row_len(const TopkArgs& a, int r) {
  const int q = a.q_pos ? a.q_pos[r] : a.seq_len[r] - 1;
  int n = q + 1;
  if (n > a.max_n) n = a.max_n;
  if (n < 0) n = 0;
  return n;
}

__device__ __forceinline__ unsigned long long pack(uint32_t key, int idx) {
  return (static_cast<unsigned long long>(key) << 32) | static_cast<uint32_t>(~static_cast<uint32_t>(idx));
}

// Element e of thread t in the register layout: sweep e/4, float4 slot e%4.
__device__ __forceinline__ int elem_index(int e, int t) {
  return (e >> 2) * kTile + 4 * t + (e & 3);
}

template <int EPT>
struct Row {
  // EPT > 0: the row lives in registers; EPT == 0: streamed from global.
  uint32_t key[EPT > 0 ? EPT : 1];
  const float* src;
  int n;

  __device__ void load(const float* row, int len) {
    src = row;
    n = len;
    if constexpr (EPT > 0) {
#pragma unroll
      for (int e = 0; e < EPT; e += 4) {
        const int i0 = elem_index(e, threadIdx.x);
        float4 v = i0 < n ? *reinterpret_cast<const float4*>(row + i0) : float4{0.f, 0.f, 0.f, 0.f};
        key[e] = order_key(v.x);
        key[e + 1] = order_key(v.y);
        key[e + 2] = order_key(v.z);
        key[e + 3] = order_key(v.w);
      }
    }
  }

  // f(sweep, slot, index, key) for every element of this thread with index < n.
  template <typename F>
  __device__ void visit(F&& f) const {
    if constexpr (EPT > 0) {
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        const int i = elem_index(e, threadIdx.x);
        if (i < n) f(e >> 2, e & 3, i, key[e]);
      }
    } else {
      for (int i0 = 4 * threadIdx.x, sw = 0; i0 < n; i0 += kTile, ++sw) {
        const float4 v = *reinterpret_cast<const float4*>(src + i0);
        const float x[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (i0 + j < n) f(sw, j, i0 + j, order_key(x[j]));
      }
    }
  }

  // eq[j] = (element at index sw*kTile + 4*t + j exists and has key T).
  __device__ void sweep_eq(int sw, uint32_t T, bool (&eq)[4]) const {
#pragma unroll
    for (int j = 0; j < 4; ++j) eq[j] = false;
    if constexpr (EPT > 0) {
#pragma unroll
      for (int e = 0; e < EPT; ++e)
        if ((e >> 2) == sw) eq[e & 3] = elem_index(e, threadIdx.x) < n && key[e] == T;
    } else {
      const int i0 = sw * kTile + 4 * threadIdx.x;
      if (i0 < n) {
        const float4 v = *reinterpret_cast<const float4*>(src + i0);
        const float x[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) eq[j] = i0 + j < n && order_key(x[j]) == T;
      }
    }
  }
};

__device__ __forceinline__ uint32_t wave_min(uint32_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = min(v, static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), m, 64)));
  return v;
}
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = max(v, static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), m, 64)));
  return v;
}

template <int EPT>
__global__ __launch_bounds__(kThreads) void topk_kernel(TopkArgs a) {
  __shared__ TopkShared sh;
  const int r = blockIdx.x;
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int n = row_len(a, r);
  const int k = a.k;
  const int k_eff = n < k ? n : k;
  int32_t* out = a.idx + int64_t(r) * k;

  Row<EPT> row;
  row.load(a.scores + int64_t(r) * a.ld, n);
  if (t == 0) sh.wcount = 0;

  if (n <= k) {
    __syncthreads();
    row.visit([&](int, int, int i, uint32_t key) {
      const uint32_t p = atomicAdd(&sh.wcount, 1u);
      if (p < kMaxTopk) sh.comp[p] = pack(key, i);
    });
  } else {
    // ---- range of the keys -------------------------------------------------
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
    row.visit([&](int, int, int, uint32_t key) {
      lo = min(lo, key);
      hi = max(hi, key);
    });
    lo = wave_min(lo);
    hi = wave_max(hi);
    if (lane == 0) {
      sh.red[wave] = lo;
      sh.red[kWavesPerBlock + wave] = hi;
    }
    __syncthreads();
    lo = 0xFFFFFFFFu;
    hi = 0u;
#pragma unroll
    for (int w = 0; w < kWavesPerBlock; ++w) {
      lo = min(lo, sh.red[w]);
      hi = max(hi, sh.red[kWavesPerBlock + w]);
    }

    // ---- radix select: narrow [lo, hi] to the k-th largest key ---------------
    uint32_t target = uint32_t(k), eq_total = uint32_t(n);
    // Each pass leaves a range of width < 2^(bits-11): three passes always
    // suffice; the cap makes termination independent of the data.
    for (int pass = 0; pass < 4 && lo < hi; ++pass) {
      const uint32_t width = hi - lo;
      const int nbits = 32 - __clz(width);
      const int shift = nbits > 11 ? nbits - 11 : 0;
      const int nb = int(width >> shift) + 1;
      for (int i = t; i < nb * kCopies; i += kThreads) sh.hist[i] = 0u;
      __syncthreads();
      row.visit([&](int, int, int, uint32_t key) {
        if (key >= lo && key <= hi) atomicAdd(&sh.hist[((key - lo) >> shift) * kCopies + (lane & (kCopies - 1))], 1u);
      });
      __syncthreads();
      // Thread t owns bins 2t (lower) and 2t+1 (upper). Suffix scan from the top bin.
      uint32_t c[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int bin = 2 * t + j;
        uint32_t s = 0;
        if (bin < nb) {
#pragma unroll
          for (int cpy = 0; cpy < kCopies; ++cpy) s += sh.hist[bin * kCopies + cpy];
        }
        c[j] = s;
      }
      const uint32_t tsum = c[0] + c[1];
      uint32_t incl = tsum;  // suffix sum over lanes >= lane within the wave
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = static_cast<uint32_t>(__shfl_down(static_cast<int>(incl), off, 64));
        if (lane + off < 64) incl += y;
      }
      if (lane == 0) sh.red[wave] = incl;  // wave total
      __syncthreads();
      uint32_t excl = incl - tsum;
      for (int w = wave + 1; w < kWavesPerBlock; ++w) excl += sh.red[w];
      // excl = number of keys in bins above this thread's two bins.
      if (c[1] && excl < target && excl + c[1] >= target) {
        sh.sel_bin = 2 * t + 1;
        sh.sel_above = excl;
        sh.sel_cnt = c[1];
      } else if (c[0] && excl + c[1] < target && excl + c[1] + c[0] >= target) {
        sh.sel_bin = 2 * t;
        sh.sel_above = excl + c[1];
        sh.sel_cnt = c[0];
      }
      __syncthreads();
      const uint32_t bsel = sh.sel_bin;
      target -= sh.sel_above;
      eq_total = sh.sel_cnt;
      const unsigned long long nlo = static_cast<unsigned long long>(lo) + (static_cast<unsigned long long>(bsel) << shift);
      const unsigned long long nhi = nlo + ((1ull << shift) - 1ull);
      lo = static_cast<uint32_t>(nlo);
      hi = nhi < hi ? static_cast<uint32_t>(nhi) : hi;
      __syncthreads();  // sel_* and red are rewritten by the next pass
    }
    const uint32_t T = lo;
    const uint32_t need = target;  // keys equal to T that are selected

    // ---- collect the winners -------------------------------------------------
    const bool take_all_ties = need == eq_total;
    row.visit([&](int, int, int i, uint32_t key) {
      if (key > T || (take_all_ties && key == T)) {
        const uint32_t p = atomicAdd(&sh.wcount, 1u);
        if (p < kMaxTopk) sh.comp[p] = pack(key, i);
      }
    });
    if (!take_all_ties) {
      // Rank of each T-valued key in index order: index = sweep*kTile + 4*t + slot,
      // so order is (sweep, wave, lane, slot). Count per (sweep, wave) first.
      const int sweeps = (n + kTile - 1) / kTile;
      for (int i = t; i < sweeps * kWavesPerBlock; i += kThreads) sh.tie_cnt[i] = 0u;
      __syncthreads();
      row.visit([&](int sw, int, int, uint32_t key) {
        if (key == T) atomicAdd(&sh.tie_cnt[sw * kWavesPerBlock + wave], 1u);
      });
      __syncthreads();
      if (t == 0) {  // exclusive prefix in (sweep, wave) order; at most 4096 entries
        uint32_t run = 0;
        for (int i = 0; i < sweeps * kWavesPerBlock; ++i) {
          const uint32_t c = sh.tie_cnt[i];
          sh.tie_cnt[i] = run;
          run += c;
        }
      }
      __syncthreads();
      // Within a (sweep, wave): lanes below this one, then this lane's lower slots.
      const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
      for (int sw = 0; sw * kTile < n; ++sw) {
        const int i0 = sw * kTile + 4 * t;
        bool eq[4];
        row.sweep_eq(sw, T, eq);
        // T-valued keys of lower lanes in this (sweep, wave), via per-slot ballots
        uint32_t before = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) before += __popcll(__ballot(eq[j]) & below);
        uint32_t rank = sh.tie_cnt[sw * kWavesPerBlock + wave] + before;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (eq[j]) {
            if (rank < need) {
              const uint32_t p = atomicAdd(&sh.wcount, 1u);
              if (p < kMaxTopk) sh.comp[p] = pack(T, i0 + j);
            }
            ++rank;
          }
        }
      }
    }
  }
  __syncthreads();

  // ---- sort the k_eff winners: bitonic, descending on (key, ~index) ------------
  int P = 1;
  while (P < k_eff) P <<= 1;
  for (int i = k_eff + t; i < P; i += kThreads) sh.comp[i] = 0ull;
  __syncthreads();
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = t; i < P / 2; i += kThreads) {
        const int l = 2 * i - (i & (stride - 1));
        const int h = l + stride;
        const unsigned long long x = sh.comp[l], y = sh.comp[h];
        const bool desc = (l & size) == 0;
        if (desc ? (x < y) : (x > y)) {
          sh.comp[l] = y;
          sh.comp[h] = x;
        }
      }
      __syncthreads();
    }
  }
  for (int j = t; j < k; j += kThreads)
    out[j] = j < k_eff ? static_cast<int32_t>(~static_cast<uint32_t>(sh.comp[j] & 0xFFFFFFFFull)) : -1;
}

}  // namespace

hipError_t launch_topk(const TopkArgs& a, hipStream_t stream) {
  if (a.R == 0) return hipSuccess;
  dim3 grid(unsigned(a.R));
  if (a.max_n <= 4 * kThreads) topk_kernel<4><<<grid, kThreads, 0, stream>>>(a);
  else if (a.max_n <= 16 * kThreads) topk_kernel<16><<<grid, kThreads, 0, stream>>>(a);
  else if (a.max_n <= 32 * kThreads) topk_kernel<32><<<grid, kThreads, 0, stream>>>(a);
  else topk_kernel<0><<<grid, kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace dsa
