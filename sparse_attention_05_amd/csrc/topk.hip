// Deterministic top-k of each score row (k <= 2048).
//
// The pages require the DSA selection to be reproducible bit for bit: a
// non-deterministic large-k top-k desynchronised rollout and training and
// collapsed RL ("GLM-5: from Vibe Coding to Agentic Engineering", section
// 3.2; "Zhipu AI / GLM", section 9.3; "GLM-5 Notes", Replay). The result here
// is unique by definition -- the first k of the stable descending sort, ties
// to the lower key index -- and every step below computes a quantity that is
// itself unique (a count, a threshold, a rank among distinct words) with
// integer arithmetic only. No step depends on the order in which threads or
// atomics happen to run.
//
// One 512-thread workgroup per row. Scores become 32-bit order-preserving
// keys (-0 folded onto +0). A row of up to 32K keys stays in registers,
// loaded as coalesced float4 sweeps (index = sweep*2048 + 4*thread + slot);
// longer rows are re-read from L2 on every pass.
//  1. pivot: a fixed sample (every SS-th index) is histogrammed over its
//     range; the pivot is the lower edge of the bin holding the
//     (ceil(k/SS)+24)-th largest sample, so ~1.2k keys clear it;
//  2. candidates: keys >= pivot are compacted into LDS (positions from a
//     block prefix sum) as unique 64-bit words (key << 32 | ~index), whose
//     descending order is exactly the stable order (score desc, index asc);
//  3. the candidates are sorted and the first k written out: bucket passes
//     on 12-bit adaptive digits of (max - word), buckets of at most 32 words
//     ranked by counting, denser buckets (those that reach below rank k)
//     split again from their exact word range (a work list, up to three
//     more levels), and a bitonic network for whatever is left;
//  fallback, when fewer than k or more than 4096 keys clear the pivot (heavy
//     ties, skewed rows): radix select over the whole row finds the k-th key
//     T, the kept keys equal to T are the `need` smallest indices (the same
//     select on complemented indices), and the k winners are sorted as above.
// Histogram bins are found with a two-level (64 x 64) search that needs
// wave-level DPP scans only.
#include <type_traits>
#include <utility>

#include "attn_core.hpp"
#include "dsa_common.hpp"
#include "dsa_internal.hpp"

namespace dsa {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kTile = 4 * kThreads;  // one coalesced sweep
constexpr int kBins = 4096;          // 12-bit digits (64 groups of 64)
constexpr int kCap = 4096;           // candidate capacity
constexpr int kMaxSamples = 8192;    // score samples behind a pivot
constexpr int kMaxSliceTiles = 8;    // tiles of kTile keys per slice of a split row
constexpr int kBatch = 8;            // streamed tiles in flight per pass over a long row
constexpr int kSmall = 32;           // rank-by-counting limit
constexpr int kFastSmall = 512;      // ... in the window selection's short form (one word per thread)
constexpr int kMaxWork = 16;         // dense buckets split per level
constexpr int kFullBins = 1024;      // whole-row histogram: 10-bit digits
constexpr int kFullCopies = 8;       // ... spread over lane & 7

struct __attribute__((aligned(16))) TopkShared {
  uint32_t bins[kBins];              // histogram counts / bucket starts
  uint32_t fill[kBins];              // bucket fill counters
  uint32_t cnt[kBins];               // bucket counts
  uint32_t coarse[64];
  uint32_t xred[(2 + kMaxSliceTiles) * kWaves];  // candidate-launch exchange
  unsigned long long wa[kCap];       // candidate / winner words, sort ping-pong
  union {
    unsigned long long wb[kCap];
    uint32_t full[kFullBins * kFullCopies];  // whole-row histogram (fallback select)
  } u;
  union {
    uint32_t samp[kMaxSamples];      // score sample keys (split pivot)
    unsigned long long net[kCap];    // bitonic scratch
  } v;
  uint32_t red[6 * kWaves];
  uint32_t misc[16];
  uint32_t work[2][6 * kMaxWork];    // dense buckets: offset, length, max (2 words), min (2 words)
};

template <int... Is, typename F>
__device__ __forceinline__ void unroll_impl(std::integer_sequence<int, Is...>, F&& f) {
  (f(std::integral_constant<int, Is>{}), ...);
}
// f(integral_constant<int, I>) for I = 0 .. N-1 (compile-time register indices)
template <int N, typename F>
__device__ __forceinline__ void unroll(F&& f) {
  unroll_impl(std::make_integer_sequence<int, N>{}, f);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

// Barrier that orders LDS accesses only. __syncthreads also waits for every
// outstanding global load and store of the wave (its workgroup fence waits
// on the whole vector-memory count), which would hold a barrier up behind
// loads issued early for later use. No thread here reads global memory that
// another thread of its workgroup wrote, and loads into registers are waited
// for where they are used, so ordering the LDS is all the selection needs.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// true in every thread when `p` holds in any thread (uniform control flow)
__device__ __forceinline__ bool block_any(bool p, uint32_t* red) {
  const bool w = __ballot(p) != 0ull;
  if (lane_id() == 0) red[wave_id()] = w ? 1u : 0u;
  lds_barrier();
  uint32_t r = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) r |= red[i];
  lds_barrier();
  return r != 0u;
}

// ---- block primitives (uniform control flow; each ends with a barrier) -----------

__device__ __forceinline__ uint32_t block_scan(uint32_t v, uint32_t* red, uint32_t& total) {
  const uint32_t x = wave_incl_scan(v);
  if (lane_id() == 63) red[wave_id()] = x;
  lds_barrier();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const uint32_t c = red[w];
    base += w < wave_id() ? c : 0u;
    tot += c;
  }
  lds_barrier();
  total = tot;
  return base + x - v;
}

// block_scan of v and, in the same exchange, the maximum of u over the block
__device__ __forceinline__ uint32_t block_scan_max(uint32_t v, uint32_t u, uint32_t* red, uint32_t& total,
                                                   uint32_t& umax) {
  const uint32_t x = wave_incl_scan(v);
  const uint32_t m = wave_max(u);
  if (lane_id() == 63) red[wave_id()] = x;
  if (lane_id() == 0) red[kWaves + wave_id()] = m;
  lds_barrier();
  uint32_t base = 0, tot = 0, mm = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const uint32_t c = red[w];
    base += w < wave_id() ? c : 0u;
    tot += c;
    mm = max(mm, red[kWaves + w]);
  }
  lds_barrier();
  total = tot;
  umax = mm;
  return base + x - v;
}

__device__ __forceinline__ uint32_t block_max(uint32_t v, uint32_t* red) {
  const uint32_t m = wave_max(v);
  if (lane_id() == 0) red[wave_id()] = m;
  lds_barrier();
  uint32_t r = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) r = max(r, red[w]);
  lds_barrier();
  return r;
}

__device__ __forceinline__ uint32_t block_min(uint32_t v, uint32_t* red) {
  const uint32_t m = wave_min(v);
  if (lane_id() == 0) red[wave_id()] = m;
  lds_barrier();
  uint32_t r = 0xFFFFFFFFu;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) r = min(r, red[w]);
  lds_barrier();
  return r;
}

// (min, max) of a value over the block with a single exchange.
__device__ __forceinline__ void block_minmax(uint32_t& mn, uint32_t& mx, uint32_t* red) {
  const uint32_t a = wave_min(mn), b = wave_max(mx);
  if (lane_id() == 0) {
    red[wave_id()] = a;
    red[kWaves + wave_id()] = b;
  }
  lds_barrier();
  mn = 0xFFFFFFFFu;
  mx = 0u;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    mn = min(mn, red[w]);
    mx = max(mx, red[kWaves + w]);
  }
  lds_barrier();
}

__device__ __forceinline__ void clear_bins(uint32_t* a, int n) {
  for (int i = 4 * threadIdx.x; i < n; i += 4 * kThreads) *reinterpret_cast<uint4*>(a + i) = uint4{0u, 0u, 0u, 0u};
}

// Bin b of sh.bins[0..kBins) (zero past the used range) such that the
// counts of the bins above b sum to `above` < target <= above + count(b).
__device__ __forceinline__ void find_crossing(TopkShared& sh, uint32_t target, uint32_t& b, uint32_t& above,
                                              uint32_t& cnt) {
  const int lane = lane_id(), wave = wave_id();
  {
    const int g = 8 * wave + (lane >> 3);  // group of 64 bins
    const int b0 = 64 * g + 8 * (lane & 7);
    const uint4 x = *reinterpret_cast<const uint4*>(sh.bins + b0);
    const uint4 y = *reinterpret_cast<const uint4*>(sh.bins + b0 + 4);
    const uint32_t s = octet_sum(x.x + x.y + x.z + x.w + y.x + y.y + y.z + y.w);
    if ((lane & 7) == 0) sh.coarse[g] = s;
  }
  lds_barrier();
  if (wave == 0) {
    const uint32_t c = sh.coarse[lane];
    const uint32_t incl = wave_incl_scan(c);
    const uint32_t above_g = lane_value(incl, 63) - incl;  // in groups above this one
    const unsigned long long hit = __ballot(c != 0u && above_g < target && above_g + c >= target);
    int g = __ffsll(static_cast<long long>(hit)) - 1;
    g = g < 0 ? 0 : g;
    const uint32_t base = lane_value(above_g, g);
    const uint32_t f = sh.bins[64 * g + lane];
    const uint32_t incl2 = wave_incl_scan(f);
    const uint32_t above_f = base + lane_value(incl2, 63) - incl2;
    const unsigned long long hit2 = __ballot(f != 0u && above_f < target && above_f + f >= target);
    int fl = __ffsll(static_cast<long long>(hit2)) - 1;
    fl = fl < 0 ? 0 : fl;
    if (lane == fl) {
      sh.misc[0] = 64 * g + lane;
      sh.misc[1] = above_f;
      sh.misc[2] = f;
    }
  }
  lds_barrier();
  b = sh.misc[0];
  above = sh.misc[1];
  cnt = sh.misc[2];
}

// Digits of width 2^shift over [lo, hi]: at most 2^bits bins.
template <typename U>
__device__ __forceinline__ void digit_plan(U lo, U hi, int bits, int& shift, int& nb) {
  const U width = hi - lo;
  int nbits = 0;
  if constexpr (sizeof(U) == 8) nbits = width ? 64 - __clzll(static_cast<long long>(width)) : 0;
  else nbits = width ? 32 - __clz(static_cast<int>(width)) : 0;
  shift = nbits > bits ? nbits - bits : 0;
  nb = int(width >> shift) + 1;
}

__device__ __forceinline__ void narrow(uint32_t& lo, uint32_t& hi, uint32_t b, int shift) {
  const unsigned long long nlo = static_cast<unsigned long long>(lo) + (static_cast<unsigned long long>(b) << shift);
  const unsigned long long nhi = nlo + ((1ull << shift) - 1ull);
  lo = static_cast<uint32_t>(nlo);
  hi = nhi < hi ? static_cast<uint32_t>(nhi) : hi;
}

// k-th largest of the visited values, all in [lo, hi] (count of them =
// count); visit(f) calls f(value) for this thread's values. Returns the
// threshold T, how many values equal to T are within the top `target`
// (need) and how many values equal T (eq_total). Values are expected to be
// spread (few collisions per histogram bin).
template <typename Visit>
__device__ __forceinline__ void select_small(TopkShared& sh, Visit&& visit, uint32_t lo, uint32_t hi,
                                             uint32_t target, uint32_t count, uint32_t& T, uint32_t& need,
                                             uint32_t& eq_total) {
  eq_total = count;
  for (int pass = 0; pass < 4 && lo < hi; ++pass) {  // 12-bit digits: <= 3 passes
    int shift, nb;
    digit_plan(lo, hi, 12, shift, nb);
    clear_bins(sh.bins, kBins);
    lds_barrier();
    visit([&](uint32_t v) {
      if (v >= lo && v <= hi) atomicAdd(&sh.bins[(v - lo) >> shift], 1u);
    });
    lds_barrier();
    uint32_t b, above, cnt;
    find_crossing(sh, target, b, above, cnt);
    target -= above;
    eq_total = cnt;
    narrow(lo, hi, b, shift);
    lds_barrier();  // bins and misc are rewritten by the next pass
  }
  T = lo;
  need = target;
}

// The same select over a whole row, whose values may collide heavily (tie
// classes): a 10-bit histogram with 8 copies per bin, reduced into sh.bins.
template <typename Visit>
__device__ __forceinline__ void select_full(TopkShared& sh, Visit&& visit, uint32_t lo, uint32_t hi,
                                            uint32_t target, uint32_t count, uint32_t& T, uint32_t& need,
                                            uint32_t& eq_total) {
  const int lane = lane_id();
  eq_total = count;
  for (int pass = 0; pass < 5 && lo < hi; ++pass) {  // 10-bit digits: <= 4 passes
    int shift, nb;
    digit_plan(lo, hi, 10, shift, nb);
    clear_bins(sh.u.full, kFullBins * kFullCopies);
    clear_bins(sh.bins, kBins);
    lds_barrier();
    visit([&](uint32_t v) {
      if (v >= lo && v <= hi) atomicAdd(&sh.u.full[((v - lo) >> shift) * kFullCopies + (lane & 7)], 1u);
    });
    lds_barrier();
    for (int i = threadIdx.x; i < kFullBins; i += kThreads) {
      const uint4 x = *reinterpret_cast<const uint4*>(sh.u.full + i * kFullCopies);
      const uint4 y = *reinterpret_cast<const uint4*>(sh.u.full + i * kFullCopies + 4);
      sh.bins[i] = x.x + x.y + x.z + x.w + y.x + y.y + y.z + y.w;
    }
    lds_barrier();
    uint32_t b, above, cnt;
    find_crossing(sh, target, b, above, cnt);
    target -= above;
    eq_total = cnt;
    narrow(lo, hi, b, shift);
    lds_barrier();
  }
  T = lo;
  need = target;
}

// A score row as keys. EPT > 0: this thread's EPT keys in registers
// (index = (e/4)*kTile + 4*t + e%4; keys past the row end are 0, below every
// real key). EPT == 0: each pass re-reads the row from global memory.
template <int EPT>
struct Row {
  uint32_t key[EPT > 0 ? EPT : 1];
  const float* src;
  int n;

  __device__ __forceinline__ void load(const float* row, int len) {
    src = row;
    n = len;
    if constexpr (EPT > 0) {
      unroll<EPT / 4>([&](auto ss) {
        constexpr int s = decltype(ss)::value;
        const int i0 = s * kTile + 4 * int(threadIdx.x);
        const float4 v = i0 < n ? *reinterpret_cast<const float4*>(row + i0) : float4{0.f, 0.f, 0.f, 0.f};
        key[4 * s + 0] = i0 + 0 < n ? order_key(v.x) : 0u;
        key[4 * s + 1] = i0 + 1 < n ? order_key(v.y) : 0u;
        key[4 * s + 2] = i0 + 2 < n ? order_key(v.z) : 0u;
        key[4 * s + 3] = i0 + 3 < n ? order_key(v.w) : 0u;
      });
    }
  }

  // f(index / SS, key) for this thread's elements whose index is a multiple
  // of SS (a power of two >= 16) and below n.
  template <typename F>
  __device__ __forceinline__ void sample(int SS, F&& f) const {
    if constexpr (EPT > 0) {
      // index = s*kTile + 4t + q is a multiple of 16 iff q == 0 and t % 4 == 0
      if ((threadIdx.x & 3) == 0 && SS == 16) {
        unroll<EPT / 4>([&](auto ss) {
          constexpr int s = decltype(ss)::value;
          const int idx = s * kTile + 4 * int(threadIdx.x);
          if (idx < n) f(idx >> 4, key[4 * s]);
        });
      }
    } else {
      // every SS-th index: the thread's indexes 4t + j*kTile that are
      // multiples of SS, kBatch loads in flight at a time
      const int lg = __ffs(SS) - 1;
      for (int b0 = 4 * int(threadIdx.x); b0 < n; b0 += kTile * kBatch) {
        float x[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int i0 = b0 + u * kTile;
          x[u] = i0 < n && (i0 & (SS - 1)) == 0 ? src[i0] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int i0 = b0 + u * kTile;
          if (i0 < n && (i0 & (SS - 1)) == 0) f(i0 >> lg, order_key(x[u]));
        }
      }
    }
  }

  // f(index, key) for every element of this thread, padding (key 0) included.
  template <typename F>
  __device__ __forceinline__ void each(F&& f) const {
    if constexpr (EPT > 0) {
      unroll<EPT>([&](auto ee) {
        constexpr int e = decltype(ee)::value;
        f((e >> 2) * kTile + 4 * int(threadIdx.x) + (e & 3), key[e]);
      });
    } else {
      // streamed from memory, kBatch tiles' loads in flight before any is used
      for (int b0 = 4 * int(threadIdx.x); b0 < n; b0 += kTile * kBatch) {
        float4 v[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int i0 = b0 + u * kTile;
          v[u] = i0 < n ? *reinterpret_cast<const float4*>(src + i0) : float4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int i0 = b0 + u * kTile;
          if (i0 < n) {
            f(i0 + 0, order_key(v[u].x));
            f(i0 + 1, i0 + 1 < n ? order_key(v[u].y) : 0u);
            f(i0 + 2, i0 + 2 < n ? order_key(v[u].z) : 0u);
            f(i0 + 3, i0 + 3 < n ? order_key(v[u].w) : 0u);
          }
        }
      }
    }
  }
};

__device__ __forceinline__ unsigned long long word(uint32_t key, int idx) {
  return (static_cast<unsigned long long>(key) << 32) | static_cast<uint32_t>(~static_cast<uint32_t>(idx));
}
__device__ __forceinline__ int32_t word_idx(unsigned long long w) {
  return static_cast<int32_t>(~static_cast<uint32_t>(w & 0xFFFFFFFFull));
}

// Winners: keys > T, and keys == T with complemented index >= I (the `need`
// smallest indices; I = 0 keeps every key equal to T). each(f) visits
// (index, key) of this thread's elements. Writes the words to sh.wa.
template <typename Each>
__device__ __forceinline__ void collect_winners(TopkShared& sh, Each&& each, uint32_t T, uint32_t I) {
  uint32_t c = 0;
  each([&](int idx, uint32_t key) { c += key > T || (key == T && ~static_cast<uint32_t>(idx) >= I); });
  uint32_t tot;
  uint32_t pos = block_scan(c, sh.red, tot);
  each([&](int idx, uint32_t key) {
    if (key > T || (key == T && ~static_cast<uint32_t>(idx) >= I)) {
      if (pos < kMaxTopk) sh.wa[pos] = word(key, idx);
      ++pos;
    }
  });
  lds_barrier();
}

// Among the keys equal to T, the `need` smallest indices are those whose
// complemented index is >= the returned threshold.
template <typename Each>
__device__ __forceinline__ uint32_t tie_threshold(TopkShared& sh, Each&& each, uint32_t T, uint32_t need,
                                                  uint32_t eq_total, int n) {
  uint32_t I, need2, eq2;
  auto visit = [&](auto&& f) {
    each([&](int idx, uint32_t key) {
      if (key == T) f(~static_cast<uint32_t>(idx));
    });
  };
  select_small(sh, visit, ~static_cast<uint32_t>(n - 1), 0xFFFFFFFFu, need, eq_total, I, need2, eq2);
  return I;
}

// ---- sorting distinct 64-bit words (descending) ----------------------------------

// Bucket the distinct words src[off .. off+m), all within [mn, mx], on 12
// bits of (mx - word); only buckets whose ranks meet the window [lo, hi) go on:
// their words are placed in dst[off ..], every such bucket of <= kSmall words
// is ranked by counting and the indices of its ranks within the window are
// written to out[rank]; denser ones are appended to the work list wl (count
// in sh.misc[6]) with their exact word range. Each thread handles the fixed
// slots i = t + 512*j (j < 8) and issues every stage for all of them at once,
// so the LDS round trips of different slots overlap.
constexpr int kJ = kCap / kThreads;  // words per thread in a bucket pass

__device__ __forceinline__ void bucket_finish(TopkShared& sh, const unsigned long long (&w)[kJ],
                                              const uint32_t (&bk)[kJ], const bool (&valid)[kJ],
                                              unsigned long long* dst, int off, unsigned long long mx,
                                              unsigned long long mn, int shift, int nb, int lo, int hi, int32_t* out,
                                              int obase, uint32_t* wl);

__device__ __forceinline__ void bucket_pass(TopkShared& sh, const unsigned long long* src, unsigned long long* dst,
                                            int off, int m, unsigned long long mx, unsigned long long mn, int lo,
                                            int hi, int32_t* out, int obase, uint32_t* wl) {
  constexpr int J = kJ;
  const int t = threadIdx.x;
  int shift, nb;
  digit_plan(mn, mx, 12, shift, nb);
  for (int i = 4 * t; i < nb; i += 4 * kThreads) {
    *reinterpret_cast<uint4*>(sh.cnt + i) = uint4{0u, 0u, 0u, 0u};
    *reinterpret_cast<uint4*>(sh.fill + i) = uint4{0u, 0u, 0u, 0u};
  }
  unsigned long long w[J];
  uint32_t bk[J];
  bool valid[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int i = t + j * kThreads;
    valid[j] = i < m;
    w[j] = valid[j] ? src[off + i] : mx;  // (unused slots: bucket 0, never placed)
    bk[j] = uint32_t((mx - w[j]) >> shift);
  }
  lds_barrier();
#pragma unroll
  for (int j = 0; j < J; ++j)
    if (valid[j]) atomicAdd(&sh.cnt[bk[j]], 1u);
  lds_barrier();
  bucket_finish(sh, w, bk, valid, dst, off, mx, mn, shift, nb, lo, hi, out, obase, wl);
}

// The rest of a bucket pass once sh.cnt holds the complete bucket counts of
// the words w[j] (valid[j]; bucket bk[j] = (mx - w) >> shift, nb buckets,
// sh.fill zero): bucket starts, the dense buckets that meet [lo, hi) listed
// in wl (count in sh.misc[6]), the words of those buckets placed into
// dst[off + ...], and the small ones ranked by counting.
__device__ __forceinline__ void bucket_finish(TopkShared& sh, const unsigned long long (&w)[kJ],
                                              const uint32_t (&bk)[kJ], const bool (&valid)[kJ],
                                              unsigned long long* dst, int off, unsigned long long mx,
                                              unsigned long long mn, int shift, int nb, int lo, int hi, int32_t* out,
                                              int obase, uint32_t* wl) {
  constexpr int J = kJ;
  const int t = threadIdx.x;
  // bucket starts: each thread owns 8 consecutive buckets
  const int b0 = 8 * t;
  uint32_t c[8], s = 0;
  if (b0 < nb) {
    const uint4 x = *reinterpret_cast<const uint4*>(sh.cnt + b0);
    const uint4 y = *reinterpret_cast<const uint4*>(sh.cnt + b0 + 4);
    c[0] = x.x; c[1] = x.y; c[2] = x.z; c[3] = x.w; c[4] = y.x; c[5] = y.y; c[6] = y.z; c[7] = y.w;
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = 0u;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    c[j] = b0 + j < nb ? c[j] : 0u;
    s += c[j];
  }
  uint32_t tot;
  uint32_t run = block_scan(s, sh.red, tot);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (b0 + j < nb) sh.bins[b0 + j] = run;
    if (c[j] > kSmall && off + int(run) < hi && off + int(run + c[j]) > lo) {
      const uint32_t slot = atomicAdd(&sh.misc[6], 1u);
      if (slot < kMaxWork) {
        const unsigned long long bmx = mx - (static_cast<unsigned long long>(b0 + j) << shift);
        const unsigned long long span = (1ull << shift) - 1ull;
        const unsigned long long bmn = bmx - mn > span ? bmx - span : mn;
        uint32_t* e = wl + 6 * slot;
        e[0] = off + run;
        e[1] = c[j];
        e[2] = uint32_t(bmx >> 32);
        e[3] = uint32_t(bmx);
        e[4] = uint32_t(bmn >> 32);
        e[5] = uint32_t(bmn);
      }
    }
    run += c[j];
  }
  lds_barrier();
  uint32_t start[J], cb[J], slot[J];
  bool keep[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    start[j] = sh.bins[bk[j]];
    cb[j] = sh.cnt[bk[j]];
    keep[j] = valid[j] && off + int(start[j]) < hi && off + int(start[j] + cb[j]) > lo;
  }
  // Slots that are not placed count on a spare word of their own (the
  // bitonic scratch, unused here), so every slot's atomic and load below is
  // unconditional: the LDS round trips of all slots of a thread are in
  // flight together.
  uint32_t* spare = reinterpret_cast<uint32_t*>(sh.v.net) + t;
#pragma unroll
  for (int j = 0; j < J; ++j) slot[j] = atomicAdd(keep[j] ? &sh.fill[bk[j]] : spare, 1u);
#pragma unroll
  for (int j = 0; j < J; ++j)
    if (keep[j]) dst[off + start[j] + slot[j]] = w[j];
  lds_barrier();
  // rank inside small buckets: count the larger words of the bucket. The
  // elements placed in a small bucket are first listed (word in the bitonic
  // scratch, bucket start and size in sh.bins, free now), so that each is
  // ranked by one thread in eight-wide batches of LDS reads, whatever slot
  // it came from.
  uint32_t nl = 0;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    cb[j] = keep[j] && cb[j] <= kSmall ? cb[j] : 0u;
    nl += cb[j] != 0u;
  }
  uint32_t n_live;
  uint32_t lp = block_scan(nl, sh.red, n_live);
#pragma unroll
  for (int j = 0; j < J; ++j) {
    if (cb[j]) {
      sh.v.net[lp] = w[j];
      sh.bins[lp] = uint32_t(off + int(start[j])) | (cb[j] << 16);
      ++lp;
    }
  }
  lds_barrier();
  for (uint32_t e = t; e < n_live; e += kThreads) {
    const unsigned long long we = sh.v.net[e];
    const uint32_t sc = sh.bins[e];
    const uint32_t b0 = sc & 0xFFFFu, c = sc >> 16;
    uint32_t rk = 0;
    for (uint32_t q0 = 0; q0 < c; q0 += 8) {
      unsigned long long y[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) y[u] = dst[b0 + (q0 + u < c ? q0 + u : 0u)];  // past the bucket: not counted
#pragma unroll
      for (int u = 0; u < 8; ++u) rk += (q0 + u < c) & (y[u] > we);
    }
    const int at = int(b0 + rk);
    if (at >= lo && at < hi) out[at - obase] = word_idx(we);
  }
  lds_barrier();  // orders the LDS use only; the index stores need not complete here
}

// Bitonic network (descending) on src[off .. off+m), m <= kCap; writes the
// indices of the ranks in [lo, hi) (rank q to out[q - obase]).
__device__ __forceinline__ void bitonic_segment(TopkShared& sh, const unsigned long long* src, int off, int m,
                                                int lo, int hi, int32_t* out, int obase) {
  const int t = threadIdx.x;
  int P = 1;
  while (P < m) P <<= 1;
  for (int i = t; i < P; i += kThreads) sh.v.net[i] = i < m ? src[off + i] : 0ull;
  lds_barrier();
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = t; i < P / 2; i += kThreads) {
        const int l = 2 * i - (i & (stride - 1));
        const int h = l + stride;
        const unsigned long long a = sh.v.net[l], b = sh.v.net[h];
        if (((l & size) == 0) ? (a < b) : (a > b)) {
          sh.v.net[l] = b;
          sh.v.net[h] = a;
        }
      }
      lds_barrier();
    }
  }
  for (int i = t; i < m; i += kThreads)
    if (off + i >= lo && off + i < hi) out[off + i - obase] = word_idx(sh.v.net[i]);
  lds_barrier();
}

__device__ __forceinline__ void sort_levels(TopkShared& sh, const unsigned long long* src, unsigned long long* dst,
                                            int cur, int nitems, int level0, int lo, int hi, int32_t* out,
                                            int obase);

// Sort the m distinct words in sh.wa (all within [mn, mx]) descending and
// write the indices of the ranks q in [lo, hi) to out[q - obase].
__device__ __forceinline__ void sort_words(TopkShared& sh, int m, unsigned long long mx, unsigned long long mn,
                                           int lo, int hi, int32_t* out, int obase = 0) {
  if (threadIdx.x == 0) {
    uint32_t* e = sh.work[0];
    e[0] = 0u;
    e[1] = uint32_t(m);
    e[2] = uint32_t(mx >> 32);
    e[3] = uint32_t(mx);
    e[4] = uint32_t(mn >> 32);
    e[5] = uint32_t(mn);
  }
  sort_levels(sh, sh.wa, sh.u.wb, 0, 1, 0, lo, hi, out, obase);
}

// The passes of sort_words from `level` on: nitems segments listed in
// sh.work[cur] (offset, length, max, min), their words in src.
__device__ __forceinline__ void sort_levels(TopkShared& sh, const unsigned long long* src, unsigned long long* dst,
                                            int cur, int nitems, int level0, int lo, int hi, int32_t* out,
                                            int obase) {
  for (int level = level0; level < 4; ++level) {
    if (threadIdx.x == 0) sh.misc[6] = 0u;
    lds_barrier();
    if (level == 3) {  // still dense after three splits: sorting network
      for (int i = 0; i < nitems; ++i)
        bitonic_segment(sh, src, int(sh.work[cur][6 * i]), int(sh.work[cur][6 * i + 1]), lo, hi, out, obase);
      return;
    }
    for (int i = 0; i < nitems; ++i) {
      const uint32_t* e = sh.work[cur] + 6 * i;
      const unsigned long long emx = (static_cast<unsigned long long>(e[2]) << 32) | e[3];
      const unsigned long long emn = (static_cast<unsigned long long>(e[4]) << 32) | e[5];
      bucket_pass(sh, src, dst, int(e[0]), int(e[1]), emx, emn, lo, hi, out, obase, sh.work[cur ^ 1]);
    }
    const int next = int(sh.misc[6]);
    if (next > kMaxWork) {  // more dense buckets than the list holds: redo these segments
      for (int i = 0; i < nitems; ++i)
        bitonic_segment(sh, src, int(sh.work[cur][6 * i]), int(sh.work[cur][6 * i + 1]), lo, hi, out, obase);
      return;
    }
    if (next == 0) return;
    nitems = next;
    cur ^= 1;
    const unsigned long long* tmp = src;
    src = dst;
    dst = const_cast<unsigned long long*>(tmp);
    lds_barrier();
  }
}

__device__ __forceinline__ int row_len(const TopkArgs& a, int r) {
  const int q = a.q_pos ? a.q_pos[r] : a.seq_len[r / a.qps] - a.qps + r % a.qps;
  int n = q + 1;
  if (n > a.max_n) n = a.max_n;
  if (n < 0) n = 0;
  return n;
}

// Pivot from the sample sh.v.samp[0..ns) (every SS-th key of the row, range
// [smin, smax]). The t-th largest sample is taken, t chosen so that the count
// of keys above it (about t*SS, with a standard deviation of about
// sqrt(t)*SS) falls below k only 3 deviations down; the pivot is the lower
// edge of the 12-bit bin holding it, refined by further 12-bit histograms
// over the samples of that bin (from their smallest to their largest value;
// at most three passes reach single values) while the bin holds more than a
// few samples past t: a heavy tail stretches the range and widens the bins.
// A bin whose samples are all equal (a tie class at the t-th sample) ends
// the search on that exact value, whose keys the candidate launch then lists
// in index order.
__device__ __forceinline__ uint32_t sample_pivot(TopkShared& sh, int ns, int SS, int k, uint32_t smin, uint32_t smax) {
  const float kq = float(k) / float(SS);
  const float rt = 1.5f + sqrtf(2.25f + kq);
  uint32_t ts = uint32_t(ceilf(rt * rt));
  if (ts > uint32_t(ns)) ts = uint32_t(ns);
  if (!(smin < smax)) return smin;
  uint32_t lo = smin, hi = smax, target = ts;
  for (int pass = 0; pass < 3; ++pass) {
    int shift, nb;
    digit_plan(lo, hi, 12, shift, nb);
    clear_bins(sh.bins, kBins);  // (find_crossing's last barrier ended the reads of the previous pass)
    lds_barrier();
    for (int i = int(threadIdx.x); i < ns; i += kThreads) {
      const uint32_t x = sh.v.samp[i];
      if (x >= lo && x <= hi) atomicAdd(&sh.bins[(x - lo) >> shift], 1u);
    }
    lds_barrier();
    uint32_t b, above, cnt;
    find_crossing(sh, target, b, above, cnt);
    const uint32_t blo = lo + (b << shift);
    if (shift == 0 || above + cnt <= target + 8) return blo;
    const unsigned long long top = static_cast<unsigned long long>(blo) + ((1ull << shift) - 1ull);
    const uint32_t bhi = top < hi ? static_cast<uint32_t>(top) : hi;
    // the bin's smallest and largest sample (find_crossing's barrier ended
    // the histogram's atomics; the exchange below orders the next clear)
    uint32_t vmin = 0xFFFFFFFFu, vmax = 0u;
    for (int i = int(threadIdx.x); i < ns; i += kThreads) {
      const uint32_t x = sh.v.samp[i];
      if (x >= blo && x <= bhi) {
        vmin = min(vmin, x);
        vmax = max(vmax, x);
      }
    }
    block_minmax(vmin, vmax, sh.red);
    if (vmin == vmax) return vmin;
    lo = vmin;
    hi = vmax;
    target -= above;
  }
  return lo;
}

// Exact selection over a whole row held by `row` (any EPT), for rows whose
// pivot did not yield k..kCap candidates: radix select finds the k-th key T,
// the kept keys equal to T are the `need` smallest indices, and the k winners
// are sorted; ranks q in [lo, hi) go to out[q - obase].
template <int EPT>
__device__ __forceinline__ void select_exact(TopkShared& sh, const Row<EPT>& row, int n, int k, int32_t* out,
                                             int lo = 0, int hi = kMaxTopk, int obase = 0) {
  auto each_row = [&](auto&& f) { row.each(f); };
  uint32_t lo_key = 0xFFFFFFFFu, hi_key = 0u;
  row.each([&](int idx, uint32_t key) {
    if (idx < n) {
      lo_key = min(lo_key, key);
      hi_key = max(hi_key, key);
    }
  });
  block_minmax(lo_key, hi_key, sh.red);
  uint32_t T, need, eq_total, I = 0u;
  auto visit_keys = [&](auto&& f) { row.each([&](int, uint32_t key) { f(key); }); };
  select_full(sh, visit_keys, lo_key, hi_key, uint32_t(k), uint32_t(n), T, need, eq_total);
  if (need < eq_total) I = tie_threshold(sh, each_row, T, need, eq_total, n);
  collect_winners(sh, each_row, T, I);
  sort_words(sh, k, (static_cast<unsigned long long>(hi_key) << 32) | 0xFFFFFFFFull,
             static_cast<unsigned long long>(T) << 32, lo, hi < k ? hi : k, out, obase);
}

template <int EPT>
__global__ __launch_bounds__(kThreads) void topk_kernel(TopkArgs a) {
  __shared__ TopkShared sh;
  const int r = blockIdx.x;
  const int t = threadIdx.x;
  const int n = row_len(a, r);
  const int k = a.k;
  const int k_eff = n < k ? n : k;
  int32_t* out = a.idx + int64_t(r) * k;
  for (int j = k_eff + t; j < k; j += kThreads) out[j] = -1;

  Row<EPT> row;
  row.load(a.scores + int64_t(r) * a.ld, n);
  auto each_row = [&](auto&& f) { row.each(f); };

  if (n <= k) {  // every key is a winner: sort them all
    uint32_t c = 0, lo = 0xFFFFFFFFu, hi = 0u;
    row.each([&](int idx, uint32_t key) {
      if (idx < n) {
        ++c;
        lo = min(lo, key);
        hi = max(hi, key);
      }
    });
    block_minmax(lo, hi, sh.red);
    uint32_t tot;
    uint32_t pos = block_scan(c, sh.red, tot);
    row.each([&](int idx, uint32_t key) {
      if (idx < n) sh.wa[pos++] = word(key, idx);
    });
    lds_barrier();
    sort_words(sh, n, (static_cast<unsigned long long>(hi) << 32) | 0xFFFFFFFFull,
               static_cast<unsigned long long>(lo) << 32, 0, n, out);
    return;
  }

  // ---- 1. pivot from the fixed sample ------------------------------------------------
  int SS = 16;
  while ((n + SS - 1) / SS > kMaxSamples) SS <<= 1;
  const int ns = (n + SS - 1) / SS;
  uint32_t smin = 0xFFFFFFFFu, smax = 0u;
  row.sample(SS, [&](int i, uint32_t key) {  // i = index / SS
    sh.v.samp[i] = key;
    smin = min(smin, key);
    smax = max(smax, key);
  });
  block_minmax(smin, smax, sh.red);
  const uint32_t pivot = sample_pivot(sh, ns, SS, k, smin, smax);

  // ---- 2. candidates >= pivot ---------------------------------------------------------
  uint32_t c = 0, cmax = 0;
  row.each([&](int, uint32_t key) {
    c += key >= pivot;
    cmax = max(cmax, key);
  });
  uint32_t C;
  uint32_t pos = block_scan(c, sh.red, C);
  if (C >= uint32_t(k) && C <= uint32_t(kCap)) {
    row.each([&](int idx, uint32_t key) {
      if (key >= pivot) sh.wa[pos++] = word(key, idx);
    });
    cmax = block_max(cmax, sh.red);  // (its barrier publishes the candidates)
    // ---- 3. the k largest candidate words, in order -----------------------------------
    sort_words(sh, int(C), (static_cast<unsigned long long>(cmax) << 32) | 0xFFFFFFFFull,
               static_cast<unsigned long long>(pivot) << 32, 0, k, out);
    return;
  }

  // ---- fallback: exact select over the whole row, then sort the k winners ----------------
  select_exact(sh, row, n, k, out);
}

// Split selection for few long rows, in two launches.
//  topk_cand_kernel: the row is cut into slices of kTile keys, one workgroup
//    each; every workgroup derives the same pivot from the row's sample and
//    writes its slice's candidates (keys >= pivot, as words, in index order)
//    and their count to the slice's own region of the workspace.
//  topk_window_kernel: one workgroup per 128 output ranks of a row gathers
//    the row's candidates, buckets them and ranks only the buckets that meet
//    its window (or, when fewer than k or more than kCap keys cleared the
//    pivot, the first workgroup of the row runs the exact selection over the
//    whole row).
// The candidate set is fixed by the pivot and every rank is unique, so the
// result does not depend on how the work is spread.
constexpr int kWindow = 128;  // output ranks per workgroup of the second launch

template <int T>
__global__ __launch_bounds__(kThreads) void topk_cand_kernel(TopkArgs a, int slices) {
  __shared__ TopkShared sh;
  const int r = blockIdx.x / slices, g = blockIdx.x % slices;
  const int t = threadIdx.x;
  const int n = row_len(a, r);
  const int k = a.k;
  const float* row = a.scores + int64_t(r) * a.ld;
  unsigned long long* cand = a.cand + (int64_t(r) * slices + g) * (int64_t(T) * kTile);
  // the slice's candidate words go out as buffer stores at device scope
  // (cache policy sc1, through the L2), so that the kernel's end has none of
  // their lines to write back before the next launch (0.4-0.5 us a step at
  // 4 x 32K and 8 x 128K; the values are the same)
  const __amdgpu_buffer_rsrc_t cand_rs =
      __builtin_amdgcn_make_buffer_rsrc(cand, 0, int(T * kTile * sizeof(unsigned long long)), 0x00020000);

  // this slice's scores (T tiles of kTile keys), loaded first so the loads
  // overlap the pivot
  float4 sv[T];
#pragma unroll
  for (int j = 0; j < T; ++j) {
    const int i0 = (g * T + j) * kTile + 4 * t;
    sv[j] = i0 < n ? *reinterpret_cast<const float4*>(row + i0) : float4{0.f, 0.f, 0.f, 0.f};
  }

  // ---- pivot (identical in every slice of the row; 0 when every key wins) ----------------
  // from the indexer's every-16th-score sample (every SS-th score, at most
  // kMaxSamples), staged in LDS
  uint32_t pivot = 0u;
  if (n > k) {
    int SS = 16;
    while ((n + SS - 1) / SS > kMaxSamples) SS <<= 1;
    const int ns = (n + SS - 1) / SS;
    // every sample load is issued before the first wait (indexes past ns
    // re-read the last sample and are not used), in batches of 2048 samples
    const float* src = a.sample ? a.sample + int64_t(r) * a.ld_sample : row;
    const int64_t stride = a.sample ? SS / 16 : SS;
    constexpr int PT = kMaxSamples / kThreads;
    constexpr int PQ = 4;
    float sv_[PT];
#pragma unroll
    for (int q = 0; q < PT / PQ; ++q) {
      if (q == 0 || ns > kThreads * PQ * q) {
#pragma unroll
        for (int j = PQ * q; j < PQ * (q + 1); ++j) sv_[j] = src[int64_t(min(t + kThreads * j, ns - 1)) * stride];
      }
    }
    uint32_t smin = 0xFFFFFFFFu, smax = 0u;
#pragma unroll
    for (int q = 0; q < PT / PQ; ++q) {
      if (q == 0 || ns > kThreads * PQ * q) {
#pragma unroll
        for (int j = PQ * q; j < PQ * (q + 1); ++j) {
          const int i = t + kThreads * j;
          if (i < ns) {
            const uint32_t key = order_key(sv_[j]);
            sh.v.samp[i] = key;
            smin = min(smin, key);
            smax = max(smax, key);
          }
        }
      }
    }
    block_minmax(smin, smax, sh.red);
    pivot = sample_pivot(sh, ns, SS, k, smin, smax);
  }

  // ---- this slice's candidates: keys above the pivot (any order), then the
  // keys equal to it in index order (tile, then thread, then slot) --------------------------
  uint32_t cg = 0, cm = 0, ce[T];
#pragma unroll
  for (int j = 0; j < T; ++j) {
    const int i0 = (g * T + j) * kTile + 4 * t;
    const uint32_t key[4] = {order_key(sv[j].x), order_key(sv[j].y), order_key(sv[j].z), order_key(sv[j].w)};
    ce[j] = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool valid = i0 + e < n;
      cg += valid && key[e] > pivot;
      ce[j] += valid && key[e] == pivot;
      cm = valid && key[e] >= pivot ? max(cm, key[e]) : cm;
    }
  }
  // one exchange: offsets of the words above the pivot (any thread order) and
  // their largest key; offsets of the keys equal to it in (tile, thread) order
  uint32_t G, cmax, E, pos, epos[T];
  {
    const uint32_t xg = wave_incl_scan(cg), xm = wave_max(cm);
    uint32_t xe[T];
#pragma unroll
    for (int j = 0; j < T; ++j) xe[j] = wave_incl_scan(ce[j]);
    if (lane_id() == 63) {
      sh.xred[wave_id()] = xg;
      sh.xred[kWaves + wave_id()] = xm;
#pragma unroll
      for (int j = 0; j < T; ++j) sh.xred[(2 + j) * kWaves + wave_id()] = xe[j];
    }
    lds_barrier();
    uint32_t gb = 0, gt = 0, mm = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const uint32_t c = sh.xred[w];
      gb += w < wave_id() ? c : 0u;
      gt += c;
      mm = max(mm, sh.xred[kWaves + w]);
    }
    pos = gb + xg - cg;
    G = gt;
    cmax = mm;
    uint32_t run = 0;
#pragma unroll
    for (int j = 0; j < T; ++j) {
      uint32_t eb = 0, et = 0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const uint32_t c = sh.xred[(2 + j) * kWaves + w];
        eb += w < wave_id() ? c : 0u;
        et += c;
      }
      epos[j] = run + eb + xe[j] - ce[j];
      run += et;
    }
    E = run;
  }
#pragma unroll
  for (int j = 0; j < T; ++j) {
    const int i0 = (g * T + j) * kTile + 4 * t;
    const uint32_t key[4] = {order_key(sv[j].x), order_key(sv[j].y), order_key(sv[j].z), order_key(sv[j].w)};
    uint32_t q = G + epos[j];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (i0 + e < n && key[e] >= pivot) {
        const bool eq = key[e] == pivot;
        const unsigned long long w = word(key[e], i0 + e);
        typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 w2 = {uint32_t(w), uint32_t(w >> 32)};
        __builtin_amdgcn_raw_buffer_store_b64(w2, cand_rs, int((eq ? q : pos) * sizeof(unsigned long long)), 0, 16);
        q += eq;
        pos += !eq;
      }
    }
  }
  if (t == 0) {
    // the slice record at device scope (sc1, through the L2 to memory), like
    // the words: the next launch reads every record first, from any XCD, and
    // started about 0.5 us sooner at 4 x 32K than after their write-back at
    // this kernel's end (the values are the same)
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 rec = {G + E, cmax, pivot, E};
    uint4* dst = reinterpret_cast<uint4*>(a.state) + int64_t(r) * slices + g;
    asm volatile("global_store_dwordx4 %0, %1, off sc1" ::"v"(dst), "v"(rec) : "memory");
  }
}

// Ranks [lo, hi) of row r (hi <= min(n, k)) from the candidates of the
// slices, indices to out[rank - obase]; when fewer than k or more than kCap
// keys cleared the pivot, the exact selection over the whole row instead.
// Slice counts (slices <= kThreads) and, in the same round trip, the first
// words of every slice's region: thread t reads words j*tps + t%tps of slice
// t/tps (tps threads per slice), which covers the typical count. Issued apart
// from the selection so that a caller can start them before other work.
struct WindowLoads {
  uint4 st;   // slice t's (count, largest candidate key, pivot, keys equal to it), t < slices;
              // for slices <= 64, every wave holds the records (lane l: slice l)
  uint32_t own;  // the count of the slice whose words this thread holds
  unsigned long long x[kCap / kThreads];
};

__device__ __forceinline__ int window_tps(int slices) {
  int tps = kThreads;
  while (tps > 1 && tps * slices > kThreads) tps >>= 1;
  return tps;
}

__device__ __forceinline__ void window_loads(const TopkArgs& a, int r, int slices, WindowLoads& L) {
  const int t = threadIdx.x;
  const int64_t stride = int64_t(a.slice_tiles) * kTile;  // words per slice region
  const unsigned long long* cand = a.cand + int64_t(r) * slices * stride;
  const uint4* st = reinterpret_cast<const uint4*>(a.state) + int64_t(r) * slices;
  const int sr = slices <= 64 ? lane_id() : t;
  L.st = sr < slices ? st[sr] : uint4{0u, 0u, 0u, 0u};
  const int tps = window_tps(slices);
  const int sg = t / tps, sl = t % tps;
  L.own = sg < slices ? st[sg].x : 0u;
#pragma unroll
  for (int j = 0; j < kCap / kThreads; ++j) L.x[j] = sg < slices ? cand[sg * stride + j * tps + sl] : 0ull;
}

// The candidates gathered into sh.wa in slice order (offset `at` of slice t
// from the scan of the counts) and sorted there: the general form, for rows
// whose slices hold more words than were read ahead, or whose window meets
// more dense buckets than one pass lists.
__device__ __forceinline__ void window_gather_sort(TopkShared& sh, const TopkArgs& a, int r, int slices, uint32_t C,
                                                   uint32_t at, uint32_t longest, int lo, int hi, int32_t* out,
                                                   int obase, const WindowLoads& L) {
  const int t = threadIdx.x;
  constexpr int J = kJ;
  const int64_t stride = int64_t(a.slice_tiles) * kTile;
  const unsigned long long* cand = a.cand + int64_t(r) * slices * stride;
  const int tps = window_tps(slices);
  const int sg = t / tps, sl = t % tps;
  if (t < slices) {
    sh.bins[t] = at;
    sh.cnt[t] = L.st.x;
  }
  lds_barrier();
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  const int m = sg < slices ? int(sh.cnt[sg]) : 0, o = sg < slices ? int(sh.bins[sg]) : 0;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int i = j * tps + sl;
    if (i < m) {
      sh.wa[o + i] = L.x[j];
      const uint32_t kx = uint32_t(L.x[j] >> 32);
      kmin = min(kmin, kx);
      kmax = max(kmax, kx);
    }
  }
  // the rest of the longer slices (rows with skewed candidates), J*tps more
  // words of every slice per round, all of a round's loads in flight at once
  for (int b0 = J * tps; b0 < int(longest); b0 += J * tps) {
    unsigned long long y[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int i = b0 + j * tps + sl;
      y[j] = i < m ? cand[sg * stride + i] : 0ull;
    }
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int i = b0 + j * tps + sl;
      if (i < m) {
        sh.wa[o + i] = y[j];
        const uint32_t ky = uint32_t(y[j] >> 32);
        kmin = min(kmin, ky);
        kmax = max(kmax, ky);
      }
    }
  }
  block_minmax(kmin, kmax, sh.red);  // (its barriers publish the gathered words)
  sort_words(sh, int(C), (static_cast<unsigned long long>(kmax) << 32) | 0xFFFFFFFFull,
             static_cast<unsigned long long>(kmin) << 32, lo, hi, out, obase);
}

// Ranks [lo, hi) when the k-th rank falls in the class of keys equal to the
// pivot (a tie class too large for the candidate capacity): the G keys above
// the pivot (G < k_eff) take ranks 0 .. G-1 in their own order; rank G + j is
// the j-th key of the class in index order (lower index first), which the
// candidate launch listed after each slice's words above the pivot. gat and
// eat: slice t's offsets among the words above the pivot and among the class.
__device__ __forceinline__ void window_ties(TopkShared& sh, const TopkArgs& a, int r, int slices, uint32_t G, int lo,
                                            int hi, int32_t* out, int obase, const WindowLoads& L, uint32_t gat,
                                            uint32_t eat) {
  const int t = threadIdx.x;
  const int64_t stride = int64_t(a.slice_tiles) * kTile;  // words per slice region
  const unsigned long long* cand = a.cand + int64_t(r) * slices * stride;
  if (t < slices) {
    sh.bins[t] = eat;               // first class rank of the slice
    sh.cnt[t] = L.st.x - L.st.w;    // its words above the pivot
    sh.fill[t] = gat;               // their offset in the order of slices
  }
  lds_barrier();
  // ranks G + j: the slice is the last one whose first class rank is <= j
  for (int q = (lo > int(G) ? lo : int(G)) + t; q < hi; q += kThreads) {
    const uint32_t j = uint32_t(q) - G;
    int s0 = 0, s1 = slices - 1;
    while (s0 < s1) {
      const int m = (s0 + s1 + 1) >> 1;
      if (sh.bins[m] <= j) s0 = m;
      else s1 = m - 1;
    }
    out[q - obase] = word_idx(cand[int64_t(s0) * stride + sh.cnt[s0] + (j - sh.bins[s0])]);
  }
  if (lo >= int(G)) return;
  // ranks [lo, min(hi, G)): the words above the pivot, gathered and sorted
  const int tps = window_tps(slices);
  const int sg = t / tps, sl = t % tps;
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  if (sg < slices) {
    const int m = int(sh.cnt[sg]), o = int(sh.fill[sg]);
    for (int i = sl; i < m; i += tps) {
      const unsigned long long w = cand[int64_t(sg) * stride + i];
      sh.wa[o + i] = w;
      kmin = min(kmin, uint32_t(w >> 32));
      kmax = max(kmax, uint32_t(w >> 32));
    }
  }
  block_minmax(kmin, kmax, sh.red);  // (its barriers publish the gathered words)
  sort_words(sh, int(G), (static_cast<unsigned long long>(kmax) << 32) | 0xFFFFFFFFull,
             static_cast<unsigned long long>(kmin) << 32, lo, hi < int(G) ? hi : int(G), out, obase);
}

// LDS that window_select_fast expects zero on entry: the first pass's bucket
// counts and fill counters and the dense-bucket count. Called before a
// barrier that the caller runs anyway.
__device__ __forceinline__ void window_fast_clear(TopkShared& sh) {
  clear_bins(sh.cnt, kBins);
  clear_bins(sh.fill, kBins);
  if (threadIdx.x == 0) sh.misc[6] = 0u;
}

// window_select for the usual row, in four barriers and few instructions
// (eight waves share four SIMDs, so each wave's instruction count is the
// time): at most 64 slices, every candidate word among the JJ slots of the
// threads of its slice, and k_eff <= C <= kCap; the slice records come
// reduced (C, longest slice, largest candidate key, pivot). One bucket pass
// on 12 bits of (largest candidate - word) over
// [pivot, largest candidate], on the keys alone (32-bit) when the digit lies
// above the index bits. The buckets that meet [lo, hi) are the index range
// [b_lo, b_hi] (those holding ranks lo and hi - 1 and all between), so a
// word's bucket number alone decides whether it is placed; placed words fill
// the contiguous range [s_lo, s_hi) of sh.u.wb (the first such bucket's
// start to the last one's end), each beside its bucket's start and count in
// sh.v.samp, and that range is ranked one word per thread (count of the
// larger words of its bucket, for buckets of up to kFastSmall words: the
// words are ranked in parallel, so a bucket of many near-equal scores costs
// one pass over it instead of further bucket passes). Every LDS access of a
// phase is issued before the first wait. Denser buckets that meet the
// window go on to sort_levels.
// Expects window_fast_clear's LDS zero (ordered by a barrier).
template <int JJ>
__device__ __forceinline__ bool window_select_fast_j(TopkShared& sh, const TopkArgs& a, int r, int slices, int lo,
                                                     int hi, int32_t* out, int obase, const WindowLoads& L, uint32_t C,
                                                     uint32_t longest, uint32_t kmax, uint32_t pivot, int tps) {
  const int t = threadIdx.x;
  constexpr int J = kJ;
  const int sg = t / tps, sl = t % tps;
  // this thread's words: the first J read ahead, the rest (JJ > J: slices
  // longer than the read-ahead) loaded now, all in one round trip
  unsigned long long w[JJ];
#pragma unroll
  for (int j = 0; j < J; ++j) w[j] = L.x[j];
  if constexpr (JJ > J) {
    const int64_t stride = int64_t(a.slice_tiles) * kTile;
    const unsigned long long* cand = a.cand + int64_t(r) * slices * stride + int64_t(sg) * stride;
#pragma unroll
    for (int j = J; j < JJ; ++j) w[j] = sg < slices && uint32_t(j * tps + sl) < L.own ? cand[j * tps + sl] : 0ull;
  }
  const unsigned long long mx = (static_cast<unsigned long long>(kmax) << 32) | 0xFFFFFFFFull;
  const unsigned long long mn = static_cast<unsigned long long>(pivot) << 32;
  int shift, nb;
  digit_plan(mn, mx, 12, shift, nb);  // nb <= kBins
  // (mx - w) >> shift == (kmax - key) >> (shift - 32) when shift >= 32: the
  // low halves (0xFFFFFFFF - ~index = index) never carry into the key half
  const bool keys_only = shift >= 32;
  const int ks = keys_only ? shift - 32 : 0;
  auto bucket = [&](unsigned long long v) -> uint32_t {
    return keys_only ? (kmax - uint32_t(v >> 32)) >> ks : uint32_t((mx - v) >> shift);
  };
  uint32_t bk[JJ];
  bool valid[JJ];
#pragma unroll
  for (int j = 0; j < JJ; ++j) {
    valid[j] = sg < slices && uint32_t(j * tps + sl) < L.own;
    bk[j] = valid[j] ? bucket(w[j]) : 0u;  // (unused slots: bucket 0, never placed)
    if (valid[j]) atomicAdd(&sh.cnt[bk[j]], 1u);
  }
  lds_barrier();
  // bucket starts: thread t owns buckets 8t .. 8t+7 (unused ones are zero);
  // the thread whose buckets hold rank lo (hi - 1) records that bucket and
  // where it starts (ends): the placed range
  uint32_t c[8], st[8];
  {
    const uint4 x = *reinterpret_cast<const uint4*>(sh.cnt + 8 * t);
    const uint4 y = *reinterpret_cast<const uint4*>(sh.cnt + 8 * t + 4);
    c[0] = x.x; c[1] = x.y; c[2] = x.z; c[3] = x.w; c[4] = y.x; c[5] = y.y; c[6] = y.z; c[7] = y.w;
  }
  uint32_t tot = 0, cmax = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    tot += c[j];
    cmax = max(cmax, c[j]);
  }
  {
    const uint32_t xs = wave_incl_scan(tot);
    if (lane_id() == 63) sh.red[wave_id()] = xs;
    lds_barrier();
    uint32_t base = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) base += w < wave_id() ? sh.red[w] : 0u;
    st[0] = base + xs - tot;
  }
#pragma unroll
  for (int j = 1; j < 8; ++j) st[j] = st[j - 1] + c[j - 1];
  *reinterpret_cast<uint4*>(sh.bins + 8 * t) = uint4{st[0], st[1], st[2], st[3]};
  *reinterpret_cast<uint4*>(sh.bins + 8 * t + 4) = uint4{st[4], st[5], st[6], st[7]};
  const uint32_t t_end = st[0] + tot;
  if (st[0] <= uint32_t(lo) && uint32_t(lo) < t_end) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (st[j] <= uint32_t(lo) && uint32_t(lo) < st[j] + c[j]) {
        sh.misc[8] = st[j];
        sh.misc[10] = 8 * t + j;
      }
  }
  if (st[0] < uint32_t(hi) && uint32_t(hi) <= t_end) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (st[j] < uint32_t(hi) && uint32_t(hi) <= st[j] + c[j]) {
        sh.misc[9] = st[j] + c[j];
        sh.misc[11] = 8 * t + j;
      }
  }
  if (cmax > uint32_t(kFastSmall)) {  // dense buckets that meet the window: listed for sort_levels
    for (int j = 0; j < 8; ++j) {
      if (c[j] > uint32_t(kFastSmall) && int(st[j]) < hi && int(st[j] + c[j]) > lo) {
        const uint32_t slot = atomicAdd(&sh.misc[6], 1u);
        if (slot < kMaxWork) {
          const unsigned long long bmx = mx - (static_cast<unsigned long long>(8 * t + j) << shift);
          const unsigned long long span = (1ull << shift) - 1ull;
          const unsigned long long bmn = bmx - mn > span ? bmx - span : mn;
          uint32_t* e = sh.work[1] + 6 * slot;
          e[0] = st[j];
          e[1] = c[j];
          e[2] = uint32_t(bmx >> 32);
          e[3] = uint32_t(bmx);
          e[4] = uint32_t(bmn >> 32);
          e[5] = uint32_t(bmn);
        }
      }
    }
  }
  lds_barrier();
  const int next = int(sh.misc[6]);
  const uint32_t s_lo = sh.misc[8], s_hi = sh.misc[9], b_lo = sh.misc[10], b_hi = sh.misc[11];
  // the words of the buckets that meet the window, placed at their bucket
  bool keep[JJ];
  uint32_t b0[JJ], cb[JJ], slot[JJ];
#pragma unroll
  for (int j = 0; j < JJ; ++j) keep[j] = valid[j] && bk[j] >= b_lo && bk[j] <= b_hi;
#pragma unroll
  for (int j = 0; j < JJ; ++j) {
    if (keep[j]) {
      b0[j] = sh.bins[bk[j]];
      cb[j] = sh.cnt[bk[j]];
      slot[j] = atomicAdd(&sh.fill[bk[j]], 1u);
    }
  }
#pragma unroll
  for (int j = 0; j < JJ; ++j) {
    if (keep[j]) {
      sh.u.wb[b0[j] + slot[j]] = w[j];
      sh.v.samp[b0[j] + slot[j]] = b0[j] | (cb[j] << 16);  // (both <= kCap < 2^16)
    }
  }
  lds_barrier();
  // rank of each placed word inside its (small) bucket
  for (uint32_t p = s_lo + uint32_t(t); p < s_hi; p += kThreads) {
    const unsigned long long w = sh.u.wb[p];
    const uint32_t m = sh.v.samp[p];
    const uint32_t wb0 = m & 0xFFFFu, wcb = m >> 16;
    if (wcb > uint32_t(kFastSmall)) continue;  // dense: sort_levels
    uint32_t rk = 0;
    for (uint32_t q0 = 0; q0 < wcb; q0 += 4) {
      unsigned long long y[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) y[u] = sh.u.wb[wb0 + (q0 + u < wcb ? q0 + u : 0u)];
#pragma unroll
      for (int u = 0; u < 4; ++u) rk += (q0 + u < wcb) & (y[u] > w);
    }
    const int at = int(wb0 + rk);
    if (at >= lo && at < hi) out[at - obase] = word_idx(w);
  }
  if (next == 0) return true;
  if (next > kMaxWork) {
    const uint4 rec = t < slices ? L.st : uint4{0u, 0u, 0u, 0u};
    const uint32_t at = wave_incl_scan(rec.x) - rec.x;  // slice t's offset (t < slices <= 64)
    lds_barrier();  // the ranking above still reads sh.bins and sh.cnt, which the gather rewrites
    window_gather_sort(sh, a, r, slices, C, at, longest, lo, hi, out, obase, L);
    return true;
  }
  sort_levels(sh, sh.u.wb, sh.wa, 1, next, 1, lo, hi, out, obase);
  return true;
}


// The usual row's short form (see window_select_fast_j): the slice records
// reduced by every wave itself, then the form whose word slots cover the
// longest slice -- the read-ahead alone, or twice it when a row's slices
// hold more candidates than the read-ahead (the slice count, and so the
// read-ahead per slice, is set by the longest row of the batch). Returns
// false, with no LDS touched, when the row needs window_select.
__device__ __forceinline__ bool window_select_fast(TopkShared& sh, const TopkArgs& a, int r, int slices, int n,
                                                   int lo, int hi, int32_t* out, int obase, const WindowLoads& L) {
  const int k_eff = n < a.k ? n : a.k;
  if (slices > 64) return false;
  const int tps = window_tps(slices);
  const uint32_t C = wave_sum(L.st.x);
  const uint32_t longest = wave_max(L.st.x), kmax = wave_max(L.st.y);
  const uint32_t pivot = lane_value(L.st.z, 0);
  if (C < uint32_t(k_eff) || C > uint32_t(kCap)) return false;
  if (longest <= uint32_t(kJ * tps))
    return window_select_fast_j<kJ>(sh, a, r, slices, lo, hi, out, obase, L, C, longest, kmax, pivot, tps);
  if (longest <= uint32_t(2 * kJ * tps))
    return window_select_fast_j<2 * kJ>(sh, a, r, slices, lo, hi, out, obase, L, C, longest, kmax, pivot, tps);
  return false;
}

// Ranks [lo, hi) of row r (hi <= min(n, k)) from the candidates of the
// slices, indices to out[rank - obase]; a tie class too large for the
// candidate capacity at the k-th rank goes to window_ties; when fewer than k
// keys, or more than kCap for another reason, cleared the pivot, the exact
// selection over the whole row runs instead.
// Usually the read-ahead words already are all of them: then the first
// bucket pass works on them in registers, on digits of the range [pivot,
// largest candidate] that the candidate kernel recorded, with no gather
// into LDS and no range reduction; later passes, if any, as in sort_words.
__device__ __forceinline__ void window_select(TopkShared& sh, const TopkArgs& a, int r, int slices, int n, int lo,
                                              int hi, int32_t* out, int obase, const WindowLoads& L) {
  const int t = threadIdx.x;
  const int k = a.k;
  const int k_eff = n < k ? n : k;
  constexpr int J = kJ;
  const int tps = window_tps(slices);
  const int sg = t / tps, sl = t % tps;
  // the first pass's bins, cleared before the exchange below orders them
  // before its histogram
  for (int i = 4 * t; i < kBins; i += 4 * kThreads) {
    *reinterpret_cast<uint4*>(sh.cnt + i) = uint4{0u, 0u, 0u, 0u};
    *reinterpret_cast<uint4*>(sh.fill + i) = uint4{0u, 0u, 0u, 0u};
  }
  if (t == 0) sh.misc[6] = 0u;
  // one exchange: slice offsets and the total (scan of the counts), the
  // largest candidate key, the longest slice, the pivot, and the same scan
  // of the counts of keys equal to the pivot
  const uint4 st = t < slices ? L.st : uint4{0u, 0u, 0u, 0u};  // (other waves may hold copies)
  const uint32_t cnt = st.x, ecnt = st.w;
  const uint32_t xs = wave_incl_scan(cnt), xe = wave_incl_scan(ecnt);
  {
    const uint32_t wm = wave_max(st.y), wc = wave_max(cnt);
    if (lane_id() == 63) {
      sh.red[wave_id()] = xs;
      sh.red[4 * kWaves + wave_id()] = xe;
    }
    if (lane_id() == 0) {
      sh.red[kWaves + wave_id()] = wm;
      sh.red[2 * kWaves + wave_id()] = wc;
    }
    if (t == 0) sh.red[3 * kWaves] = st.z;
    lds_barrier();
  }
  uint32_t C = 0, base = 0, kmax = 0, longest = 0, E = 0, ebase = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const uint32_t c = sh.red[w];
    base += w < wave_id() ? c : 0u;
    C += c;
    kmax = max(kmax, sh.red[kWaves + w]);
    longest = max(longest, sh.red[2 * kWaves + w]);
    const uint32_t ce = sh.red[4 * kWaves + w];
    ebase += w < wave_id() ? ce : 0u;
    E += ce;
  }
  const uint32_t pivot = sh.red[3 * kWaves];
  const uint32_t at = base + xs - cnt;  // slice t's offset in the gathered order
  const uint32_t G = C - E;             // keys above the pivot
  if (C > uint32_t(kCap) && G < uint32_t(k_eff) && C >= uint32_t(k_eff) && G <= uint32_t(kCap)) {
    window_ties(sh, a, r, slices, G, lo, hi, out, obase, L, at - (ebase + xe - ecnt), ebase + xe - ecnt);
    return;
  }
  if (C < uint32_t(k_eff) || C > uint32_t(kCap)) {
    Row<0> full;
    full.load(a.scores + int64_t(r) * a.ld, n);
    select_exact(sh, full, n, k, out, lo, hi, obase);
    return;
  }
  if (longest > uint32_t(J * tps)) {
    window_gather_sort(sh, a, r, slices, C, at, longest, lo, hi, out, obase, L);
    return;
  }
  const unsigned long long mx = (static_cast<unsigned long long>(kmax) << 32) | 0xFFFFFFFFull;
  const unsigned long long mn = static_cast<unsigned long long>(pivot) << 32;
  int shift, nb;
  digit_plan(mn, mx, 12, shift, nb);
  uint32_t bk[J];
  bool valid[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    valid[j] = sg < slices && uint32_t(j * tps + sl) < L.own;
    bk[j] = valid[j] ? uint32_t((mx - L.x[j]) >> shift) : 0u;  // (unused slots: bucket 0, never placed)
    if (valid[j]) atomicAdd(&sh.cnt[bk[j]], 1u);
  }
  lds_barrier();
  bucket_finish(sh, L.x, bk, valid, sh.u.wb, 0, mx, mn, shift, nb, lo, hi, out, obase, sh.work[1]);
  const int next = int(sh.misc[6]);
  if (next == 0) return;
  if (next > kMaxWork) {
    window_gather_sort(sh, a, r, slices, C, at, longest, lo, hi, out, obase, L);
    return;
  }
  sort_levels(sh, sh.u.wb, sh.wa, 1, next, 1, lo, hi, out, obase);
}

__global__ __launch_bounds__(kThreads) void topk_window_kernel(TopkArgs a, int slices, int windows) {
  __shared__ TopkShared sh;
  const int r = blockIdx.x / windows, w = blockIdx.x % windows;
  const int t = threadIdx.x;
  const int n = row_len(a, r);
  const int k = a.k;
  const int k_eff = n < k ? n : k;
  int32_t* out = a.idx + int64_t(r) * k;
  if (w == 0)
    for (int j = k_eff + t; j < k; j += kThreads) out[j] = -1;
  const int lo = w * kWindow, hi = lo + kWindow < k_eff ? lo + kWindow : k_eff;
  if (lo >= hi) return;
  WindowLoads L;
  window_loads(a, r, slices, L);
  window_fast_clear(sh);
  lds_barrier();
  if (!window_select_fast(sh, a, r, slices, n, lo, hi, out, 0, L)) window_select(sh, a, r, slices, n, lo, hi, out, 0, L);
}

// Decode with selection and attention fused: the workgroup of (query r, key
// split, head group) first selects the split's ranks [j_beg, j_end) exactly as
// topk_window_kernel does (8 waves), into LDS and (head group 0) the index
// output, then its waves 0..3 run the same attention core as the attention
// kernel over those keys. Same split plan and same core: the same bits as
// selection followed by the attention kernel on the recorded indices.
// M: kBF16 (bf16 latent rows) or kFP8 (e4m3 rows with a row scale).
template <int M>
__global__ __launch_bounds__(kThreads) void topk_attn_kernel(TopkArgs ta, AttnArgs aa, int slices, int splits,
                                                             int kps) {
  __shared__ union Shared {
    TopkShared sel;
    typename std::conditional<M == kFP8, attn::Smem8, attn::Smem<false>>::type att;
  } u;
  __shared__ int s_idx[kMaxTopk];
  const int HG = (aa.H + attn::kGroupHeads - 1) / attn::kGroupHeads;
  int r, split, hg;
  attn::map_block(blockIdx.x, aa.R, splits, HG, r, split, hg);
  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  // The selection's global loads go out first, in one round trip: the
  // candidate counts and words, the row's length and first cache row; then
  // (bf16 rows) the gather waves' query pieces, which land during the
  // selection.
  WindowLoads L;
  window_loads(ta, r, slices, L);
  const int64_t base = attn::seq_base(aa, r);
  const int n = row_len(ta, r);
  attn::QRegs qr;
  if (M != kFP8 && wave >= 4) attn::q_issue(aa, r, hg, wave - 4, t & 63, qr);
  const int k = ta.k;
  const int k_eff = n < k ? n : k;
  const int j_beg = split * kps;
  const int j_end = j_beg + kps < k ? j_beg + kps : k;
  // ranks past k_eff, and the attention's chunk tail past j_end, stay -1
  const int span = (j_end - j_beg + attn::kChunkKeys - 1) / attn::kChunkKeys * attn::kChunkKeys;
  for (int i = t; i < span; i += kThreads) s_idx[i] = -1;
  window_fast_clear(u.sel);
  lds_barrier();
  const int hi = j_end < k_eff ? j_end : k_eff;
  if (j_beg < hi && !window_select_fast(u.sel, ta, r, slices, n, j_beg, hi, s_idx, j_beg, L))
    window_select(u.sel, ta, r, slices, n, j_beg, hi, s_idx, j_beg, L);
  lds_barrier();  // the split's indices are in LDS; the selection's LDS is free
  if (hg == 0) {
    // the recorded indices at device scope (sc1), so that this kernel's end
    // has none of their lines to write back (0.6 us at 4 x 32K)
    for (int i = t; i < j_end - j_beg; i += kThreads) {
      int32_t* dst = ta.idx + int64_t(r) * k + j_beg + i;
      const int v = s_idx[i];
      asm volatile("global_store_dword %0, %1, off sc1" ::"v"(dst), "v"(v) : "memory");
    }
  }
  if constexpr (M == kFP8) {
    if (wave >= 4) return;  // barriers below count the four attention waves only
    attn::attend8(aa, r, split, splits, hg, j_beg, j_end, base, s_idx, u.att);
  } else {
    // the same thread stored these indices above: no barrier before the rewrite
    attn::rows_of_indices<kThreads>(aa, base, s_idx, span);
    lds_barrier();
    attn::attend_bf16(aa, r, split, splits, hg, j_beg, j_end, s_idx, qr, u.att);
  }
}


}  // namespace

bool topk_use_split(int R, int max_n) {
  return max_n > 4 * kTile && R <= device_cu_count() / 2;
}

// Tiles of kTile keys per slice: the fewest (a power of two up to
// kMaxSliceTiles) that keep the candidate launch to one workgroup per CU, so
// long rows do not queue several rounds of workgroups that each recompute
// the pivot.
static int split_tiles(int R, int max_n) {
  int T = 1;
  while (T < kMaxSliceTiles && int64_t(R) * ((max_n + kTile * T - 1) / (kTile * T)) > device_cu_count()) T *= 2;
  return T;
}

static int split_slices(int max_n, int T) { return (max_n + kTile * T - 1) / (kTile * T); }

static void launch_cand(const TopkArgs& a, int slices, hipStream_t stream) {
  const dim3 grid(unsigned(a.R) * unsigned(slices));
  switch (a.slice_tiles) {
    case 1: topk_cand_kernel<1><<<grid, kThreads, 0, stream>>>(a, slices); break;
    case 2: topk_cand_kernel<2><<<grid, kThreads, 0, stream>>>(a, slices); break;
    case 4: topk_cand_kernel<4><<<grid, kThreads, 0, stream>>>(a, slices); break;
    default: topk_cand_kernel<kMaxSliceTiles><<<grid, kThreads, 0, stream>>>(a, slices); break;
  }
}

// Split workspace: the candidate words [R][slices][T * kTile], then the
// slice records [R][slices] (uint4).
size_t topk_split_ws_bytes(int R, int max_n) {
  const int T = split_tiles(R, max_n);
  const size_t slices = size_t(split_slices(max_n, T));
  return size_t(R) * slices * T * kTile * sizeof(unsigned long long) + size_t(R) * slices * sizeof(uint4);
}

void topk_split_carve(void* ws, int R, int max_n, TopkArgs& a) {
  const int T = split_tiles(R, max_n);
  const size_t slices = size_t(split_slices(max_n, T));
  a.slice_tiles = T;
  a.cand = static_cast<unsigned long long*>(ws);
  a.state = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) +
                                        size_t(R) * slices * T * kTile * sizeof(unsigned long long));
}

hipError_t launch_topk_attn(const TopkArgs& ta, const AttnArgs& aa, const AttnPlan& plan, hipStream_t stream) {
  if (ta.R == 0) return hipSuccess;
  const int slices = split_slices(ta.max_n, ta.slice_tiles);  // <= kThreads for rows up to 2^23 keys
  launch_cand(ta, slices, stream);
  const dim3 grid(unsigned(aa.R) * unsigned(plan.splits) * unsigned(plan.head_groups));
  if (aa.latent_dtype == kFP8) topk_attn_kernel<kFP8><<<grid, kThreads, 0, stream>>>(ta, aa, slices, plan.splits, plan.keys_per_split);
  else topk_attn_kernel<kBF16><<<grid, kThreads, 0, stream>>>(ta, aa, slices, plan.splits, plan.keys_per_split);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_attn_combine(aa, plan, stream);
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t stream) {
  if (a.R == 0) return hipSuccess;
  if (a.state && a.cand && topk_use_split(a.R, a.max_n)) {
    const int slices = split_slices(a.max_n, a.slice_tiles);  // <= kThreads for rows up to 2^23 keys
    const int windows = (a.k + kWindow - 1) / kWindow;
    launch_cand(a, slices, stream);
    topk_window_kernel<<<dim3(unsigned(a.R) * unsigned(windows)), kThreads, 0, stream>>>(a, slices, windows);
    return hipGetLastError();
  }
  dim3 grid(unsigned(a.R));
  if (a.max_n <= 4 * kTile) topk_kernel<16><<<grid, kThreads, 0, stream>>>(a);
  else if (a.max_n <= 8 * kTile) topk_kernel<32><<<grid, kThreads, 0, stream>>>(a);
  else if (a.max_n <= 16 * kTile) topk_kernel<64><<<grid, kThreads, 0, stream>>>(a);
  else topk_kernel<0><<<grid, kThreads, 0, stream>>>(a);  // longer rows: streamed from L2
  return hipGetLastError();
}

}  // namespace dsa
