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
// Work split: one wave owns consecutive keys of one query and walks them in
// groups of 64 (4 MFMA column tiles of 16 keys); the launch gives each CU one
// 4-wave workgroup and spreads all keys over the CUs once (up to 64 queries:
// shares of the CUs in proportion to the rows' actual lengths). Key rows go from HBM straight into the wave's LDS stage buffers
// with 16-byte direct-to-LDS loads, all stages issued up front (after the
// small query loads) so that the whole working set is in flight at once;
// each group is multiplied as soon as its own loads have landed, while the
// later ones are still arriving, and a consumed stage is refilled with the
// group NS places ahead. The query's head tile(s) stay in registers as
// the A operand (heads on M), the B operand is read from LDS (key n =
// lane % 16, 8 consecutive dims per K-step). Epilogue per lane: ReLU,
// multiply by the head weight, sum over the lane's 16 heads; a 3-shuffle
// butterfly then leaves lane l with the full score of key s0 + l, so the 64
// scores go out as one coalesced 256-byte store. Every sum has a fixed order:
// the scores are bitwise reproducible.
#include <type_traits>

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

// max(x, 0) in one instruction (v_med3_f32 clamps to [0, +inf]).
__device__ __forceinline__ float relu(float x) {
  return __builtin_amdgcn_fmed3f(x, 0.f, __builtin_inff());
}

// Keys of a group sit in LDS as rows of DI elements, the 16-byte chunks of
// row k permuted (XOR) by k mod 8 or k mod 16 (by k mod CPR for shorter
// rows): the B-operand reads of 8 (16) consecutive keys at one chunk offset
// then fall on distinct banks.
template <int QK, int DI, bool WIDE = false>
struct KeyCfg {
  static constexpr int ESZ = QK == 0 ? 4 : (QK == 1 ? 2 : 1);  // bytes per key element
  static constexpr int ROW = DI * ESZ;                        // bytes per key row
  static constexpr int CPR = ROW / 16;                        // 16-byte chunks per row
  // WIDE: 4-bit permutation (conflict-free 16-lane reads; the prefill kernel,
  // bound by LDS); otherwise 3 bits, which keeps each 8-lane part of a direct
  // load inside one 128-byte line (the decode kernel, bound by HBM).
  static constexpr int SWZ = WIDE ? (CPR < 16 ? CPR - 1 : 15) : (CPR < 8 ? CPR - 1 : 7);
  static constexpr int GK = 64;                               // keys per group
  static constexpr int GBYTES = GK * ROW;
  static constexpr int LOADS = GBYTES / 1024;                 // 1 KiB direct loads per group
  static constexpr int GLOADS = LOADS + (QK == 2 ? 1 : 0);     // + the row scales (fp8)
  static constexpr int W = QK == 0 ? 4 : 8;                    // waves per workgroup (decode form)
  static constexpr int WBUDGET = 131072 / W;                    // stage bytes per wave
  static constexpr int NS = GBYTES >= WBUDGET ? 1 : (WBUDGET / GBYTES > 4 ? 4 : WBUDGET / GBYTES);  // stages
};

// One 16-byte direct-to-LDS load per lane: lane l's bytes land at LDS byte
// address lds + 16*l (lds wave-uniform). Issued from inline assembly so the
// compiler, which cannot tell which LDS bytes such a load writes, does not
// add a wait for every outstanding load before each LDS read; the kernel
// waits itself, per group, with exact vmcnt counts. M0 is saved and restored.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(lds)
      : "memory");
}

// 4-byte variant: lane l's word lands at LDS byte address lds + 4*l.
__device__ __forceinline__ void dma4(const void* src, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "global_load_lds_dword %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(lds)
      : "memory");
}

// 16-byte direct-to-LDS load through a buffer resource: lane l reads the
// 16 bytes at byte offset `off` of the buffer (zeros past its end) into LDS
// byte address lds + 16*l.
__device__ __forceinline__ void dma16_buf(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(off), "s"(r), "s"(lds)
      : "memory");
}

// 2-byte direct-to-LDS load through a buffer resource: lane l reads the
// 16-bit value at byte offset `off` (zero past the buffer's end) and writes
// it, zero-extended, to the 32-bit LDS word lds + 4*l.
__device__ __forceinline__ void dma2_buf(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "buffer_load_ushort %1, %2, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(off), "s"(r), "s"(lds)
      : "memory");
}

// Cache policy bits of a buffer store: sc1, device scope.
constexpr int kStoreThrough = 16;

// s_waitcnt vmcnt(min(N, 63)): a smaller count only waits longer.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N < 63 ? N : 63) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)p)));
}

// Cache row of key s of the sequence `base` names: base + s, or (paged) row
// s mod page of page table[base][s / page], the page id clamped into the pool.
__device__ __forceinline__ int64_t key_row(const IndexArgs& a, int64_t base, int64_t s) {
  if (!a.table) return base + s;
  int pg = a.table[base * a.max_pages + (s >> a.page_shift)];
  const int npages = int(a.cache_rows >> a.page_shift);
  pg = pg < 0 ? 0 : (pg >= npages ? npages - 1 : pg);
  return (int64_t(pg) << a.page_shift) + (s & ((int64_t(1) << a.page_shift) - 1));
}

// Start the direct-to-LDS load of keys s0 .. s0+63 (those below s_end) into
// stage buffer `dst`; fp8 keys: then their row scales (bf16 bits), key s0+l
// into the 32-bit word sc_dst + 4*l (zero past s_end). All earlier LDS reads
// of the wave are complete first (the buffers may be a stage that was just
// consumed). GLOADS loads in all.
template <int QK, int DI>
__device__ __forceinline__ void load_group(const IndexArgs& a, int64_t base, int64_t s0, int64_t s_end, char* dst,
                                           uint32_t* sc_dst, int lane, int tile_beg = 0, int tile_end = 4) {
  using C = KeyCfg<QK, DI>;
  const char* keys = static_cast<const char*>(a.keys);
  const uint32_t to = lds_addr(dst);
  // the group's 64 keys are consecutive cache rows (a page holds whole groups)
  const int64_t g0 = key_row(a, base, s0);
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  // loads [tile_beg, tile_end) * LOADS/4: the rows of those 16-key tiles
#pragma unroll
  for (int m = 0; m < C::LOADS; ++m) {
    if (m < tile_beg * (C::LOADS / 4) || m >= tile_end * (C::LOADS / 4)) continue;
    const int pch = 64 * m + lane;      // physical chunk index in the group
    const int row = pch / C::CPR;
    const int lc = (pch % C::CPR) ^ (row & C::SWZ);
    const int64_t key = s0 + row < s_end ? g0 + row : g0;  // rows past the range re-read the first
    dma16(keys + key * C::ROW + 16 * lc, to + 1024 * m);
  }
  if constexpr (QK == 2) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(a.k_scale + g0), 0, int(2 * (s_end - s0)), 0x00020000);
    dma2_buf(rs, uint32_t(2 * lane), lds_addr(sc_dst));
  }
}

// Wait until at most `ahead` key groups of direct loads are outstanding
// (0 <= ahead <= 4; every group is LOADS instructions).
template <int LOADS>
__device__ __forceinline__ void wait_groups(int ahead) {
  if (ahead >= 4) wait_vmcnt<4 * LOADS>();
  else if (ahead == 3) wait_vmcnt<3 * LOADS>();
  else if (ahead == 2) wait_vmcnt<2 * LOADS>();
  else if (ahead == 1) wait_vmcnt<LOADS>();
  else wait_vmcnt<0>();
}

// B operand of K-step ks for key row `row` of a stage: dims 32*ks + 8*grp .. +8.
template <int QK, int DI, bool WIDE = false>
__device__ __forceinline__ typename Frag<QK>::type key_frag(const char* stage, int row, int grp, int ks) {
  using C = KeyCfg<QK, DI, WIDE>;
  const char* rp = stage + row * C::ROW;
  const int sw = row & C::SWZ;
  typename Frag<QK>::type f;
  if constexpr (QK == 0) {
    const int c0 = 8 * ks + 2 * grp;
    const float4 x = *reinterpret_cast<const float4*>(rp + 16 * (c0 ^ sw));
    const float4 y = *reinterpret_cast<const float4*>(rp + 16 * ((c0 + 1) ^ sw));
    f = f32x8{{x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w}};
  } else if constexpr (QK == 1) {
    f = *reinterpret_cast<const bf16x8*>(rp + 16 * ((4 * ks + grp) ^ sw));
  } else {
    const uint2 c = *reinterpret_cast<const uint2*>(rp + 16 * ((2 * ks + (grp >> 1)) ^ sw) + 8 * (grp & 1));
    f = fp8x8_to_bf16(c);
  }
  return f;
}

// ReLU on the bit pattern: a float with the sign bit set is a negative int32,
// so an integer max with 0 sends it to +0.0 (one VALU op; the float min/max
// forms cost a NaN-quieting op on top).
__device__ __forceinline__ float relu_bits(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

// Lane 16*r + n holds p[t] = the part of 16-lane row r for key 16*t + n;
// returns, in lane 16*t + n, the sum over the 4 rows of p[t]. The 32-lane
// swap leaves rows {0+2, 1+3} sums of p[0], p[2] (and of p[1], p[3]) side by
// side; the 16-lane swap pairs those up. Three lane swaps on the VALU, no
// LDS round trip; the sum order is (r0 + r2) + (r1 + r3).
__device__ __forceinline__ float rows_transpose_sum(const float (&p)[4]) {
  const auto s02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[0]), __float_as_uint(p[2]), false, false);
  const auto s13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[1]), __float_as_uint(p[3]), false, false);
  const float x = __uint_as_float(s02[0]) + __uint_as_float(s02[1]);  // rows: p0 r0+r2, p0 r1+r3, p2 .., p2 ..
  const float y = __uint_as_float(s13[0]) + __uint_as_float(s13[1]);  // rows: p1 r0+r2, p1 r1+r3, p3 .., p3 ..
  const auto sxy = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return __uint_as_float(sxy[0]) + __uint_as_float(sxy[1]);
}

// s_waitcnt vmcnt(min(n, A)): at most n vector memory operations of this
// wave still outstanding (they complete in issue order).
template <int A>
__device__ __forceinline__ void wait_ops(int n) {
  if constexpr (A == 0) {
    wait_vmcnt<0>();
  } else {
    if (n >= A) wait_vmcnt<A>();
    else wait_ops<A - 1>(n);
  }
}

// Keys 0 .. n-1 of query r's sequence; base is the sequence's first cache
// row, or (paged caches) the sequence's index (see key_row).
__device__ __forceinline__ void query_range(const IndexArgs& a, int r, int64_t& base, int64_t& n) {
  int b = a.q_seq ? a.q_seq[r] : r / a.qps;
  b = b < 0 ? 0 : (b >= a.B ? a.B - 1 : b);
  const int qpos = a.q_pos ? a.q_pos[r] : a.seq_len[b] - a.qps + r % a.qps;
  n = qpos + 1 < a.max_n ? qpos + 1 : a.max_n;
  if (n < 0) n = 0;
  if (a.table) {
    base = b;
    const int64_t cap = int64_t(a.max_pages) << a.page_shift;
    if (n > cap) n = cap;
    return;
  }
  base = a.row_off[b];
  if (base < 0 || base >= a.cache_rows) n = 0;
  else if (n > a.cache_rows - base) n = a.cache_rows - base;
}


// Balanced form (R <= 64, a 1-D grid of G >= R workgroups): every wave works
// out the same split from all the rows' lengths (lane r: row r), with no
// barrier. Row r gets 1 + floor((G - R) * u_r / U) workgroups, u_r its
// length in units of 1024 keys (rounded up) and U their sum (32-bit integer
// arithmetic: the shares add up to at most G), consecutive in the grid, and
// its keys in equal multiples of 64 per wave; returns this workgroup's row,
// the row's base and length, the first key of the workgroup and the keys per
// wave (a workgroup past the shares gets n = 0).
__device__ __forceinline__ void balanced_split(const IndexArgs& a, int w, int G, int waves, int& r, int64_t& base,
                                               int64_t& n, int64_t& wg_beg, int64_t& kpw) {
  // a workgroup past every row's share keeps these: no key, nothing loaded
  r = 0;
  base = 0;
  n = 0;
  wg_beg = 0;
  kpw = 64;
  const int lane = threadIdx.x & 63;
  int64_t bl = 0, nl = 0;
  if (lane < a.R) query_range(a, lane, bl, nl);
  const uint32_t ul = uint32_t((nl + 1023) >> 10);  // < 2^22
  uint32_t tot = ul;                                // < 2^28
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) tot += __shfl_xor(tot, d, 64);
  uint32_t share = 0;
  if (lane < a.R) {
    // (G - R) * ul < 2^10 * 2^22: 32 bits
    share = 1u + (tot ? uint32_t(G - a.R) * ul / tot : 0u);
  }
  const uint32_t incl = wave_incl_scan(share);
  const unsigned long long hit = __ballot(lane < a.R && uint32_t(w) < incl && uint32_t(w) >= incl - share);
  if (hit == 0ull) return;
  r = __ffsll(static_cast<long long>(hit)) - 1;
  const uint32_t sh_r = __builtin_amdgcn_readlane(share, r);
  const uint32_t first = __builtin_amdgcn_readlane(incl, r) - sh_r;
  base = (int64_t(__builtin_amdgcn_readlane(uint32_t(uint64_t(bl) >> 32), r)) << 32) |
         __builtin_amdgcn_readlane(uint32_t(bl), r);
  const uint32_t n32 = __builtin_amdgcn_readlane(uint32_t(nl), r);
  n = n32;
  const uint32_t per = (n32 + sh_r * waves - 1) / (sh_r * waves);
  kpw = per < 64 ? 64 : int64_t((per + 63) / 64 * 64);
  wg_beg = int64_t(w - int(first)) * waves * kpw;
}

template <int QK, int MT, int DI>
__global__ __launch_bounds__((KeyCfg<QK, DI>::W * 64)) void index_scores_kernel(IndexArgs a, int keys_per_wave) {
  using C = KeyCfg<QK, DI>;
  constexpr int kWaves = C::W;
  constexpr int NKS = DI / 32;       // K-steps of 32 dims
  constexpr bool kQLds = QK != 0;    // bf16 query and weights staged through LDS
  constexpr int QCPR = DI / 8;       // 16-byte chunks per bf16 query row
  using F = typename Frag<QK>::type;
  __shared__ __attribute__((aligned(1024))) char smem[kWaves][C::NS][C::GBYTES];
  __shared__ __attribute__((aligned(16))) char s_q[kQLds ? 64 * DI * 2 : 16];
  __shared__ __attribute__((aligned(16))) float s_w[64];
  __shared__ __attribute__((aligned(16))) uint32_t s_sc[kWaves][C::NS][QK == 2 ? 64 : 1];  // fp8 row scales

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int col = lane & 15;  // MFMA column: key within a 16-key tile
  const int grp = lane >> 4;  // K-slot group / C-row group

  // keys_per_wave > 0: query blockIdx.x, chunk blockIdx.y of that many keys
  // per wave; 0: the balanced split over a 1-D grid
  int r;
  int64_t base, n, wg_beg, kpw64;
  if (keys_per_wave > 0) {
    r = blockIdx.x;
    query_range(a, r, base, n);
    kpw64 = keys_per_wave;
    wg_beg = int64_t(blockIdx.y) * kWaves * kpw64;
  } else {
    balanced_split(a, blockIdx.x, gridDim.x, kWaves, r, base, n, wg_beg, kpw64);
  }
  r = __builtin_amdgcn_readfirstlane(r);
  if (wg_beg >= n) return;  // the whole workgroup has no key
  const int keys_per_wave_r = int(kpw64);
  const int64_t s_beg = wg_beg + int64_t(wave) * keys_per_wave_r;
  const int64_t s_end = s_beg + keys_per_wave_r < n ? s_beg + keys_per_wave_r : n;
  const int groups = s_beg < s_end ? int((s_end - s_beg + 63) / 64) : 0;

  F qa[MT][NKS];
  float wr[MT][4];
  int issued = 0;
  // One bf16 group per wave (the usual decode batch: each wave's keys fit
  // one 64-key group): its four tiles go out two ahead, so the first tiles
  // land early in the stream and their MFMA work overlaps the later tiles'
  // transfer instead of all of it following the last load.
  const bool roll = QK == 1 && groups == 1;
  if constexpr (kQLds) {
    // Query rows (H_I x DI bf16, chunks of row h XOR-permuted by h mod 8) and
    // the H_I weights go to LDS by direct loads, shared by the 4 waves; the
    // rows and weights of padded heads are zeroed.
    const int qchunks = a.H_I * QCPR;
    const char* qsrc = static_cast<const char*>(a.q) + int64_t(r) * a.H_I * (DI * 2);
    const uint32_t qlds = lds_addr(s_q);
    for (int m = wave; 64 * m < qchunks; m += kWaves) {
      const int pch = 64 * m + lane;
      const int h = pch / QCPR;
      const int lc = (pch % QCPR) ^ (h & 7);
      const char* src = qsrc + int64_t(h) * (DI * 2) + 16 * lc;
      if (pch < qchunks) dma16(src, qlds + 1024 * m);
    }
    if (wave == 0 && lane < a.H_I) dma4(a.w + int64_t(r) * a.H_I + lane, lds_addr(s_w));
    for (int i = threadIdx.x + qchunks; i < 16 * MT * QCPR; i += kWaves * 64)
      *reinterpret_cast<uint4*>(s_q + 16 * i) = uint4{0u, 0u, 0u, 0u};
    if (threadIdx.x >= a.H_I && threadIdx.x < 16 * MT) s_w[threadIdx.x] = 0.f;
    // then all key stages, so the whole working set is in flight; a wave
    // with a single bf16 group starts with its first two 16-key tiles only
    // and issues each later one as a tile lands (see below)
    if (roll) {
      load_group<QK, DI>(a, base, s_beg, s_end, smem[wave][0], s_sc[wave][0], lane, 0, 2);
      issued = 1;
      wait_vmcnt<2 * (C::LOADS / 4)>();  // this wave's query and weight loads have landed
    } else {
      for (; issued < C::NS && issued < groups; ++issued)
        load_group<QK, DI>(a, base, s_beg + 64 * issued, s_end, smem[wave][issued], s_sc[wave][issued], lane);
      wait_groups<C::GLOADS>(issued);  // this wave's query and weight loads have landed
    }
    __syncthreads();
    // A operand: head 16*mt + col, dims 32*ks + 8*grp .. +8
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int h = 16 * mt + col;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        qa[mt][ks] = *reinterpret_cast<const bf16x8*>(s_q + h * (DI * 2) + 16 * ((4 * ks + grp) ^ (h & 7)));
      const float4 w4 = *reinterpret_cast<const float4*>(s_w + 16 * mt + 4 * grp);
      wr[mt][0] = w4.x;
      wr[mt][1] = w4.y;
      wr[mt][2] = w4.z;
      wr[mt][3] = w4.w;
    }
  } else {
    if (groups == 0) return;
    // fp32: query fragments and weights straight into registers
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
    for (; issued < C::NS && issued < groups; ++issued)
      load_group<QK, DI>(a, base, s_beg + 64 * issued, s_end, smem[wave][issued], s_sc[wave][issued], lane);
  }

  if constexpr (QK != 0) {
    // bf16 and fp8 keys: the score (and sample) stores are branch-free
    // buffer stores (lanes past this wave's range are dropped by the
    // bounds), one per group each, so the wait for a group can count them
    // exactly instead of also waiting for the stores issued after its loads.
    const bool smp = a.sample != nullptr;
    const int spg = smp ? 2 : 1;  // stores per group
    const __amdgpu_buffer_rsrc_t srow = __builtin_amdgcn_make_buffer_rsrc(
        a.scores + int64_t(r) * a.ld + s_beg, 0, int((s_end - s_beg) * 4), 0x00020000);
    const int64_t smp0 = s_beg >> 4;  // s_beg is a multiple of 64
    const int nsmp = smp && s_beg < s_end ? int((s_end - 1) / 16 - smp0 + 1) : 0;
    const __amdgpu_buffer_rsrc_t ssmp = __builtin_amdgcn_make_buffer_rsrc(
        smp ? a.sample + int64_t(r) * a.ld_sample + smp0 : a.scores, 0, nsmp * 4, 0x00020000);
    for (int g = 0; g < groups; ++g) {
      const int64_t s0 = s_beg + 64 * g;
      const char* stage = smem[wave][g % C::NS];
      // behind group g's loads: those of the later groups and the stores of
      // the groups computed since it was issued
      const int behind = C::GLOADS * (issued - 1 - g) + spg * (g < C::NS ? g : C::NS);
      float part[4];
      if (!roll) wait_ops<C::GLOADS * (C::NS - 1) + 2 * C::NS>(behind);  // group g landed
      // fp8: the row scale of the key in this lane's MFMA column for each
      // block, and of key s0 + lane (read before the stage is refilled)
      float scb[4] = {1.f, 1.f, 1.f, 1.f};
      uint32_t scl = 0u;
      if constexpr (QK == 2) {
        const uint32_t* scs = s_sc[wave][g % C::NS];
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) scb[blk] = bf16_bits_to_f32(scs[16 * blk + col]);
        scl = scs[lane];
      }
      // ReLU, head weight and the sum over the lane's heads of a tile's
      // products: this lane's part of one key's score. fp8 keys with a
      // negative row scale sc (NEG: some key of the group has one): relu(sc*z)
      // per head, the scale applied first; a non-negative scale is applied to
      // the summed score instead, and the factor here is 1, exact, so the
      // code has no branch to split the instruction stream the scheduler
      // interleaves. Without NEG the factor is left out.
      auto tile_epi = [&](const f32x4 (&c)[MT], float sc, auto neg) -> float {
        constexpr bool NEG = decltype(neg)::value;
        float p = 0.f;
        if constexpr (QK == 2 && NEG) {
          const float m = sc < 0.f ? sc : 1.f;
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) p += wr[mt][i] * relu_bits(m * c[mt][i]);
        } else {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) p += wr[mt][i] * relu_bits(c[mt][i]);
        }
        return p;
      };
      if (roll) {
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
          // tile blk+2 goes out; tile blk has landed once only the tiles
          // issued after it are outstanding (no store has been issued yet)
          constexpr int LPT = C::LOADS / 4;
          if (blk + 2 < 4) load_group<QK, DI>(a, base, s_beg, s_end, smem[wave][0], s_sc[wave][0], lane, blk + 2, blk + 3);
          if (blk <= 1) wait_vmcnt<2 * LPT>();
          else if (blk == 2) wait_vmcnt<LPT>();
          else wait_vmcnt<0>();
          f32x4 acc[MT];
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) {
            const F kb = key_frag<QK, DI>(stage, 16 * blk + col, grp, ks);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[mt] = mfma_k32(qa[mt][ks], kb, ks ? acc[mt] : f32x4{0.f, 0.f, 0.f, 0.f});
          }
          part[blk] = tile_epi(acc, scb[blk], std::integral_constant<bool, QK == 2>{});
        }
      } else {
        // the whole group has landed: tile blk is multiplied from kb[blk&1]
        // into acc[blk&1] while tile blk-1's epilogue runs from the other
        // accumulators and tile blk+1's fragments are read into the other
        // fragment registers, and the scheduler is told to interleave the
        // three, so the epilogue and the fp8 widening run under the matrix
        // core's work instead of after it (the same products in the same
        // order)
        auto tiles = [&](auto neg) {
          F kb[2][NKS];
          f32x4 acc[2][MT];
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) kb[0][ks] = key_frag<QK, DI>(stage, col, grp, ks);
#pragma unroll
          for (int blk = 0; blk < 4; ++blk) {
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
              for (int mt = 0; mt < MT; ++mt)
                acc[blk & 1][mt] = mfma_k32(qa[mt][ks], kb[blk & 1][ks], ks ? acc[blk & 1][mt] : f32x4{0.f, 0.f, 0.f, 0.f});
            if (blk > 0) part[blk - 1] = tile_epi(acc[(blk - 1) & 1], scb[blk - 1], neg);
            if (blk + 1 < 4) {
#pragma unroll
              for (int ks = 0; ks < NKS; ++ks) kb[(blk + 1) & 1][ks] = key_frag<QK, DI>(stage, 16 * (blk + 1) + col, grp, ks);
            }
            // the next tile's fragment reads first, then each MFMA followed
            // by VALU work: the previous tile's epilogue (and, fp8, the
            // widening of the fragments just read)
            __builtin_amdgcn_sched_group_barrier(0x100, NKS, 0);
#pragma unroll
            for (int i = 0; i < MT * NKS; ++i) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
              __builtin_amdgcn_sched_group_barrier(0x002, QK == 2 ? 4 : 2, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x002, 32, 0);
            // the epilogue's result is defined here, so that it is not sunk
            // to the score store after the last tile
            if (blk > 0) asm volatile("" : "+v"(part[blk - 1]));
            __builtin_amdgcn_sched_barrier(0);
          }
          part[3] = tile_epi(acc[1], scb[3], neg);
        };
        // a negative row scale among the group's keys is rare: the group runs
        // the form without the per-head factor otherwise (same bits)
        bool neg = false;
        if constexpr (QK == 2) neg = __ballot(bf16_bits_to_f32(scl) < 0.f) != 0ull;
        if (neg) tiles(std::integral_constant<bool, true>{});
        else tiles(std::integral_constant<bool, false>{});
      }
      // this stage is consumed: refill it with group g + NS
      if (issued < groups) {
        load_group<QK, DI>(a, base, s_beg + 64 * issued, s_end, smem[wave][g % C::NS], s_sc[wave][g % C::NS], lane);
        ++issued;
      }
      float v = rows_transpose_sum(part);
      if constexpr (QK == 2) {
        // non-negative row scale: relu(sc*z) = sc*relu(z), applied once per key
        const float sc = bf16_bits_to_f32(scl);
        if (!(sc < 0.f)) v *= sc;
      }
      const int64_t s = s0 + lane;
      // at device scope (cache policy sc1): through the L2, so that the
      // kernel's end has none of these lines to write back before the
      // selection launch can start (0.4-0.9 us a step at 4 x 32K)
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), srow, int(s - s_beg) * 4, 0, kStoreThrough);
      if (smp)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), ssmp,
                                              (s & 15) ? -16 : int((s >> 4) - smp0) * 4, 0, kStoreThrough);
    }
    return;
  }

  float* out = a.scores + int64_t(r) * a.ld;
  for (int g = 0; g < groups; ++g) {
    const int64_t s0 = s_beg + 64 * g;
    const char* stage = smem[wave][g % C::NS];
    wait_groups<C::LOADS>(issued - 1 - g);  // group g has landed
    float part[4];
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
      f32x4 acc[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const F kb = key_frag<QK, DI>(stage, 16 * blk + col, grp, ks);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt] = mfma_k32(qa[mt][ks], kb, acc[mt]);
      }
      float sc = 1.f;
      if constexpr (QK == 2) {
        const int64_t s = s0 + 16 * blk + col;
        sc = s < s_end ? bf16_bits_to_f32(a.k_scale[key_row(a, base, s)]) : 1.f;
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
    // this stage is consumed: refill it with group g + NS
    if (issued < groups) {
      load_group<QK, DI>(a, base, s_beg + 64 * issued, s_end, smem[wave][g % C::NS], s_sc[wave][g % C::NS], lane);
      ++issued;
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
        const float sc = bf16_bits_to_f32(a.k_scale[key_row(a, base, s)]);
        if (!(sc < 0.f)) v *= sc;
      }
      out[s] = v;
      if (a.sample && (s & 15) == 0) a.sample[int64_t(r) * a.ld_sample + (s >> 4)] = v;
    }
  }
}

// ---- prefill: many queries of one sequence ----------------------------------------
// A workgroup of kPfWaves waves (two per SIMD) takes kPfWaves consecutive
// query rows of one sequence, one row per wave; the waves share a ring of
// kPfStages key groups in LDS, which they fill together with direct loads,
// one group per barrier. A key row read from L2 feeds kPfWaves queries x H_I
// heads of MFMA work (the decode kernel feeds one). Within a group each wave
// works tile by tile (16 keys): while the matrix core multiplies tile b, the
// wave runs tile b-1's epilogue (ReLU, head weights, head sum) on the VALU
// and then refills tile b-1's fragment registers with the next group's keys,
// so neither the epilogue nor the LDS reads leave the matrix core idle; the
// scheduler is told to interleave the streams. Workgroups run from the last
// rows (longest key ranges) to the first, so the short ones fill the tail.
// bf16 query and keys.
constexpr int kPfWaves = 8;
constexpr int kPfRows = kPfWaves;
constexpr int kPfKeys = 128;  // keys per group (one barrier each)
constexpr int kPfTiles = kPfKeys / 16;
// fp8 keys in the multi-token form: groups of 256 keys, so that each wave
// has as many tiles per barrier as a bf16 group gives it (the ring takes the
// same bytes, and two of its stages take the staged queries)
template <int QK, bool SLICED>
constexpr int pf_keys() {
  return QK == 2 && SLICED ? 2 * kPfKeys : kPfKeys;
}
constexpr int kPfStages = 4;


// s_waitcnt vmcnt(A * LPW) for the largest A <= ahead (A <= 8).
template <int LPW, int A = 8>
__device__ __forceinline__ void wait_ahead(int ahead) {
  if constexpr (A == 0) {
    wait_vmcnt<0>();
  } else {
    if (ahead >= A) wait_vmcnt<A * LPW>();
    else wait_ahead<LPW, A - 1>(ahead);
  }
}



// Length-balanced slices of the multi-token decode form (B <= 64 sequences,
// a 1-D grid of G >= B workgroups): every wave works out the same shares
// from all the sequences' lengths (lane b: sequence b, its first cache row
// loaded in the same round trip), with no barrier. Sequence b gets
// 1 + floor((G - B) u_b / U) workgroups, u_b its groups of PK keys (up to its
// last token's key count) and U their sum, consecutive in the grid, each
// taking an equal run of its groups; returns this workgroup's sequence, its
// first cache row and length, and its key range (empty past every share).
// A grid cut by the longest sequence alone left the CUs of the shorter
// sequences' missing slices idle.
template <int PK>
__device__ __forceinline__ void balanced_slice(const IndexArgs& a, int w, int G, int& b, int64_t& base,
                                               int64_t& slen, int64_t& k_beg, int64_t& k_lim) {
  b = 0;
  base = 0;
  slen = 0;
  k_beg = 0;
  k_lim = 0;
  const int lane = threadIdx.x & 63;
  int64_t bl = 0;
  int32_t sl = 0;
  if (lane < a.B) {
    bl = a.row_off[lane];
    sl = a.seq_len[lane];
  }
  const int64_t nl = sl <= 0 ? 0 : (sl < a.max_n ? sl : a.max_n);
  const uint32_t ul = uint32_t((nl + PK - 1) / PK);  // <= 2^15 groups
  uint32_t tot = ul;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) tot += __shfl_xor(tot, d, 64);
  uint32_t share = 0;
  if (lane < a.B) share = 1u + (tot ? uint32_t(G - a.B) * ul / tot : 0u);  // (G - B) ul < 2^23
  const uint32_t incl = wave_incl_scan(share);
  const unsigned long long hit = __ballot(lane < a.B && uint32_t(w) < incl && uint32_t(w) >= incl - share);
  if (hit == 0ull) return;
  b = __ffsll(static_cast<long long>(hit)) - 1;
  const uint32_t sh_b = __builtin_amdgcn_readlane(share, b);
  const uint32_t first = __builtin_amdgcn_readlane(incl, b) - sh_b;
  const uint32_t gpw = (__builtin_amdgcn_readlane(ul, b) + sh_b - 1) / sh_b;
  base = (int64_t(__builtin_amdgcn_readlane(uint32_t(uint64_t(bl) >> 32), b)) << 32) |
         __builtin_amdgcn_readlane(uint32_t(bl), b);
  slen = int32_t(__builtin_amdgcn_readlane(uint32_t(sl), b));
  k_beg = int64_t(w - int(first)) * gpw * PK;
  k_lim = k_beg + int64_t(gpw) * PK;
}

// kPfWaves waves share a ring of key groups; QW query rows of one sequence
// per workgroup, each row's tiles split over kPfWaves / QW waves (QW = 8:
// one wave per row, all the tiles of a group; QW = 4: two waves per row,
// half the tiles each).
// SLICED false (prefill form: B = 1, q_pos given, QW = 8): workgroup
// blockIdx.x takes rows 8*blk .. +7, counted from the last, and keys 0 ..
// the end of its longest row.
// SLICED true (decode form with qps <= QW new tokens per sequence):
// workgroup (blockIdx.x, blockIdx.y) takes the qps rows of sequence
// blockIdx.y and its keys kps*blockIdx.x .. +kps-1 (kps = 0: the 1-D
// length-balanced grid, balanced_slice), so each key row is read once for
// all of them; rows past qps are idle. With QW = 4 the query rows
// and head weights go to LDS once per workgroup (through ring stages 2-3,
// while key groups 0-1 load) instead of every wave loading its row.
// Scores (and the score sample, when asked) are stored up to each row's end.
template <int QK, int MT, int DI, int QW, bool SLICED>
__global__ __launch_bounds__(kPfWaves * 64) void index_scores_prefill_kernel(IndexArgs a, int kps) {
  using C = KeyCfg<QK, DI, true>;
  using F = typename Frag<QK>::type;
  static_assert(QK == 1 || (QK == 2 && SLICED), "fp8 keys: the multi-token decode form only");
  constexpr int RW = kPfWaves;
  constexpr int NKS = DI / 32;
  constexpr int PK = pf_keys<QK, SLICED>();  // keys per group
  constexpr int GB = PK * C::ROW;           // bytes per group
  constexpr int KL = GB / 1024 / RW;        // key loads per wave per group
  constexpr int LPW = KL + (QK == 2 ? 1 : 0);  // + fp8: the row scales of PK/8 keys
  constexpr int TPW = PK / 16 * QW / RW;    // tiles per wave per group
  constexpr bool QLDS = SLICED && QW == 4;  // query rows staged in LDS
  constexpr int QCPR = DI / 8;              // 16-byte chunks per query row
  constexpr int QB = 16 * MT * DI * 2;      // staged bytes per query (heads padded to 16*MT)
  static_assert((GB / 1024) % RW == 0, "group loads split evenly over the waves");
  static_assert(kPfStages >= 3, "a group lands while the one before it is multiplied");
  static_assert(TPW % 4 == 0, "a wave's tiles of a group form whole 64-key score stores");
  constexpr bool QRING = QK == 1 || PK > kPfKeys;  // queries staged through ring stages 2-3
  static_assert(!QLDS || !QRING || QW * QB <= 2 * GB, "the staged bf16 queries fit two ring stages");
  __shared__ __attribute__((aligned(1024))) char ring[kPfStages][GB];
  __shared__ __attribute__((aligned(16))) float s_w[QLDS ? QW : 1][64];
  // fp8: row scales (bf16 bits, zero-extended words); wave w's dma2 fills
  // words 64w .. 64w+63, the first PK/8 for keys (PK/8)w .. (PK/8)(w+1)-1
  // of the group
  __shared__ __attribute__((aligned(16))) uint32_t s_ksc[QK == 2 ? kPfStages : 1][QK == 2 ? RW * 64 : 1];
  // stages too small to stage the queries in: a buffer of their own
  __shared__ __attribute__((aligned(1024))) char s_qst[QLDS && !QRING ? QW * QB : 16];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int qrow = wave % QW;                  // this wave's query row in the workgroup
  const int tb = (wave / QW) * TPW;            // its first tile of each group

  int r0, nrows, b;
  int64_t k_beg, k_lim, base, slen = 0;
  if constexpr (!SLICED) {
    const int blk = int(gridDim.x) - 1 - int(blockIdx.x);
    r0 = blk * QW;
    nrows = a.R - r0 < QW ? a.R - r0 : QW;
    b = 0;
    k_beg = 0;
    k_lim = a.max_n;
    base = a.row_off[0];
  } else {
    if (kps > 0) {
      b = blockIdx.y;
      k_beg = int64_t(blockIdx.x) * kps;
      k_lim = k_beg + kps;
      base = a.row_off[b];
      slen = a.seq_len[b];
    } else {
      balanced_slice<PK>(a, int(blockIdx.x), int(gridDim.x), b, base, slen, k_beg, k_lim);
    }
    r0 = b * a.qps;
    nrows = a.qps < QW ? a.qps : QW;
  }
  const bool base_ok = base >= 0 && base < a.cache_rows;
  auto row_n = [&](int i) -> int64_t {
    const int rr = r0 + i;
    int64_t n = (a.q_pos ? int64_t(a.q_pos[rr]) : slen - a.qps + i) + 1;
    if (n > a.max_n) n = a.max_n;
    if (n > a.cache_rows - base) n = a.cache_rows - base;
    return base_ok && n > 0 ? n : 0;
  };
  const int rr = r0 + qrow;
  const bool rv = qrow < nrows;
  const int64_t n_w = rv ? row_n(qrow) : 0;
  int64_t n_wg = 0;
  for (int i = 0; i < nrows; ++i) {
    const int64_t ni = row_n(i);
    n_wg = ni > n_wg ? ni : n_wg;
  }
  const int64_t k_end = n_wg < k_lim ? n_wg : k_lim;
  const int groups = k_end > k_beg ? int((k_end - k_beg + PK - 1) / PK) : 0;
  if (groups == 0) return;  // the same for every wave of the workgroup

  // Group g is the buffer of key rows k_beg + PK*g .. k_end-1 (rows past
  // the range read as zeros); this lane's byte offset in it for each of the
  // wave's loads is the same in every group.
  const char* keys = static_cast<const char*>(a.keys) + (base + k_beg) * C::ROW;
  const int64_t span = k_end - k_beg;
  uint32_t src_off[LPW];
#pragma unroll
  for (int j = 0; j < KL; ++j) {
    const int m = wave * KL + j;
    const int pch = 64 * m + lane;
    const int row = pch / C::CPR;
    const int lc = (pch % C::CPR) ^ (row & C::SWZ);
    src_off[j] = uint32_t(row * C::ROW + 16 * lc);
  }
  auto issue = [&](int g) {
    const uint32_t to = lds_addr(ring[g % kPfStages]);
    const int64_t s0 = int64_t(g) * PK;
    const __amdgpu_buffer_rsrc_t src = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(keys + s0 * C::ROW), 0, int((span - s0) * C::ROW), 0x00020000);
#pragma unroll
    for (int j = 0; j < KL; ++j) dma16_buf(src, src_off[j], to + 1024 * (wave * KL + j));
    if constexpr (QK == 2) {
      // scales of keys s0 + (PK/8)*wave .. +PK/8-1 (zero past the range)
      constexpr int SPW = PK / 8;
      const int64_t first = s0 + SPW * wave;
      const int64_t cnt = span - first < SPW ? (span - first > 0 ? span - first : 0) : SPW;
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(a.k_scale + base + k_beg + (cnt > 0 ? first : 0)), 0, int(2 * cnt), 0x00020000);
      dma2_buf(rs, uint32_t(2 * lane), lds_addr(&s_ksc[g % kPfStages][64 * wave]));
    }
  };

  bf16x8 qa[MT][NKS];
  float wr[MT][4];
  int issued = 0;
  if constexpr (QLDS) {
    // query rows (chunks of head h XOR-permuted by h mod 8; heads past H_I
    // and idle rows zeroed) and head weights into LDS, ahead of key groups
    // 0-1; once every wave's part has landed the fragments go to registers
    // and stages 2-3 take key groups 2-3
    char* qst = QRING ? ring[2] : s_qst;
    const uint32_t qlds = lds_addr(qst);
    for (int m = wave; 64 * m < QW * 16 * MT * QCPR; m += RW) {
      const int pch = 64 * m + lane;
      const int q = pch / (16 * MT * QCPR);
      const int h = (pch / QCPR) % (16 * MT);
      const int lc = (pch % QCPR) ^ (h & 7);
      if (q < nrows && h < a.H_I)
        dma16(static_cast<const char*>(a.q) + (int64_t(r0 + q) * a.H_I + h) * (DI * 2) + 16 * lc, qlds + 1024 * m);
      else
        *reinterpret_cast<uint4*>(qst + 16 * pch) = uint4{0u, 0u, 0u, 0u};
    }
    if (wave < QW) {
      if (wave < nrows && lane < a.H_I) dma4(a.w + int64_t(r0 + wave) * a.H_I + lane, lds_addr(s_w[wave]));
      else s_w[wave][lane] = 0.f;
    }
    for (; issued < 2 && issued < groups; ++issued) issue(issued);
    wait_ops<2 * LPW>(LPW * issued);  // this wave's query and weight loads have landed
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int h = 16 * mt + col;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        qa[mt][ks] = *reinterpret_cast<const bf16x8*>(qst + qrow * QB + h * (DI * 2) + 16 * ((4 * ks + grp) ^ (h & 7)));
      const float4 w4 = *reinterpret_cast<const float4*>(&s_w[qrow][16 * mt + 4 * grp]);
      wr[mt][0] = w4.x;
      wr[mt][1] = w4.y;
      wr[mt][2] = w4.z;
      wr[mt][3] = w4.w;
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // stages 2-3 are free
    for (; issued < kPfStages && issued < groups; ++issued) issue(issued);
  } else {
    for (; issued < kPfStages && issued < groups; ++issued) issue(issued);
    // query fragments and weights of this wave's row (zero for padded heads
    // or a missing row), loaded behind the first key groups and waited for
    // with them, then re-defined through an empty asm, so that no later use
    // waits on them behind the key loads
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int h = 16 * mt + col;
      const bool hv = rv && h < a.H_I;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int64_t off = (int64_t(hv ? rr : 0) * a.H_I + (hv ? h : 0)) * DI + 32 * ks + 8 * grp;
        const uint4 x = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.q) + off);
        qa[mt][ks] = __builtin_bit_cast(bf16x8, hv ? x : uint4{0u, 0u, 0u, 0u});
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int hw = 16 * mt + 4 * grp + i;
        const bool wv = rv && hw < a.H_I;
        const float x = a.w[int64_t(wv ? rr : 0) * a.H_I + (wv ? hw : 0)];
        wr[mt][i] = wv ? x : 0.f;
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      uint4 u = __builtin_bit_cast(uint4, qa[mt][ks]);
      asm volatile("" : "+v"(u.x), "+v"(u.y), "+v"(u.z), "+v"(u.w));
      qa[mt][ks] = __builtin_bit_cast(bf16x8, u);
    }
    asm volatile("" : "+v"(wr[mt][0]), "+v"(wr[mt][1]), "+v"(wr[mt][2]), "+v"(wr[mt][3]));
  }

  // fragments of tile t (keys 16*t .. +16) of group g (a stage past the last
  // group holds stale keys: reading it is harmless, its products are never
  // stored)
  auto tile_frags = [&](int g, int t, F (&kt)[NKS]) {
    const char* stage = ring[g % kPfStages];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) kt[ks] = key_frag<QK, DI, true>(stage, 16 * t + col, grp, ks);
  };
  // fp8: row scale of key j of group g's stage
  auto key_scale = [&](int g, int j) -> float {
    return bf16_bits_to_f32(s_ksc[g % kPfStages][64 * (j / (PK / 8)) + (j % (PK / 8))]);
  };
  // ReLU, head weight and the sum over the lane's 4 heads of each of the MT
  // head tiles: this lane's part of the score of key 16*t + n (fp8 with a
  // negative row scale sc: relu(sc * dot) per head; a non-negative scale is
  // applied to the summed score)
  // (NEG: some key of the wave's tiles of the group has a negative scale;
  // the factor is then taken branch-free, 1 (exact) for the others, so no
  // branch splits the instruction stream the scheduler interleaves)
  auto tile_epi = [&](const f32x4 (&c)[MT], float sc, auto neg) -> float {
    constexpr bool NEG = decltype(neg)::value;
    float pm[MT];
    if constexpr (QK == 2 && NEG) {
      const float m = sc < 0.f ? sc : 1.f;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        pm[mt] = wr[mt][0] * relu_bits(m * c[mt][0]);
#pragma unroll
        for (int i = 1; i < 4; ++i) pm[mt] += wr[mt][i] * relu_bits(m * c[mt][i]);
      }
    } else {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        pm[mt] = wr[mt][0] * relu_bits(c[mt][0]);
#pragma unroll
        for (int i = 1; i < 4; ++i) pm[mt] += wr[mt][i] * relu_bits(c[mt][i]);
      }
    }
    float pp = pm[0];
#pragma unroll
    for (int mt = 1; mt < MT; ++mt) pp += pm[mt];
    return pp;
  };

  // this wave's score row from key k_beg, as a buffer that ends at the row's
  // end: stores past it are dropped; likewise its score sample (every 16th
  // key; k_beg is a multiple of PK)
  const int64_t own = n_w > k_beg ? n_w - k_beg : 0;
  const __amdgpu_buffer_rsrc_t srow = __builtin_amdgcn_make_buffer_rsrc(
      a.scores + int64_t(rv ? rr : 0) * a.ld + k_beg, 0, int(own * 4), 0x00020000);
  const bool smp = SLICED && a.sample != nullptr;
  const int spg = smp ? 2 * (TPW / 4) : TPW / 4;  // stores per group
  const __amdgpu_buffer_rsrc_t ssmp = __builtin_amdgcn_make_buffer_rsrc(
      smp ? a.sample + int64_t(rv ? rr : 0) * a.ld_sample + (k_beg >> 4) : a.scores, 0,
      smp ? int((own + 15) / 16 * 4) : 0, 0x00020000);

  // two fragment tiles and two accumulator tiles: tile t is multiplied from
  // kb[t&1] into acc[t&1] while tile t-1's epilogue runs from acc[(t-1)&1]
  // and tile t+1's fragments are read into kb[(t+1)&1]
  F kb[2][NKS];
  f32x4 acc[2][MT];
  // group 0 has landed for every wave (behind it: the later groups' loads)
  wait_ops<LPW * (kPfStages - 1)>(LPW * (issued - 1));
  asm volatile("s_barrier" ::: "memory");
  tile_frags(0, tb, kb[0]);

  for (int g = 0; g < groups; ++g) {
    // own parts of group g+1 landed (its first tile is read during this
    // group's last one): behind them are the direct loads of the later
    // groups and spg score stores per group since
    if (g + 1 < groups) wait_ops<LPW * (kPfStages - 2) + PK / 32 * (kPfStages - 1)>(
        LPW * (issued - (g + 2)) + spg * (g < kPfStages - 2 ? g : kPfStages - 2));
    // every part of g+1 has landed; every wave is done with group g-1, so
    // its stage takes group g-1 + kPfStages
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (g >= 1 && issued < groups) {
      issue(issued);
      ++issued;
    }
    float part[TPW];
    auto run_tiles = [&](auto neg) {
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            acc[t & 1][mt] =
                mfma_k32(qa[mt][ks], kb[t & 1][ks], ks ? acc[t & 1][mt] : f32x4{0.f, 0.f, 0.f, 0.f});
        if (t > 0) part[t - 1] = tile_epi(acc[(t - 1) & 1], QK == 2 ? key_scale(g, 16 * (tb + t - 1) + col) : 1.f, neg);
        if (t + 1 < TPW) tile_frags(g, tb + t + 1, kb[(t + 1) & 1]);
        else tile_frags(g + 1, tb, kb[(t + 1) & 1]);
        // the next tile's fragment reads first, then each MFMA followed by
        // VALU work of the previous tile's epilogue
        __builtin_amdgcn_sched_group_barrier(0x100, NKS, 0);
#pragma unroll
        for (int i = 0; i < MT * NKS; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      part[TPW - 1] = tile_epi(acc[(TPW - 1) & 1], QK == 2 ? key_scale(g, 16 * (tb + TPW - 1) + col) : 1.f, neg);
    };
    // a negative row scale among the keys of this wave's tiles is rare: the
    // group runs the form without the per-head factor otherwise (same bits)
    bool neg = false;
    if constexpr (QK == 2) {
      bool any = false;
#pragma unroll
      for (int u = 0; u < TPW / 4; ++u) any |= key_scale(g, 16 * tb + 64 * u + lane) < 0.f;
      neg = __ballot(any) != 0ull;
    }
    if (neg) run_tiles(std::integral_constant<bool, true>{});
    else run_tiles(std::integral_constant<bool, false>{});
#pragma unroll
    for (int h = 0; h < TPW / 4; ++h) {
      const float p4[4] = {part[4 * h], part[4 * h + 1], part[4 * h + 2], part[4 * h + 3]};
      float v = rows_transpose_sum(p4);
      if constexpr (QK == 2) {
        const float sc = key_scale(g, 16 * tb + 64 * h + lane);
        if (!(sc < 0.f)) v *= sc;
      }
      // non-temporal: the scores are read by the next kernel, not this one
      const int key = g * PK + 16 * tb + 64 * h + lane;
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), srow, key * 4, 0, 2);
      if constexpr (SLICED) {
        if (smp) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), ssmp, (key & 15) ? -16 : (key >> 4) * 4, 0, 2);
      }
    }
  }
}

template <int MT, int DI>
hipError_t launch_prefill(const IndexArgs& a, hipStream_t stream) {
  const unsigned blocks = unsigned((a.R + kPfRows - 1) / kPfRows);
  index_scores_prefill_kernel<1, MT, DI, kPfRows, false><<<dim3(blocks), kPfWaves * 64, 0, stream>>>(a, 0);
  return hipGetLastError();
}

// Decode form with 2..8 new tokens per sequence. Up to 64 sequences: one
// workgroup per CU, the CUs shared out by the sequences' lengths
// (balanced_slice). More: a workgroup per (key slice, sequence), the slices
// sized so that the grid covers the CUs about once.
template <int QK, int MT, int DI>
hipError_t launch_multi_token(const IndexArgs& a, hipStream_t stream) {
  const int cus = device_cu_count();
  if (a.B <= 64 && a.B <= cus) {
    // one workgroup per CU, shared out by the sequences' lengths (read on
    // the device)
    if (a.qps <= 4) index_scores_prefill_kernel<QK, MT, DI, 4, true><<<dim3(unsigned(cus)), kPfWaves * 64, 0, stream>>>(a, 0);
    else index_scores_prefill_kernel<QK, MT, DI, 8, true><<<dim3(unsigned(cus)), kPfWaves * 64, 0, stream>>>(a, 0);
    return hipGetLastError();
  }
  const int per_seq = (cus + a.B - 1) / a.B;
  int64_t kps = (int64_t(a.max_n) + per_seq - 1) / per_seq;
  constexpr int PK = pf_keys<QK, true>();
  kps = (kps + PK - 1) / PK * PK;
  const unsigned slices = unsigned((a.max_n + kps - 1) / kps);
  const dim3 grid(slices, unsigned(a.B));
  if (a.qps <= 4) index_scores_prefill_kernel<QK, MT, DI, 4, true><<<grid, kPfWaves * 64, 0, stream>>>(a, int(kps));
  else index_scores_prefill_kernel<QK, MT, DI, 8, true><<<grid, kPfWaves * 64, 0, stream>>>(a, int(kps));
  return hipGetLastError();
}

template <int QK>
hipError_t launch_multi_token_m(const IndexArgs& a, hipStream_t stream) {
  if (a.H_I <= 16) return a.D_I == 64 ? launch_multi_token<QK, 1, 64>(a, stream) : launch_multi_token<QK, 1, 128>(a, stream);
  if (a.H_I <= 32) return a.D_I == 64 ? launch_multi_token<QK, 2, 64>(a, stream) : launch_multi_token<QK, 2, 128>(a, stream);
  return a.D_I == 64 ? launch_multi_token<QK, 4, 64>(a, stream) : launch_multi_token<QK, 4, 128>(a, stream);
}

template <int QK, int MT, int DI>
hipError_t launch_t(const IndexArgs& a, hipStream_t stream) {
  constexpr int kWaves = KeyCfg<QK, DI>::W;
  // One 4-wave workgroup per CU (the stage buffers take most of the LDS).
  // Up to 64 queries: the balanced split, which shares the CUs out by the
  // rows' actual lengths (read on the device), so rows shorter than max_n
  // leave no CU idle.
  if (a.R <= 64) {
    index_scores_kernel<QK, MT, DI><<<dim3(unsigned(device_cu_count())), kWaves * 64, 0, stream>>>(a, 0);
    return hipGetLastError();
  }
  // Otherwise keys per wave: a multiple of 64 that spreads all keys over the
  // CUs once, and a grid of (query, chunk).
  const int64_t total = int64_t(a.R) * a.max_n;
  const int64_t waves = int64_t(device_cu_count()) * kWaves;
  int64_t kpw = (total + waves - 1) / waves;
  const int64_t quarter = (int64_t(a.max_n) + kWaves - 1) / kWaves;  // keep all 4 waves of a row busy
  if (kpw > quarter) kpw = quarter;
  kpw = ((kpw + 63) / 64) * 64;
  if (kpw < 64) kpw = 64;
  if (kpw > (int64_t(1) << 20)) kpw = int64_t(1) << 20;
  const int64_t per_wg = int64_t(kWaves) * kpw;
  const unsigned chunks = unsigned((a.max_n + per_wg - 1) / per_wg);
  dim3 grid(unsigned(a.R), chunks);
  index_scores_kernel<QK, MT, DI><<<grid, kWaves * 64, 0, stream>>>(a, int(kpw));
  return hipGetLastError();
}

template <int QK, int MT>
hipError_t launch_d(const IndexArgs& a, hipStream_t stream) {
  return a.D_I == 64 ? launch_t<QK, MT, 64>(a, stream) : launch_t<QK, MT, 128>(a, stream);
}

template <int QK>
hipError_t launch_m(const IndexArgs& a, hipStream_t stream) {
  if (a.H_I <= 16) return launch_d<QK, 1>(a, stream);
  if (a.H_I <= 32) return launch_d<QK, 2>(a, stream);
  return launch_d<QK, 4>(a, stream);
}

}  // namespace

hipError_t launch_index_scores(const IndexArgs& a, hipStream_t stream) {
  if (a.R == 0) return hipSuccess;
  const int mode = a.q_dtype == kF32 ? 0 : (a.k_dtype == kFP8 ? 2 : 1);
  // many bf16 queries of one sequence (causal prefill form): key tiles shared by 8 queries
  // (key and score rows are addressed with 32-bit byte offsets there)
  // several new tokens per sequence (decode form, bf16 or fp8 keys): each key row read once for all of them
  if ((mode == 1 || mode == 2) && !a.q_seq && !a.q_pos && !a.table && a.qps >= 2 && a.qps <= kPfWaves &&
      a.max_n <= (int64_t(1) << 22))
    return mode == 1 ? launch_multi_token_m<1>(a, stream) : launch_multi_token_m<2>(a, stream);
  if (mode == 1 && a.B == 1 && a.q_pos && !a.table && a.R >= 4 * kPfRows && a.max_n <= (int64_t(1) << 22) &&
      !a.sample) {
    if (a.H_I <= 16) return a.D_I == 64 ? launch_prefill<1, 64>(a, stream) : launch_prefill<1, 128>(a, stream);
    if (a.H_I <= 32) return a.D_I == 64 ? launch_prefill<2, 64>(a, stream) : launch_prefill<2, 128>(a, stream);
    return a.D_I == 64 ? launch_prefill<4, 64>(a, stream) : launch_prefill<4, 128>(a, stream);
  }
  if (mode == 0) return launch_m<0>(a, stream);
  if (mode == 1) return launch_m<1>(a, stream);
  return launch_m<2>(a, stream);
}

}  // namespace dsa
