// Core of the absorbed (MQA-form) sparse MLA attention: the work of one
// workgroup -- (query r, 16 heads, a range of selected positions) -- shared
// by the attention kernel and the fused selection + attention kernel, so
// that both compute the same bits from the same indices.
//
// For query r and head h over the selected positions j (idx[r, j] >= 0):
//   l_j = scale * q[r, h, :] . C[row_j, :]        (576-dim dots)
//   O[r, h, :] = sum_j softmax(l)_j * C[row_j, :512],  LSE[r, h] = log sum_j exp(l_j)
// ("GLM-5: from Vibe Coding to Agentic Engineering", section 2.1 and 3.2.)
// The decomposition is described in sparse_mla.hip.
#pragma once

#include <type_traits>

#include "dsa_common.hpp"
#include "dsa_internal.hpp"

namespace dsa {
namespace attn {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kAttnThreads = 256;   // 4 waves
constexpr int kGroupHeads = 16;     // heads per workgroup
constexpr int kChunkKeys = 64;      // keys per LDS buffer, 16 per wave
constexpr int kPRow = kChunkKeys + 4;  // padded row of the P^T staging array

template <bool F32>
struct AttnCfg {
  static constexpr int ESZ = F32 ? 4 : 2;                    // bytes per element
  static constexpr int ROW_BYTES = kLatentDim * ESZ;         // one latent row
  static constexpr int ROW_CHUNKS = ROW_BYTES / 16;          // 16-byte chunks per row (multiple of 8)
  static constexpr int BUF_BYTES = kChunkKeys * ROW_BYTES;
  static constexpr int NBUF = F32 ? 1 : 2;                   // LDS buffers (147,456 bytes either way)
  static constexpr int WAVE_LOADS = 16 * ROW_CHUNKS / 64;    // 1 KiB direct loads per wave per chunk
};
static_assert(AttnCfg<false>::ROW_CHUNKS % 8 == 0 && AttnCfg<true>::ROW_CHUNKS % 8 == 0, "swizzle groups");

typedef short short4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr;

// 16-byte direct-to-LDS load issued from inline assembly: lane l's 16 bytes
// land at LDS byte lds + 16*l (lds wave-uniform). The compiler does not see
// these loads, so it adds no waits for them: every use waits explicitly
// (vm_wait_all), and it never holds an LDS read of one buffer behind the
// loads into another.
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

// Wait until every vector memory operation of this wave has completed.
__device__ __forceinline__ void vm_wait_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)(p))));
}

// Chunk permutation of key row r (see the header comment).
__device__ __forceinline__ int row_swz(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }

// Cache row of selected position s of the sequence `base` names (its first
// row; paged caches: its index, the row then being row s mod page of page
// table[base][s / page], the page id clamped into the pool); false for a
// missing key (s < 0 or outside the cache or the block table).
__device__ __forceinline__ bool attn_row(const AttnArgs& a, int64_t base, int s, int64_t& row) {
  row = 0;
  if (s < 0 || base < 0) return false;
  if (a.table) {
    const int pi = s >> a.page_shift;
    if (pi >= a.max_pages) return false;
    int pg = a.table[base * a.max_pages + pi];
    const int npages = int(a.cache_rows >> a.page_shift);
    pg = pg < 0 ? 0 : (pg >= npages ? npages - 1 : pg);
    row = (int64_t(pg) << a.page_shift) + (s & ((1 << a.page_shift) - 1));
    return true;
  }
  if (base + s >= a.cache_rows) return false;
  row = base + s;
  return true;
}

// The gather of wave `wave`'s 16 rows of chunk c: keys
// j_beg + 64c + 16*wave + (0..15), whose raw indices the wave left in
// s_idx[64c + 16*wave + i] (-1 past the range). gather_plan reads the indices
// and zero-fills the rows of missing keys (idx < 0, outside the cache);
// gather_load(m) then issues the wave's direct load m (0 .. WAVE_LOADS-1),
// so the loads of a chunk can be spread over other work.
struct Gather {
  uint32_t src_lo, src_hi;  // lanes < 16: byte offset in the cache of row i (-1: missing)
  uint32_t ok;              // 16-bit mask of present rows (bit i: row 16*wave + i of the chunk)
  char* wbuf;               // the wave's block of the buffer
};

template <bool F32>
__device__ __forceinline__ Gather gather_plan(const AttnArgs& a, int64_t base, const int* s_idx, int c, char* buf,
                                              int wave, int lane) {
  using Cfg = AttnCfg<F32>;
  int64_t src = -1;
  if (lane < 16) {
    int64_t row;
    if (attn_row(a, base, s_idx[kChunkKeys * c + 16 * wave + lane], row)) src = row * Cfg::ROW_BYTES;
  }
  Gather g;
  g.ok = uint32_t(__ballot(src >= 0)) & 0xFFFFu;
  g.src_lo = uint32_t(uint64_t(src));
  g.src_hi = uint32_t(uint64_t(src) >> 32);
  g.wbuf = buf + 16 * wave * Cfg::ROW_BYTES;
  if (g.ok != 0xFFFFu) {
    for (int q = lane; q < 16 * Cfg::ROW_CHUNKS; q += 64)
      if (!((g.ok >> (q / Cfg::ROW_CHUNKS)) & 1u)) *reinterpret_cast<uint4*>(g.wbuf + 16 * q) = uint4{0u, 0u, 0u, 0u};
  }
  return g;
}

// Direct load m of a planned gather: the 64 16-byte pieces of rows rA (lanes
// < cut) and rA + 1, each landing at its permuted place in the row (the
// compiler's builtin, which the compiler waits for itself).
template <bool F32>
__device__ __forceinline__ void gather_load(const AttnArgs& a, const Gather& g, int m, int lane) {
  using Cfg = AttnCfg<F32>;
  const int rA = (64 * m) / Cfg::ROW_CHUNKS;
  const int cut = Cfg::ROW_CHUNKS * (rA + 1) - 64 * m;
  const int rB = rA + 1 < 16 ? rA + 1 : 15;
  const bool inA = lane < cut;
  const int rl = inA ? rA : rA + 1;
  const int pc = 64 * m + lane - Cfg::ROW_CHUNKS * rl;  // physical chunk in the row
  const int lc = pc ^ row_swz(rl);                      // logical chunk it holds
  const uint32_t loA = __builtin_amdgcn_readlane(g.src_lo, rA), loB = __builtin_amdgcn_readlane(g.src_lo, rB);
  const uint32_t hiA = __builtin_amdgcn_readlane(g.src_hi, rA), hiB = __builtin_amdgcn_readlane(g.src_hi, rB);
  const int64_t so = int64_t((uint64_t(inA ? hiA : hiB) << 32) | (inA ? loA : loB));
  const char* src = static_cast<const char*>(a.latent) + so + 16 * lc;
  if ((g.ok >> rl) & 1u) __builtin_amdgcn_global_load_lds(src, (lds_ptr)(g.wbuf + 1024 * m), 16, 0, 0);
}

// bf16 chunks use the block layout instead: rows 16w .. 16w+15 form a block
// of 18,432 bytes in which 16-byte piece p of row i sits at
// 1024*(p/4) + 64*i + 16*((p%4) ^ blk_sw(i)) (blk_off), blk_sw(i) =
// 2*((i/4)%2): rows 4..7 and 12..15 of a block hold their piece pairs
// swapped. The q.c reads (one row per lane, a 64-byte stride) and the
// transposed p.c reads then spread over all LDS banks; without the swap
// each of their passes met every bank twice (LDS bank-conflict counter).
constexpr int kBlock = 16 * 1152;
__device__ __forceinline__ int blk_sw(int row) { return 2 * ((row >> 2) & 1); }
__device__ __forceinline__ int blk_off(int row, int p) {
  return kBlock * (row >> 4) + 1024 * (p >> 2) + 64 * (row & 15) + 16 * ((p & 3) ^ blk_sw(row));
}

// The whole gather of chunk c at once; returns the mask of present rows.
template <bool F32>
__device__ __forceinline__ uint32_t issue_chunk(const AttnArgs& a, int64_t base, const int* s_idx, int c,
                                                char* buf, int wave, int lane) {
  const Gather g = gather_plan<F32>(a, base, s_idx, c, buf, wave, lane);
#pragma unroll
  for (int m = 0; m < AttnCfg<F32>::WAVE_LOADS; ++m) gather_load<F32>(a, g, m, lane);
  return g.ok;
}

// bf16 logits of this wave's 16 keys of the chunk: S^T = C[16 x 576] . Q^T.
// Lane (col, grp) reads piece 4ks + grp of row col of the wave's block (at
// blk + 64*col + 16*grp + 1024*ks: each K-step reads 1 KiB contiguously),
// four K-steps ahead of its MFMA (a compute wave has no other wave of its
// role on its SIMD to hide the LDS latency).
__device__ __forceinline__ f32x4 qc_bf16(const char* rp, const bf16x8 (&qf)[18]) {
  f32x4 part[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  constexpr int D = 4;
  bf16x8 fr[D];
#pragma unroll
  for (int i = 0; i < D; ++i) fr[i] = *reinterpret_cast<const bf16x8*>(rp + 1024 * i);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int ks = 0; ks < 18; ++ks) {
    const bf16x8 af = fr[ks % D];
    if (ks + D < 18) fr[ks % D] = *reinterpret_cast<const bf16x8*>(rp + 1024 * (ks + D));
    part[ks & 1] = mfma_k32(af, qf[ks], part[ks & 1]);
    if (ks + D < 18) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  return part[0] + part[1];
}

template <bool F32>
using QFrag = typename std::conditional<F32, f32x8, bf16x8>::type;

template <bool F32>
using PType = typename std::conditional<F32, float, __bf16>::type;

// bf16: the 16 heads' query rows staged once per workgroup in LDS (at dst,
// row h at 16-byte piece kQPitch*h: the pitch of 73 pieces makes the
// fragment reads conflict-free), 18 KiB of loads per workgroup instead of
// every wave loading all of them. All lanes load: pad slots and heads past H
// read the query's first piece, which nothing reads back.
constexpr int kQPitch = 73;
__device__ __forceinline__ void stage_q(const AttnArgs& a, int r, int hg, char* dst, int wave, int lane) {
  const char* q = static_cast<const char*>(a.q);
  const uint32_t d = lds_addr(dst);
  for (int m = wave; 64 * m < kGroupHeads * kQPitch; m += 4) {
    const int s = 64 * m + lane;
    const int h = s / kQPitch, j = s - kQPitch * h;
    const int hh = hg * kGroupHeads + h;
    const bool v = h < kGroupHeads && j < kLatentDim / 8 && hh < a.H;
    dma16(v ? q + ((int64_t(r) * a.H + hh) * kLatentDim + 8 * j) * 2 : q, d + 1024 * m);
  }
}

// This lane's query fragments (head hg*16 + col, dims 32*ks + 8*grp .. +8)
// from the staged rows; heads past H are zero.
__device__ __forceinline__ void read_q(const char* src, bool hv, int col, int grp, bf16x8 (&qf)[18]) {
#pragma unroll
  for (int ks = 0; ks < 18; ++ks) {
    const uint4 x = *reinterpret_cast<const uint4*>(src + 16 * (kQPitch * col + 4 * ks + grp));
    qf[ks] = __builtin_bit_cast(bf16x8, hv ? x : uint4{0u, 0u, 0u, 0u});
  }
}

// LDS of one workgroup's attention.
template <bool F32>
struct Smem {
  char buf[AttnCfg<F32>::NBUF * AttnCfg<F32>::BUF_BYTES] __attribute__((aligned(1024)));
  PType<F32> s_p[kGroupHeads * kPRow] __attribute__((aligned(16)));  // P^T as [head][key]
  float s_max[4][kGroupHeads];
  float s_l[4][kGroupHeads];
  uint32_t s_ok[2][4];  // bf16 gather: present rows of each 16-row block of the chunk in each buffer
};

// Workgroup u -> (query r, key split, head group). Workgroup u runs on XCD
// u mod 8: the head groups of one (query, split) go to the same XCD, so three
// of every four gathers of a latent row hit that XCD's L2.
__device__ __forceinline__ void map_block(int u, int R, int splits, int HG, int& r, int& split, int& hg) {
  const int pairs = R * splits;
  int pair;
  if ((pairs & 7) == 0) {
    const int local = u >> 3;
    pair = (local / HG) * 8 + (u & 7);
    hg = local % HG;
  } else {
    pair = u / HG;
    hg = u % HG;
  }
  r = pair / splits;
  split = pair % splits;
}

// Query fragments (B operand of q.c) of this lane's head: dims 32*ks + 8*grp .. +8.
template <bool F32>
__device__ __forceinline__ void load_q(const AttnArgs& a, int r, int h, int grp, QFrag<F32> (&qf)[18]) {
  // Heads past H (last group) load head H-1 and are zeroed.
  {
    const bool hv = h < a.H;
    const int64_t qoff = (int64_t(r) * a.H + (hv ? h : a.H - 1)) * kLatentDim + 8 * grp;
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
      if constexpr (F32) {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(a.q) + qoff + 32 * ks);
        const float4 x = p[0], y = p[1];
        qf[ks] = hv ? f32x8{{x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w}} : f32x8{{0, 0, 0, 0, 0, 0, 0, 0}};
      } else {
        const uint4 x = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.q) + qoff + 32 * ks);
        qf[ks] = __builtin_bit_cast(bf16x8, hv ? x : uint4{0u, 0u, 0u, 0u});
      }
    }
  }

}

// First cache row of query r's sequence, or (paged caches) the sequence's
// index (load it before the query fragments: waits are in issue order).
__device__ __forceinline__ int64_t seq_base(const AttnArgs& a, int r) {
  int b = a.q_seq ? a.q_seq[r] : r / a.qps;
  b = b < 0 ? 0 : (b >= a.B ? a.B - 1 : b);
  return a.table ? int64_t(b) : a.row_off[b];
}

// A 16-byte store at device scope (sc1): it goes through the L2 to memory.
// Whatever a kernel leaves dirty in an XCD's L2 is written back at its end,
// before the next launch on the stream can start; stores that went through
// already leave nothing of theirs to write back then. For the split outputs
// (read by the merge launch on every XCD) the merge starts about 1 us sooner
// at 4 x 32K; the same bits, the cache policy changes no value. Issued from
// inline assembly; nothing in the issuing kernel reads them.
__device__ __forceinline__ void store_through(float* p, float4 v) {
  const f32x4 x = __builtin_bit_cast(f32x4, v);
  asm volatile("global_store_dwordx4 %0, %1, off sc1" ::"v"(p), "v"(x) : "memory");
}
__device__ __forceinline__ void store_through(float* p, float2 v) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const f32x2 x = {v.x, v.y};
  asm volatile("global_store_dwordx2 %0, %1, off sc1" ::"v"(p), "v"(x) : "memory");
}
__device__ __forceinline__ void store_through(float* p, float v) {
  asm volatile("global_store_dword %0, %1, off sc1" ::"v"(p), "v"(v) : "memory");
}

// Epilogue of a workgroup: the row sums over the lanes and waves, then the
// normalised output rows as float4 (splits == 1) or the split's unnormalised
// output, its maximum and its sum.
__device__ __forceinline__ void write_result(const AttnArgs& a, int r, int split, int splits, int h, int wave,
                                             int col, int grp, const f32x4 (&acc)[8], float m_run, float l_part,
                                             float (*s_l)[kGroupHeads]) {
  float l_w = l_part + wave_shfl_xor(l_part, 16);
  l_w += wave_shfl_xor(l_w, 32);
  if (grp == 0) s_l[wave][col] = l_w;
  __syncthreads();
  const float L = ((s_l[0][col] + s_l[1][col]) + s_l[2][col]) + s_l[3][col];
  if (h >= a.H) return;
  const int64_t rh = int64_t(r) * a.H + h;
  const bool final_out = splits == 1;
  const float inv = final_out ? (L > 0.f ? 1.f / L : 0.f) : 1.f;
  float* dst = final_out ? a.out + rh * kValueDim
                         : static_cast<float*>(a.ws) + ((int64_t(r) * splits + split) * a.H + h) * kValueDim;
#pragma unroll
  for (int vt = 0; vt < 8; ++vt)
    store_through(dst + 128 * wave + 16 * vt + 4 * grp,
                  float4{acc[vt][0] * inv, acc[vt][1] * inv, acc[vt][2] * inv, acc[vt][3] * inv});
  if (wave == 0 && grp == 0) {
    if (final_out) {
      if (a.lse) store_through(a.lse + rh, L > 0.f ? (m_run + __log2f(L)) * kLn2 : -INFINITY);
    } else {
      float* ml = static_cast<float*>(a.ws) + int64_t(a.R) * splits * a.H * kValueDim;
      const int64_t slot = (int64_t(r) * splits + split) * a.H + h;
      store_through(ml + 2 * slot, float2{m_run, L});
    }
  }
}

// fp32 rows and queries: the chunk loop and the epilogue over keys j_beg ..
// j_end-1 of query r, for a 4-wave workgroup; s_idx[j - j_beg] holds the raw
// index of key j (-1: none), base the sequence's first cache row. One LDS
// buffer: each chunk's rows are gathered (direct loads into the row-major
// layout with the row_swz permutation), then q.c, softmax and p.c as in
// attend_bf16 on the fp32 matrix cores. Writes the normalised output
// (splits == 1) or the split's unnormalised output, maximum and sum.
__device__ __forceinline__ void attend_f32(const AttnArgs& a, int r, int split, int splits, int hg, int j_beg,
                                           int j_end, int64_t base, const int* s_idx, const f32x8 (&qf)[18],
                                           Smem<true>& sm) {
  using Cfg = AttnCfg<true>;
  char* smem = sm.buf;
  float* s_p = sm.s_p;
  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int lane = t & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int h = hg * kGroupHeads + col;
  const int nchunks = j_end > j_beg ? (j_end - j_beg + kChunkKeys - 1) / kChunkKeys : 0;

  f32x4 acc[8];
#pragma unroll
  for (int vt = 0; vt < 8; ++vt) acc[vt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;  // running max (log2 domain) of head h, equal in all waves
  float l_part = 0.f;       // this lane's share of the running sum
  const float scale2 = a.scale * kLog2e;

  for (int c = 0; c < nchunks; ++c) {
    char* buf = smem;
    if (c > 0) __syncthreads();  // every wave is done with the previous chunk
    const uint32_t okc = issue_chunk<true>(a, base, s_idx, c, buf, wave, lane);
    vm_wait_all();

    // ---- logits of this wave's 16 keys: S^T = C[16 x 576] . Q^T ----------------------
    f32x4 sacc;
    {
      const char* rp = buf + (16 * wave + col) * Cfg::ROW_BYTES;
      const int sw = row_swz(col);
      f32x4 part[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) {
        const int c0 = 8 * ks + 2 * grp;
        const float4 x = *reinterpret_cast<const float4*>(rp + 16 * (c0 ^ sw));
        const float4 y = *reinterpret_cast<const float4*>(rp + 16 * ((c0 + 1) ^ sw));
        const f32x8 af{{x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w}};
        part[ks & 1] = mfma_k32(af, qf[ks], part[ks & 1]);
      }
      sacc = part[0] + part[1];
    }

    // ---- chunk maximum per head over the 4 waves ----------------------------------------
    float x[4];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = ((okc >> (4 * grp + i)) & 1u) ? sacc[i] * scale2 : -INFINITY;
      mx = fmaxf(mx, x[i]);
    }
    mx = fmaxf(mx, wave_shfl_xor(mx, 16));
    mx = fmaxf(mx, wave_shfl_xor(mx, 32));
    if (grp == 0) sm.s_max[wave][col] = mx;
    __syncthreads();  // maxima visible; every wave has its rows of chunk c
    const float cmax = fmaxf(fmaxf(sm.s_max[0][col], sm.s_max[1][col]), fmaxf(sm.s_max[2][col], sm.s_max[3][col]));

    const float m_new = fmaxf(m_run, cmax);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;  // no key seen yet: p = alpha = 0
    const float alpha = exp2f(m_run - m_use);
    float psum = 0.f;
    float pv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pv[i] = exp2f(x[i] - m_use);
      psum += pv[i];
    }
    l_part = l_part * alpha + psum;
    m_run = m_new;
    if (__ballot(alpha != 1.f)) {
#pragma unroll
      for (int vt = 0; vt < 8; ++vt) acc[vt] *= alpha;
    }
    *reinterpret_cast<float4*>(s_p + col * kPRow + 16 * wave + 4 * grp) = float4{pv[0], pv[1], pv[2], pv[3]};
    __syncthreads();  // P^T of all 64 keys in LDS

    // ---- O^T[128*wave + 16*vt + (0..15)][head] += C^T . P^T over the 64 keys -------------
#pragma unroll
    for (int kq = 0; kq < kChunkKeys / 4; ++kq) {
      const int row = 4 * kq + grp;
      const float pf = s_p[col * kPRow + row];
      const char* rp = buf + row * Cfg::ROW_BYTES;
      const int sw = row_swz(row);
#pragma unroll
      for (int vt = 0; vt < 8; ++vt) {
        const int v = 128 * wave + 16 * vt + col;
        const float cv = *reinterpret_cast<const float*>(rp + 16 * ((v >> 2) ^ sw) + 4 * (v & 3));
        acc[vt] = __builtin_amdgcn_mfma_f32_16x16x4f32(cv, pf, acc[vt], 0, 0, 0);
      }
    }
  }

  write_result(a, r, split, splits, h, wave, col, grp, acc, m_run, l_part, sm.s_l);
}

// ---- bf16 rows, gathered by direct loads ---------------------------------------------------
// The workgroup has 8 waves: waves 0..3 compute (the q.c / softmax / p.c of
// attend, unchanged), waves 4..7 stage the query and gather. Rows 16w ..
// 16w+15 of a 64-row chunk form block w of the chunk buffer (blk_off), and a
// block is 18 direct loads: load m puts piece 4m + ((l%4) ^ blk_sw(l/4)) of
// the block's row l/4 at byte 1024m + 16l of the block, which is its place
// in the layout; a missing row's lanes write zeros there instead. Chunk 0
// goes out from the compute waves and chunk 1 from the gather waves, both
// before the first q.c, so a split of two chunks has all its rows in flight
// from eight waves at once; a later chunk goes out into the buffer of the
// chunk two before it as soon as that one's p.c is done.
constexpr int kAttnWaves8 = 8;
constexpr int kBlockLoads = kLatentDim * 2 / 64;  // 1-KiB direct loads per 16-row block (18)

// A barrier that orders LDS only: the direct loads in flight stay in flight.
__device__ __forceinline__ void lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// The range's raw indices s_idx[0 .. span) become cache rows (-1: missing
// key), by all threads of the workgroup, every lookup in flight at once (a
// paged cache reads its block table here, once per key, not in the gather).
// Cache rows fit in 31 bits (the entry points refuse larger caches).
template <int THREADS>
__device__ __forceinline__ void rows_of_indices(const AttnArgs& a, int64_t base, int* s_idx, int span) {
  constexpr int kPer = kMaxTopk / THREADS;
  int64_t row[kPer];
  bool ok[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int e = int(threadIdx.x) + u * THREADS;
    ok[u] = e < span && attn_row(a, base, s_idx[e < span ? e : 0], row[u]);
  }
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int e = int(threadIdx.x) + u * THREADS;
    if (e < span) s_idx[e] = ok[u] ? int(row[u]) : -1;
  }
}

// Issue the direct loads of block `blk` of chunk c (cache rows in s_row, -1
// for a missing key) into `buf`; returns the 16-bit mask of present rows.
// The caller waits (vm_wait_all) before the barrier that publishes the chunk.
__device__ __forceinline__ uint32_t gather_block(const AttnArgs& a, const int* s_row, int c, char* buf, int blk,
                                                 int lane) {
  const int i = lane >> 2;
  const int row = s_row[kChunkKeys * c + 16 * blk + i];
  const bool live = row >= 0;
  const unsigned long long okm = __ballot(live && (lane & 3) == 0);  // bit 4i: row i
  uint32_t ok = 0;
#pragma unroll
  for (int k = 0; k < 16; ++k) ok |= uint32_t((okm >> (4 * k)) & 1ull) << k;
  char* b = buf + kBlock * blk;
  if (live) {
    const char* src = static_cast<const char*>(a.latent) + int64_t(row) * 1152 + 16 * ((lane & 3) ^ blk_sw(i));
    const uint32_t d = lds_addr(b);
#pragma unroll
    for (int m = 0; m < kBlockLoads; ++m) dma16(src + 64 * m, d + 1024 * m);
  } else {
#pragma unroll
    for (int m = 0; m < kBlockLoads; ++m) *reinterpret_cast<uint4*>(b + 1024 * m + 16 * lane) = uint4{0u, 0u, 0u, 0u};
  }
  return ok;
}

// The query rows of the workgroup's 16 heads (16 x 72 pieces of 16 bytes),
// loaded by the gather waves into registers -- early, so that they land while
// the indices are being found -- and staged once in LDS for the compute waves
// (four compute waves loading them each would quadruple this traffic on the
// CU's load path, which bounds the kernel). Piece e = 256u + 64p + lane of
// gather wave p; heads past H read head H-1 (their columns are computed and
// never written).
constexpr int kQPieces = kGroupHeads * kLatentDim / 8;  // 1152
struct QRegs {
  bf16x8 v[5];  // a clang vector type: a HIP uint4 member is copied through private memory here
};
__device__ __forceinline__ void q_issue(const AttnArgs& a, int r, int hg, int p, int lane, QRegs& qr) {
#pragma unroll
  for (int u = 0; u < 5; ++u) {
    const int e0 = 256 * u + 64 * p + lane;
    const int e = e0 < kQPieces ? e0 : kQPieces - 1;  // past the rows: a piece that exists, not stored
    const int h = e / 72, j = e - 72 * (e / 72);
    const int hh = hg * kGroupHeads + h < a.H ? hg * kGroupHeads + h : a.H - 1;
    qr.v[u] = *reinterpret_cast<const bf16x8*>(static_cast<const uint16_t*>(a.q) +
                                               (int64_t(r) * a.H + hh) * kLatentDim + 8 * j);
  }
}
// Row h at piece kQPitch*h of `dst` (the pitch makes the fragment reads conflict-free).
__device__ __forceinline__ void q_store(const QRegs& qr, char* dst, int p, int lane) {
#pragma unroll
  for (int u = 0; u < 5; ++u) {
    const int e = 256 * u + 64 * p + lane;
    const int h = e / 72, j = e - 72 * (e / 72);
    if (e < kQPieces) *reinterpret_cast<bf16x8*>(dst + 16 * (kQPitch * h + j)) = qr.v[u];
  }
}

// attend() for bf16 rows with gather waves: the same split, arithmetic and
// order of operations as attend<false>, hence the same bits. All 8 waves call
// it; s_row holds the range's cache rows (rows_of_indices), filled by the
// caller, and qr the gather waves' query pieces (q_issue). Prologue: the
// compute waves issue chunk 0 into buffer 0 while the gather waves stage the
// query in buffer 1; the compute waves read the query into registers, which
// frees buffer 1 for chunk 1 (gather waves); chunk 0 lands. Then the two
// roles run separate loops with the same barriers, per chunk c:
//   compute: q.c(c) | B1 | softmax(c) | B2 | p.c(c)             | B3 |
//   gather :        | B1 |            | B2 | wait for c+1      | B3 | issue c+2
// (buffer c%2 holds chunk c, and takes chunk c+2 once B3 has closed c's p.c).
__device__ __forceinline__ void attend_bf16(const AttnArgs& a, int r, int split, int splits, int hg, int j_beg,
                                            int j_end, const int* s_row, const QRegs& qr, Smem<false>& sm) {
  using Cfg = AttnCfg<false>;
  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int lane = t & 63;
  const int nchunks = j_end > j_beg ? (j_end - j_beg + kChunkKeys - 1) / kChunkKeys : 0;

  if (wave >= 4) {
    // ---- gather waves: block p of chunks 1, 2, ... ---------------------------------------
    const int p = wave - 4;
    if (nchunks > 0) q_store(qr, sm.buf + Cfg::BUF_BYTES, p, lane);
    lds_sync();  // the query staged in buffer 1
    lds_sync();  // the compute waves have read the query: buffer 1 is free
    if (nchunks > 1) {
      const uint32_t m1 = gather_block(a, s_row, 1, sm.buf + Cfg::BUF_BYTES, p, lane);
      if (lane == 0) sm.s_ok[1][p] = m1;
    }
    lds_sync();  // chunk 0 in buffer 0
    for (int c = 0; c < nchunks; ++c) {
      lds_sync();  // B1
      lds_sync();  // B2
      if (c + 1 < nchunks) vm_wait_all();  // this wave's block of chunk c+1 has landed
      lds_sync();  // B3
      if (c + 2 < nchunks) {
        const int bn = c & 1;
        const uint32_t mk = gather_block(a, s_row, c + 2, sm.buf + bn * Cfg::BUF_BYTES, p, lane);
        if (lane == 0) sm.s_ok[bn][p] = mk;
      }
    }
    lds_sync();  // the row sums
    return;
  }

  // ---- compute waves ------------------------------------------------------------------------
  const int col = lane & 15, grp = lane >> 4;
  const int h = hg * kGroupHeads + col;
  if (nchunks > 0) {
    const uint32_t m0 = gather_block(a, s_row, 0, sm.buf, wave, lane);
    if (lane == 0) sm.s_ok[0][wave] = m0;
  }
  lds_sync();  // the query staged in buffer 1
  bf16x8 qf[18];  // B operand of q.c: head h, dims 32*ks + 8*grp .. +8
#pragma unroll
  for (int ks = 0; ks < 18; ++ks)
    qf[ks] = *reinterpret_cast<const bf16x8*>(sm.buf + Cfg::BUF_BYTES + 16 * (kQPitch * col + 4 * ks + grp));
  lds_sync();  // buffer 1 is free
  vm_wait_all();  // this wave's block of chunk 0 has landed
  lds_sync();  // chunk 0 in buffer 0
  f32x4 acc[8];
#pragma unroll
  for (int vt = 0; vt < 8; ++vt) acc[vt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;  // running max (log2 domain) of head h, equal in all compute waves
  float l_part = 0.f;       // this lane's share of the running sum
  const float scale2 = a.scale * kLog2e;
  const int tr_row = 4 * grp + (col >> 2);

  for (int c = 0; c < nchunks; ++c) {
    const int bi = c & 1;
    const char* buf = sm.buf + bi * Cfg::BUF_BYTES;
    float x[4];
    {
      const uint32_t okc = sm.s_ok[bi][wave];
      const char* rp = buf + kBlock * wave + 64 * col + 16 * (grp ^ blk_sw(col));
      const f32x4 sacc = qc_bf16(rp, qf);
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[i] = ((okc >> (4 * grp + i)) & 1u) ? sacc[i] * scale2 : -INFINITY;
        mx = fmaxf(mx, x[i]);
      }
      mx = fmaxf(mx, wave_shfl_xor(mx, 16));
      mx = fmaxf(mx, wave_shfl_xor(mx, 32));
      if (grp == 0) sm.s_max[wave][col] = mx;
    }
    lds_sync();  // B1: chunk maxima visible
    {
      const float cmax =
          fmaxf(fmaxf(sm.s_max[0][col], sm.s_max[1][col]), fmaxf(sm.s_max[2][col], sm.s_max[3][col]));
      const float m_new = fmaxf(m_run, cmax);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;  // no key seen yet: p = alpha = 0
      const float alpha = exp2f(m_run - m_use);
      float psum = 0.f;
      __bf16 pv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = exp2f(x[i] - m_use);
        pv[i] = static_cast<__bf16>(e);
        psum += static_cast<float>(pv[i]);
      }
      l_part = l_part * alpha + psum;
      m_run = m_new;
      if (__ballot(alpha != 1.f)) {
#pragma unroll
        for (int vt = 0; vt < 8; ++vt) acc[vt] *= alpha;
      }
      __bf16* prow = sm.s_p + col * kPRow + 16 * wave + 4 * grp;
      const uint32_t w0 = uint32_t(__builtin_bit_cast(uint16_t, pv[0])) | (uint32_t(__builtin_bit_cast(uint16_t, pv[1])) << 16);
      const uint32_t w1 = uint32_t(__builtin_bit_cast(uint16_t, pv[2])) | (uint32_t(__builtin_bit_cast(uint16_t, pv[3])) << 16);
      *reinterpret_cast<uint2*>(prow) = uint2{w0, w1};
    }
    lds_sync();  // B2: P^T of all 64 keys in LDS
    {
      // O^T[128*wave + 16*vt + (0..15)][head] += C^T . P^T over the 64 keys (as in attend)
      bf16x8 pf[2];
#pragma unroll
      for (int kq = 0; kq < 2; ++kq) {
        const __bf16* pp = sm.s_p + col * kPRow + 32 * kq + 4 * grp;
        const uint2 plo = *reinterpret_cast<const uint2*>(pp);
        const uint2 phi = *reinterpret_cast<const uint2*>(pp + 16);
        pf[kq] = __builtin_bit_cast(bf16x8, uint4{plo.x, plo.y, phi.x, phi.y});
      }
      auto vfrag = [&](int q) -> bf16x8 {
        const int kb = 32 * (q >> 3), vt = q & 7;
        const char* p0 = buf + blk_off(kb + tr_row, 16 * wave + 2 * vt + ((col >> 1) & 1)) + 8 * (col & 1);
        const short4v t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4v*)(lds_ptr)p0);
        const short4v t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) short4v*)(lds_ptr)(p0 + kBlock));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(t0, t1, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      constexpr int D = 3;
      bf16x8 vr[D];
#pragma unroll
      for (int i = 0; i < D; ++i) vr[i] = vfrag(i);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const bf16x8 af = vr[q % D];
        if (q + D < 16) vr[q % D] = vfrag(q + D);
        acc[q & 7] = mfma_k32(af, pf[q >> 3], acc[q & 7]);
        if (q + D < 16) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    lds_sync();  // B3: chunk c+1 in the other buffer; every compute wave is done with this one
  }

  // epilogue: the row sums over lanes and compute waves, then the output
  {
    float l_w = l_part + wave_shfl_xor(l_part, 16);
    l_w += wave_shfl_xor(l_w, 32);
    if (grp == 0) sm.s_l[wave][col] = l_w;
  }
  lds_sync();
  if (h >= a.H) return;
  const float L = ((sm.s_l[0][col] + sm.s_l[1][col]) + sm.s_l[2][col]) + sm.s_l[3][col];
  const int64_t rh = int64_t(r) * a.H + h;
  const bool final_out = splits == 1;
  const float inv = final_out ? (L > 0.f ? 1.f / L : 0.f) : 1.f;
  float* dst = final_out ? a.out + rh * kValueDim
                         : static_cast<float*>(a.ws) + ((int64_t(r) * splits + split) * a.H + h) * kValueDim;
#pragma unroll
  for (int vt = 0; vt < 8; ++vt)
    store_through(dst + 128 * wave + 16 * vt + 4 * grp,
                  float4{acc[vt][0] * inv, acc[vt][1] * inv, acc[vt][2] * inv, acc[vt][3] * inv});
  if (wave == 0 && grp == 0) {
    if (final_out) {
      if (a.lse) store_through(a.lse + rh, L > 0.f ? (m_run + __log2f(L)) * kLn2 : -INFINITY);
    } else {
      float* ml = static_cast<float*>(a.ws) + int64_t(a.R) * splits * a.H * kValueDim;
      const int64_t slot = (int64_t(r) * splits + split) * a.H + h;
      store_through(ml + 2 * slot, float2{m_run, L});
    }
  }
}

// ---- FP8 latent rows: e4m3 codes with one float32 scale per cache row ----------------------
// C[s, :] = e4m3(code[s, :]) * scale[s]. The codes convert exactly to bf16
// (every e4m3 value is a bf16 value), so q.c and p.c run on the same bf16
// MFMA; the row scale stays outside the products: it multiplies key j's
// logit (l_j = scale * s_j * (q . code_j)) and its softmax weight before the
// p.c (O = sum_j (p_j s_j) code_j / sum_j p_j).
// A chunk of 64 rows takes 36,864 bytes: wave w's rows 16w .. 16w+15 form a
// block of 9,216 bytes in which 16-byte piece p (0..35) of row i sits at
// 1024*(p/4) + 64*i + 16*(p%4) (blk8_off). Lane l loads row 16w + l/4, pieces
// 4m + l%4 for m = 0..8, and the scale of row 16w + l%16 into the wave's
// 64-word scale slot (four copies of its 16 scales), so a chunk is ten direct
// loads per wave.
// q.c: lane (col, grp) reads piece 4kk + grp of key row col (16 codes, one
// contiguous KiB per read over the wave) and feeds K-steps 2kk and 2kk+1 with
// its two halves; the query fragments use the same dims per K-slot.
// p.c: the value operand comes from the key-major rows through the
// transposing byte read (ds_read_b64_tr_b8: lane n of a 16-lane group names 8
// bytes of row n/2, and receives byte n of the group's 8 rows), converted to
// bf16 in registers.
constexpr int kBlock8 = 16 * kLatentDim;
constexpr int kBuf8 = 4 * kBlock8;
constexpr int kLoads8 = kLatentDim / 64;   // 1-KiB row loads per wave per chunk (then one for the scales)
constexpr int kPRow8 = kChunkKeys + 8;     // P^T row (bf16): 144 bytes, 16-byte aligned reads
static_assert(kGroupHeads * kQPitch * 16 <= kBuf8, "the staged query fits one fp8 buffer");

__device__ __forceinline__ int blk8_off(int row, int p) {
  return kBlock8 * (row >> 4) + 1024 * (p >> 2) + 64 * (row & 15) + 16 * (p & 3);
}

// 4-byte direct-to-LDS load (lane l's word lands at lds + 4*l), waited for
// like dma16.
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

struct Smem8 {
  char buf[2 * kBuf8] __attribute__((aligned(1024)));
  float sc[2][4][64] __attribute__((aligned(16)));  // [buffer][wave]: scales of the wave's 16 keys, 4 copies
  __bf16 s_p[kGroupHeads * kPRow8] __attribute__((aligned(16)));  // P^T as [head][key], scaled
  float s_max[4][kGroupHeads];
  float s_l[4][kGroupHeads];
};

struct BGather8 {
  const char* src;    // this lane's row + 16*(lane%4) (row 0 when missing: not loaded)
  const float* ssrc;  // scale of row 16w + lane%16 (row 0 when missing)
  uint32_t lds;       // LDS address of the wave's block
  uint32_t slds;      // LDS address of the wave's scale slot
  bool live;          // this lane's row is present
  uint32_t ok;        // 16-bit mask of present rows
};

__device__ __forceinline__ BGather8 bgather8_plan(const AttnArgs& a, int64_t base, const int* s_idx, int c,
                                                  char* buf, float* sc, int wave, int lane) {
  const int* si = s_idx + kChunkKeys * c + 16 * wave;
  int64_t row;
  BGather8 g;
  g.live = attn_row(a, base, si[lane >> 2], row);
  const unsigned long long okm = __ballot(g.live && (lane & 3) == 0);  // bit 4i: row i
  uint32_t ok = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) ok |= uint32_t((okm >> (4 * i)) & 1ull) << i;
  g.ok = ok;
  g.src = static_cast<const char*>(a.latent) + row * kLatentDim + 16 * (lane & 3);
  int64_t row2;
  attn_row(a, base, si[lane & 15], row2);  // row 0 when missing
  g.ssrc = a.latent_scale + row2;
  char* blk = buf + kBlock8 * wave;
  g.lds = lds_addr(blk);
  g.slds = lds_addr(sc + 64 * wave);
  if (!g.live) {
#pragma unroll
    for (int m = 0; m < kLoads8; ++m) *reinterpret_cast<uint4*>(blk + 1024 * m + 16 * lane) = uint4{0u, 0u, 0u, 0u};
  }
  return g;
}

// Direct load m (0 .. kLoads8) of a planned fp8 gather; the last one is the scales.
__device__ __forceinline__ void bgather8_load(const BGather8& g, int m) {
  if (m < kLoads8) {
    const char* p = g.src;
    asm volatile("" : "+v"(p));  // the address is formed here, not hoisted
    if (g.live) dma16(p + 64 * m, g.lds + 1024 * m);
  } else {
    dma4(g.ssrc, g.slds);
  }
}

// Query fragments for the fp8 K-slot order: K-step 2kk + hf of lane (col,
// grp) holds dims 64kk + 16grp + 8hf .. +8 (staged piece 8kk + 2grp + hf).
__device__ __forceinline__ void read_q8(const char* src, bool hv, int col, int grp, bf16x8 (&qf)[18]) {
#pragma unroll
  for (int kk = 0; kk < 9; ++kk)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const uint4 x = *reinterpret_cast<const uint4*>(src + 16 * (kQPitch * col + 8 * kk + 2 * grp + hf));
      qf[2 * kk + hf] = __builtin_bit_cast(bf16x8, hv ? x : uint4{0u, 0u, 0u, 0u});
    }
}

// fp8 logits of this wave's 16 keys, before the row scales: S^T = code[16 x 576] . Q^T.
// LOADS: direct load kk of the next chunk's gather rides on piece kk (the
// scale load after the loop).
template <bool LOADS>
__device__ __forceinline__ f32x4 qc_fp8(const char* rp, const bf16x8 (&qf)[18], const BGather8& gn) {
  f32x4 part[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  constexpr int D = 3;
  uint4 fr[D];
#pragma unroll
  for (int i = 0; i < D; ++i) fr[i] = *reinterpret_cast<const uint4*>(rp + 1024 * i);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int kk = 0; kk < kLoads8; ++kk) {
    const uint4 x = fr[kk % D];
    if (kk + D < kLoads8) fr[kk % D] = *reinterpret_cast<const uint4*>(rp + 1024 * (kk + D));
    part[0] = mfma_k32(fp8x8_to_bf16(uint2{x.x, x.y}), qf[2 * kk], part[0]);
    part[1] = mfma_k32(fp8x8_to_bf16(uint2{x.z, x.w}), qf[2 * kk + 1], part[1]);
    if constexpr (LOADS) bgather8_load(gn, kk);
  }
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (LOADS) bgather8_load(gn, kLoads8);
  return part[0] + part[1];
}

// attend() for fp8 latent rows (bf16 queries); same decomposition, split
// order and epilogue.
__device__ __forceinline__ void attend8(const AttnArgs& a, int r, int split, int splits, int hg, int j_beg,
                                       int j_end, int64_t base, const int* s_idx, Smem8& sm) {
  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int lane = t & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int h = hg * kGroupHeads + col;
  const int nchunks = j_end > j_beg ? (j_end - j_beg + kChunkKeys - 1) / kChunkKeys : 0;

  bf16x8 qf[18];
  uint32_t ok[2] = {0u, 0u};
  if (nchunks > 0) {
    // chunk 0 and the staged query (in buffer 1) in one round trip
    const BGather8 g = bgather8_plan(a, base, s_idx, 0, sm.buf, &sm.sc[0][0][0], wave, lane);
#pragma unroll
    for (int m = 0; m <= kLoads8; ++m) bgather8_load(g, m);
    ok[0] = g.ok;
    stage_q(a, r, hg, sm.buf + kBuf8, wave, lane);
    vm_wait_all();
    __syncthreads();
    read_q8(sm.buf + kBuf8, h < a.H, col, grp, qf);
    __syncthreads();  // every wave has its fragments: buffer 1 is free
  }

  f32x4 acc[8];
#pragma unroll
  for (int vt = 0; vt < 8; ++vt) acc[vt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;
  float l_part = 0.f;
  const float scale2 = a.scale * kLog2e;

  for (int c = 0; c < nchunks; ++c) {
    const int bi = c & 1;
    char* buf = sm.buf + bi * kBuf8;
    if (c > 0) vm_wait_all();  // this wave's rows and scales of chunk c have landed
    const uint32_t okc = ok[bi];

    // ---- logits of this wave's 16 keys --------------------------------------------------
    const char* rp = buf + kBlock8 * wave + 64 * col + 16 * grp;
    f32x4 sacc;
    if (c == 0 && nchunks > 1) {  // buffer 1 is free since the query was read
      const BGather8 gn = bgather8_plan(a, base, s_idx, 1, sm.buf + kBuf8, &sm.sc[1][0][0], wave, lane);
      ok[1] = gn.ok;
      sacc = qc_fp8<true>(rp, qf, gn);
    } else {
      sacc = qc_fp8<false>(rp, qf, BGather8{});
    }
    const float4 s4 = *reinterpret_cast<const float4*>(&sm.sc[bi][wave][4 * grp]);  // keys 4grp + i
    float sk[4] = {s4.x, s4.y, s4.z, s4.w};
    float x[4];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool live = (okc >> (4 * grp + i)) & 1u;
      sk[i] = live ? sk[i] : 0.f;
      x[i] = live ? (sacc[i] * sk[i]) * scale2 : -INFINITY;
      mx = fmaxf(mx, x[i]);
    }
    mx = fmaxf(mx, wave_shfl_xor(mx, 16));
    mx = fmaxf(mx, wave_shfl_xor(mx, 32));
    if (grp == 0) sm.s_max[wave][col] = mx;
    __syncthreads();  // maxima visible; every wave is done with chunk c-1 and has its rows of chunk c
    const float cmax = fmaxf(fmaxf(sm.s_max[0][col], sm.s_max[1][col]), fmaxf(sm.s_max[2][col], sm.s_max[3][col]));
    const bool pc_loads = c + 1 < nchunks && c >= 1;
    BGather8 gn{};
    if (pc_loads) {
      gn = bgather8_plan(a, base, s_idx, c + 1, sm.buf + (bi ^ 1) * kBuf8, &sm.sc[bi ^ 1][0][0], wave, lane);
      ok[bi ^ 1] = gn.ok;
    }

    const float m_new = fmaxf(m_run, cmax);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    float psum = 0.f;
    __bf16 pv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float e = exp2f(x[i] - m_use);
      psum += e;
      pv[i] = static_cast<__bf16>(e * sk[i]);
    }
    l_part = l_part * alpha + psum;
    m_run = m_new;
    if (__ballot(alpha != 1.f)) {
#pragma unroll
      for (int vt = 0; vt < 8; ++vt) acc[vt] *= alpha;
    }
    {
      __bf16* prow = sm.s_p + col * kPRow8 + 16 * wave + 4 * grp;
      const uint32_t w0 = uint32_t(__builtin_bit_cast(uint16_t, pv[0])) | (uint32_t(__builtin_bit_cast(uint16_t, pv[1])) << 16);
      const uint32_t w1 = uint32_t(__builtin_bit_cast(uint16_t, pv[2])) | (uint32_t(__builtin_bit_cast(uint16_t, pv[3])) << 16);
      *reinterpret_cast<uint2*>(prow) = uint2{w0, w1};
    }
    __syncthreads();  // P^T of all 64 keys in LDS

    // ---- O^T[128*wave + 16*vt + (0..15)][head] += code^T . (P s)^T over the 64 keys ------
    // K-slot 8*grp + i <-> key 32*kq + 8*grp + i.
    bf16x8 pf[2];
#pragma unroll
    for (int kq = 0; kq < 2; ++kq)
      pf[kq] = *reinterpret_cast<const bf16x8*>(sm.s_p + col * kPRow8 + 32 * kq + 8 * grp);
    // value fragment of step q = (kq = q/8, vt = q%8): lane (col, grp) names 8
    // bytes of row 32kq + 8grp + col/2, value dims 128*wave + 16vt + 8(col%2) ..,
    // that is piece 8*wave + vt, half col%2
    auto vfrag = [&](int q) -> bf16x8 {
      const int kq = q >> 3, vt = q & 7;
      const char* p0 = buf + blk8_off(32 * kq + 8 * grp + (col >> 1), 8 * wave + vt) + 8 * (col & 1);
      typedef int v2i __attribute__((ext_vector_type(2)));
      const v2i w = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) v2i*)(lds_ptr)p0);
      return fp8x8_to_bf16(uint2{uint32_t(w.x), uint32_t(w.y)});
    };
    auto pc = [&](auto loads) {
      constexpr bool LOADS = decltype(loads)::value;
      constexpr int D = 3;
      bf16x8 vr[D];
#pragma unroll
      for (int i = 0; i < D; ++i) vr[i] = vfrag(i);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const bf16x8 af = vr[q % D];
        if (q + D < 16) vr[q % D] = vfrag(q + D);
        acc[q & 7] = mfma_k32(af, pf[q >> 3], acc[q & 7]);
        if constexpr (LOADS) {
          if (q <= kLoads8) bgather8_load(gn, q);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    if (pc_loads) pc(std::true_type{});
    else pc(std::false_type{});
  }

  write_result(a, r, split, splits, h, wave, col, grp, acc, m_run, l_part, sm.s_l);
}

}  // namespace attn
}  // namespace dsa
