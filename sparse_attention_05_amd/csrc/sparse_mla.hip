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

// M: kF32 (fp32 queries and rows), kBF16, or kFP8 (bf16 queries, e4m3 rows
// with a row scale).
template <int M>
__global__ __launch_bounds__(kAttnThreads) void sparse_mla_kernel(AttnArgs a, int splits, int kps) {
  constexpr bool F32 = M == kF32;
  __shared__ typename std::conditional<M == kFP8, Smem8, Smem<F32>>::type sm;
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
  if constexpr (M == kFP8) {
    attend8(a, r, split, splits, hg, j_beg, j_end, base, s_idx, sm);
  } else {
    f32x8 qf[18];
    load_q<true>(a, r, h, grp, qf);
    attend_f32(a, r, split, splits, hg, j_beg, j_end, base, s_idx, qf, sm);
  }
}

// bf16 rows: 8 waves, the four compute waves of sparse_mla_kernel plus four
// waves that stage the query and gather rows by direct loads (attend_bf16).
__global__ __launch_bounds__(kAttnWaves8 * 64) void sparse_mla_bf16_kernel(AttnArgs a, int splits, int kps) {
  __shared__ Smem<false> sm;
  __shared__ int s_idx[kMaxTopk];  // the range's cache rows, -1 past it up to the chunk boundary
  const int HG = (a.H + kGroupHeads - 1) / kGroupHeads;
  int r, split, hg;
  map_block(blockIdx.x, a.R, splits, HG, r, split, hg);
  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int lane = t & 63;
  const int j_beg = split * kps;
  const int j_end = (j_beg + kps < a.k) ? j_beg + kps : a.k;
  const int span = j_end > j_beg ? (j_end - j_beg + kChunkKeys - 1) / kChunkKeys * kChunkKeys : 0;
  // the range's indices (every load in flight before the first store), the
  // sequence's first row, the compute waves' query fragments
  constexpr int kPer = kMaxTopk / (kAttnWaves8 * 64);
  int v[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int e = t + u * kAttnWaves8 * 64;
    const int j = j_beg + e;
    v[u] = e < span && j < j_end ? a.idx[int64_t(r) * a.k + j] : -1;
  }
  const int64_t base = seq_base(a, r);
  QRegs qr;  // the gather waves' query pieces
  if (wave >= 4) q_issue(a, r, hg, wave - 4, lane, qr);
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int e = t + u * kAttnWaves8 * 64;
    if (e < span) s_idx[e] = v[u];
  }
  rows_of_indices<kAttnWaves8 * 64>(a, base, s_idx, span);  // each thread rewrites the entries it stored
  lds_sync();
  attend_bf16(a, r, split, splits, hg, j_beg, j_end, s_idx, qr, sm);
}

// ---- many queries: one workgroup per query for all (<= 64) heads ---------------------
// With a workgroup per (query, 16 heads) every selected latent row would be
// gathered once per head group; here the 8 waves of one workgroup share each
// gathered chunk of 64 rows among all 64 heads, so a row is read once per
// query. Eight waves, two per SIMD, so that each SIMD has a second
// instruction stream to issue while the other waits (with one wave per SIMD
// the matrix cores sat idle three quarters of the time: the softmax, the
// LDS reads and the barriers were all exposed). Wave w = 4*kh + hg:
//  * q.c by (key half, head group): S^T for keys 32kh .. 32kh+31 and heads
//    16hg .. 16hg+15 (the query fragments of those heads stay in registers);
//    each head's chunk maximum combines its two key halves through LDS;
//  * softmax against each head's current reference maximum, right after the
//    wave's own q.c and without waiting for the other waves: the reference
//    moves only when a chunk's maximum exceeds it by more than 8 (log2), so
//    for almost every chunk the probabilities need no exchange; a wave that
//    sees a logit above its reference + 8 raises a flag, published with
//    P^T, and then every wave redoes the chunk's softmax exactly from the
//    exchanged maxima (one more barrier);
//  * P^T (bf16) goes to an array of its own, 144-byte rows per head;
//  * p.c by value slice: wave w forms O^T[64w .. 64w+63][all heads], each
//    transposed value fragment feeding the 4 head tiles.
// Rows go from HBM to LDS with direct loads issued from inline assembly and
// waited for exactly, so the gather of chunk c+1 overlaps chunk c: the two
// waves of head group hg each issue half of the loads of rows
// 16hg .. 16hg+15, each lane's row index loaded one chunk ahead into a
// register. Chunks past the last selected position are skipped (they would
// add exactly 0).
constexpr int kWideHeads = 64;
constexpr int kWideThreads = 512;
constexpr int kWidePtPitch = 144;  // bytes per head row of P^T (64 keys + 8 of padding: conflict-free reads and writes)

// LDS layout of a chunk (64 rows x 72 chunks of 16 bytes): wave w's rows
// 16w .. 16w+15 form a block of 18,432 bytes in which chunk c of row p sits
// at 1024*(c/4) + 64*p + 16*((c%4) ^ sw(p)), sw(p) = 2*((p/4)%2): rows 4..7
// and 12..15 of a block hold their chunk pairs swapped, which spreads the
// q.c reads (row per lane, a 64-byte stride), the transposed p.c reads and
// the P^T writes over all LDS banks (without it each pass of these reads
// met every bank twice, as the bank-conflict counter showed). The direct
// load m of a wave then covers chunks 4m .. 4m+3 of all 16 rows: lane l
// always reads row l/4 (its chunk 4m + ((l%4) ^ sw(l/4)) lands at 16-byte
// offset 4m + l%4), so a gather needs one address per lane.
constexpr int kWideBlock = 16 * 1152;
__device__ __forceinline__ int wide_sw(int row) { return 2 * ((row >> 2) & 1); }
__device__ __forceinline__ int wide_off(int row, int c) {
  return kWideBlock * (row >> 4) + 1024 * (c >> 2) + 64 * (row & 15) + 16 * ((c & 3) ^ wide_sw(row));
}

// The gather of rows 16*blk .. +15 of a chunk into buf, `key` being this
// lane's raw index (of row 16*blk + lane/4; -1 past the range): this lane's
// source row (a missing row reads cache row 0 and is zero-filled once it has
// landed), the LDS base of the block and the 16-bit mask of present rows;
// load m (0..17) is then dma16(src + 64m, lds + 1024m).
struct WideGather {
  const char* src;
  uint32_t lds;
  uint32_t mask;
};
__device__ __forceinline__ WideGather wide_gather(const AttnArgs& a, int64_t base, int key, char* buf, int blk,
                                                  int lane) {
  using Cfg = AttnCfg<false>;
  int64_t row;
  const bool ok = attn_row(a, base, key, row);
  const unsigned long long okm = __ballot(ok && (lane & 3) == 0);  // bit 4i: row i
  uint32_t mask = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) mask |= uint32_t((okm >> (4 * i)) & 1ull) << i;
  WideGather g;
  // (the lane's piece offset is recomputed per call: hoisted out of the
  // chunk loop it is a 64-bit register pair held across the whole loop)
  int ln = lane;
  asm volatile("" : "+v"(ln));
  g.src = static_cast<const char*>(a.latent) + row * Cfg::ROW_BYTES + 16 * ((ln & 3) ^ wide_sw(ln >> 2));
  g.lds = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)(buf + kWideBlock * blk))));
  g.mask = mask;
  return g;
}

// Reference maximum of a head's running softmax (log2 domain) after a chunk
// whose maximum is cmax: it moves (and the output accumulators are rescaled)
// only when cmax exceeds it by more than 8, so probabilities stay <= 2^8
// (exact in bf16's range, summed in fp32) and the 128-register rescale is
// rare. The softmax stays exact: sums and outputs use the same reference,
// the LSE adds it back.
// 2^x by the hardware's exponential (one instruction): results below 2^-126
// flush to 0, which only drops terms that cannot move a softmax sum whose
// largest term is >= 1, and -inf gives 0 as the softmax needs.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float wide_ref_max(float m_run, float cmax) {
  return (m_run == -INFINITY || cmax > m_run + 8.f) ? fmaxf(m_run, cmax) : m_run;
}

__global__ __launch_bounds__(kWideThreads) void sparse_mla_wide_kernel(AttnArgs a, int kps) {
  using Cfg = AttnCfg<false>;
  constexpr int WL = Cfg::WAVE_LOADS;  // direct loads per 16-row block per chunk
  static_assert(WL == 18, "18 direct loads cover a 16-row block");
  constexpr int WLH = WL / 2;          // each of the block's two waves issues half
  __shared__ __attribute__((aligned(1024))) char smem[2 * Cfg::BUF_BYTES];
  __shared__ __attribute__((aligned(16))) char s_pt[kWideHeads * kWidePtPitch];  // P^T: head h's 64 keys at h*pitch
  __shared__ float s_max[2][kWideHeads];  // chunk maximum of each head, per key half
  __shared__ float s_l[2][kWideHeads];
  __shared__ uint32_t s_ok[2][4];
  __shared__ uint32_t s_over[2][8];       // per chunk parity and wave: a logit above its reference + 8
  __shared__ int s_last[8];
  const int r = int(gridDim.x) - 1 - int(blockIdx.x);  // later queries (more keys) first
  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int lane = t & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int hg = wave & 3;   // q.c heads 16hg .. 16hg+15; gathered rows 16hg .. 16hg+15
  const int kh = wave >> 2;  // q.c keys 32kh .. 32kh+31; loads WLH*kh .. +WLH of the block
  const int64_t base = seq_base(a, r);
  const int j_end = kps < a.k ? kps : a.k;  // one split: keys 0 .. j_end-1
  const int32_t* ridx = a.idx + int64_t(r) * a.k;

  // The start's loads go out together, each unconditional (a clamped
  // position, head 0's row past H) with its condition applied after it has
  // landed: a load under a branch, or a select right behind it, makes the
  // compiler wait for it on the spot, and the start then paid the latency of
  // the index scan, the query fragments and chunk 0 one after another. First
  // the row indices of chunks 0 and 1, then the scan of the index row for the
  // last selected position (which bounds the chunks walked), then the query
  // fragments of this wave's q.c head 16*hg + col; chunk 0 is gathered as soon
  // as its indices have landed, while the rest are in flight.
  const int jl = 16 * hg + (lane >> 2);  // this lane's key within a chunk
  int key0 = ridx[min(jl, j_end - 1)];
  int key1 = ridx[min(kChunkKeys + jl, j_end - 1)];
  constexpr int kScan = 4;  // scan entries per thread held at once
  int sv[kScan];
  const bool scan_regs = j_end <= kScan * kWideThreads;
#pragma unroll
  for (int i = 0; i < kScan; ++i) sv[i] = ridx[min(t + i * kWideThreads, j_end - 1)];
  bf16x8 qf[18];
  const bool hv = 16 * hg + col < a.H;
  {
    const int64_t qoff = (int64_t(r) * a.H + (hv ? 16 * hg + col : 0)) * kLatentDim + 8 * grp;
#pragma unroll
    for (int ks = 0; ks < 18; ++ks)
      qf[ks] = __builtin_bit_cast(bf16x8,
                                  *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.q) + qoff + 32 * ks));
  }
  // chunk 0 (cache row 0 stands in for a missing row, and is zeroed): issued
  // before the chunk count is known, and drained by the epilogue's barrier
  // when there is no chunk to walk; chunk c+1 is issued during the q.c of
  // chunk c, one direct load per K-step, once every wave is done with the
  // buffer (chunk c-1's)
  uint32_t okw[2] = {0u, 0u};
  {
    const WideGather g = wide_gather(a, base, jl < j_end ? key0 : -1, smem, hg, lane);
#pragma unroll
    for (int m = WLH * kh; m < WLH * kh + WLH; ++m) dma16(g.src + 64 * m, g.lds + 1024 * m);
    okw[0] = g.mask;
  }
  key1 = kChunkKeys + jl < j_end ? key1 : -1;
  int last = -1;
  if (scan_regs) {
#pragma unroll
    for (int i = 0; i < kScan; ++i) last = t + i * kWideThreads < j_end && sv[i] >= 0 ? t + i * kWideThreads : last;
  } else {
    for (int e = t; e < j_end; e += kWideThreads) last = ridx[e] >= 0 ? e : last;
  }
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) last = max(last, __shfl_xor(last, d, 64));
  if (lane == 0) s_last[wave] = last;
  // every load above has landed; the fragments are re-defined through an
  // empty asm, so that no wait for them is placed inside the chunk loop
  // (where it would also wait for the next chunk's rows), and zeroed past H
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
  for (int ks = 0; ks < 18; ++ks) {
    uint4 u = __builtin_bit_cast(uint4, qf[ks]);
    asm volatile("" : "+v"(u.x), "+v"(u.y), "+v"(u.z), "+v"(u.w));
    qf[ks] = __builtin_bit_cast(bf16x8, hv ? u : uint4{0u, 0u, 0u, 0u});
  }
  __syncthreads();
  int lmax = s_last[0];
#pragma unroll
  for (int w = 1; w < 8; ++w) lmax = max(lmax, s_last[w]);
  const int nchunks = (lmax + kChunkKeys) / kChunkKeys;

  f32x4 acc[4][4];  // O^T[64*wave + 16*vt + (0..15)][16*ht + (0..15)]
#pragma unroll
  for (int vt = 0; vt < 4; ++vt)
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) acc[vt][ht] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mq = -INFINITY;  // running reference max of the q.c head 16*hg + col
  float lq = 0.f;        // this lane's share of its running sum (this key half)
  float mo[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};  // of the p.c heads 16ht + col
  const float scale2 = a.scale * kLog2e;
  const int hq = 16 * hg + col;  // this lane's q.c head

  for (int c = 0; c < nchunks; ++c) {
    const int bi = c & 1;
    char* buf = smem + bi * Cfg::BUF_BYTES;
    // this wave's loads of chunk c have landed (nothing else is in flight);
    // the parts of missing rows it loaded are zeroed; then every wave's are
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (okw[bi] != 0xFFFFu) {
      for (int q = lane; q < 16 * 4 * WLH; q += 64) {
        const int rr = q / (4 * WLH), cc = 4 * WLH * kh + q % (4 * WLH);
        if (!((okw[bi] >> rr) & 1u)) *reinterpret_cast<uint4*>(buf + wide_off(16 * hg + rr, cc)) = uint4{0u, 0u, 0u, 0u};
      }
    }
    if (lane == 0 && kh == 0) s_ok[bi][hg] = okw[bi];
    if (c > 0) key1 = kChunkKeys * (c + 1) + jl < j_end ? key1 : -1;
    __syncthreads();  // chunk c in LDS; every wave is done with p.c of chunk c-1 (its buffer and P^T)
    const bool more = c + 1 < nchunks;
    WideGather gn{nullptr, 0u, 0u};
    if (more) gn = wide_gather(a, base, key1, smem + (bi ^ 1) * Cfg::BUF_BYTES, hg, lane);
    // the raw index of this lane's key in chunk c+2 (lands with the chunk's
    // loads; its condition is applied at the next chunk, after the wait)
    key1 = ridx[min(kChunkKeys * (c + 2) + jl, j_end - 1)];
    okw[bi ^ 1] = gn.mask;

    // ---- q.c: S^T for keys 32kh + 16kt + (0..15), heads 16*hg + (0..15) ------------------
    // (the key fragments are read two K-steps ahead of their MFMAs; the
    // loop is instantiated with and without the next chunk's loads, so that
    // no branch splits it)
    f32x4 sc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    auto qc = [&](auto load_next) {
      constexpr bool LOADS = decltype(load_next)::value;
      // key row 16(2kh+kt) + col, dims 32ks + 8grp .. +8: chunk 4ks + grp
      const char* fbase = buf + kWideBlock * (2 * kh) + 64 * col + 16 * (grp ^ wide_sw(col));
      constexpr int AH = 3;  // K-steps of key fragments in flight
      bf16x8 fa[AH][2];
#pragma unroll
      for (int j = 0; j < AH - 1; ++j)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) fa[j][kt] = *reinterpret_cast<const bf16x8*>(fbase + kWideBlock * kt + 1024 * j);
      __builtin_amdgcn_sched_barrier(0);  // the pattern below starts with the reads of K-step AH-1
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) {
        if (ks + AH - 1 < 18) {
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
            fa[(ks + AH - 1) % AH][kt] =
                *reinterpret_cast<const bf16x8*>(fbase + kWideBlock * kt + 1024 * (ks + AH - 1));
        }
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) sc[kt] = mfma_k32(fa[ks % AH][kt], qf[ks], sc[kt]);
        if (LOADS && ks < WLH) dma16(gn.src + 64 * (WLH * kh + ks), gn.lds + 1024 * (WLH * kh + ks));
        if (ks + AH - 1 < 18) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      }
    };
    if (more) qc(std::true_type{});
    else qc(std::false_type{});

    // logits (log2 domain), -inf for missing keys (16-key tiles with a
    // missing key only); the head's maximum over this key half
    float x[2][4];
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const uint32_t okt = s_ok[bi][2 * kh + kt];
#pragma unroll
      for (int i = 0; i < 4; ++i) x[kt][i] = sc[kt][i] * scale2;
      if (okt != 0xFFFFu) {
#pragma unroll
        for (int i = 0; i < 4; ++i) x[kt][i] = ((okt >> (4 * grp + i)) & 1u) ? x[kt][i] : -INFINITY;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, x[kt][i]);
    }
    // ---- softmax against the current reference, P^T of this wave's heads and keys -------
    // (exact whenever no logit of the chunk exceeds its head's reference by
    // more than 8; a wave that sees one flags the chunk, and the exact form
    // below replaces these values)
    auto softmax = [&](float m_ref) -> float {
      const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
      float psum = 0.f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        __bf16 pv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // (the clamp only matters for a flagged chunk, whose values are replaced)
          pv[i] = static_cast<__bf16>(fast_exp2(fminf(x[kt][i] - m_use, 8.f)));
          psum += static_cast<float>(pv[i]);
        }
        // keys 16(2kh+kt) + 4grp .. +3 of head hq
        const uint32_t w0 = uint32_t(__builtin_bit_cast(uint16_t, pv[0])) | (uint32_t(__builtin_bit_cast(uint16_t, pv[1])) << 16);
        const uint32_t w1 = uint32_t(__builtin_bit_cast(uint16_t, pv[2])) | (uint32_t(__builtin_bit_cast(uint16_t, pv[3])) << 16);
        *reinterpret_cast<uint2*>(s_pt + kWidePtPitch * hq + 2 * (16 * (2 * kh + kt) + 4 * grp)) = uint2{w0, w1};
      }
      return psum;
    };
    float psum = softmax(mq);
    const bool over = __ballot(mx > mq + 8.f || (mq == -INFINITY && mx > -INFINITY)) != 0ull;
    mx = fmaxf(mx, wave_shfl_xor(mx, 16));
    mx = fmaxf(mx, wave_shfl_xor(mx, 32));
    {
      // (the address recomputed from an opaque lane index: held across the
      // loop it is spilled, and its reload would wait for the chunk's loads)
      int ln = lane;
      asm volatile("" : "+v"(ln));
      if ((ln >> 4) == 0) s_max[kh][16 * hg + (ln & 15)] = mx;
    }
    if (lane == 0) s_over[bi][wave] = over ? 1u : 0u;
    __syncthreads();  // P^T, the flags and the maxima visible
    uint32_t any = 0;
#pragma unroll
    for (int w = 0; w < 8; ++w) any |= s_over[bi][w];
    if (any) {
      // a reference moves: new references of every head from both key halves'
      // maxima, this wave's probabilities again against its head's, and the
      // p.c accumulators rescaled by the same per-head factors
      const float m_new = wide_ref_max(mq, fmaxf(s_max[0][hq], s_max[1][hq]));
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2(mq - m_use);
      psum = softmax(m_new);
      lq = lq * alpha + psum;
      mq = m_new;
#pragma unroll
      for (int ht = 0; ht < 4; ++ht) {
        const float cmax = fmaxf(s_max[0][16 * ht + col], s_max[1][16 * ht + col]);
        const float mn = wide_ref_max(mo[ht], cmax);
        const float mu = mn == -INFINITY ? 0.f : mn;
        const float al = fast_exp2(mo[ht] - mu);
        mo[ht] = mn;
        if (__ballot(al != 1.f)) {
#pragma unroll
          for (int vt = 0; vt < 4; ++vt) acc[vt][ht] *= al;
        }
      }
      __syncthreads();  // the exact P^T visible
    } else {
      lq += psum;
    }

    // ---- O^T[64*wave + 16*vt + (0..15)][16*ht + (0..15)] += C^T . P^T ---------------
    {
      const int tr_row = 4 * grp + (col >> 2);
      // P^T of head 16ht + col for K-step kq: keys 32kq + 4grp .. +3 and 32kq + 16 + 4grp .. +3
      auto pfrag = [&](int kq, bf16x8 (&pf)[4]) {
#pragma unroll
        for (int ht = 0; ht < 4; ++ht) {
          const char* pp = s_pt + kWidePtPitch * (16 * ht + col) + 2 * (32 * kq + 4 * grp);
          const uint2 plo = *reinterpret_cast<const uint2*>(pp);
          const uint2 phi = *reinterpret_cast<const uint2*>(pp + 32);
          pf[ht] = __builtin_bit_cast(bf16x8, uint4{plo.x, plo.y, phi.x, phi.y});
        }
      };
      // transposed value fragment of step q = (kq, vt), read one step ahead:
      // lane (col, grp) names key row 32kq + tr_row (+16 for the second
      // read), value dims 64*wave + 16vt + 4(col%4) .. +3: chunk
      // 8*wave + 2vt + (col%4)/2, half (col%4)&1
      auto vfrag = [&](int q) -> bf16x8 {
        const int kq = q >> 2, vt = q & 3;
        const char* p0 = buf + wide_off(32 * kq + tr_row, 8 * wave + 2 * vt + ((col & 3) >> 1)) + 8 * (col & 1);
        const short4v t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4v*)(lds_ptr)p0);
        const short4v t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) short4v*)(lds_ptr)(p0 + kWideBlock));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(t0, t1, 0, 1, 2, 3, 4, 5, 6, 7));
      };
#pragma unroll
      for (int kq = 0; kq < 2; ++kq) {
        bf16x8 pf[4], vf[2];
        pfrag(kq, pf);
        vf[0] = vfrag(4 * kq);
        __builtin_amdgcn_sched_barrier(0);  // the pattern below starts with the reads of step 1
#pragma unroll
        for (int vt = 0; vt < 4; ++vt) {
          if (vt + 1 < 4) vf[(vt + 1) & 1] = vfrag(4 * kq + vt + 1);
#pragma unroll
          for (int ht = 0; ht < 4; ++ht) acc[vt][ht] = mfma_k32(vf[vt & 1], pf[ht], acc[vt][ht]);
          if (vt + 1 < 4) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // ---- epilogue: row sums of each head (both key halves), then O rows --------------------
  {
    float l = lq + wave_shfl_xor(lq, 16);
    l += wave_shfl_xor(l, 32);
    if (grp == 0) s_l[kh][hq] = l;
  }
  __syncthreads();
#pragma unroll
  for (int ht = 0; ht < 4; ++ht) {
    const int h = 16 * ht + col;
    if (h >= a.H) continue;
    const float L = s_l[0][h] + s_l[1][h];
    const float inv = L > 0.f ? 1.f / L : 0.f;
    const int64_t rh = int64_t(r) * a.H + h;
    float* dst = a.out + rh * kValueDim;
#pragma unroll
    for (int vt = 0; vt < 4; ++vt)
      *reinterpret_cast<float4*>(dst + 64 * wave + 16 * vt + 4 * grp) =
          float4{acc[vt][ht][0] * inv, acc[vt][ht][1] * inv, acc[vt][ht][2] * inv, acc[vt][ht][3] * inv};
    if (wave == 0 && grp == 0 && a.lse) a.lse[rh] = L > 0.f ? (mo[ht] + __log2f(L)) * kLn2 : -INFINITY;
  }
}

// Merge key splits: O = sum_s e_s O_s / sum_s e_s l_s, e_s = 2^(m_s - max m),
// splits with an empty sum skipped. P adjacent lanes share one output float4,
// each lane loading and summing its SPL consecutive splits (all loads issued
// together), then the P partial sums are added in lane order (P * SPL >= splits). Every order is
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
  // (at device scope, like the split outputs: nothing of it is left for this
  // kernel's end to write back, and the next launch starts about 0.7 us
  // sooner at 4 x 32K)
  store_through(a.out + rh * kValueDim + 4 * v4, float4{acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv});
  if (a.lse && v4 == 0) store_through(a.lse + rh, L > 0.f ? (M + __log2f(L)) * kLn2 : -INFINITY);
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
  // many queries (two workgroups per CU even at one split): one workgroup per
  // query for all heads (bf16). Only past half as many rows as CUs: up to
  // there the fused decode step may run its own selection + attention kernel
  // (the 16-head core), and replaying its indices must run the same one.
  p.wide = H <= kWideHeads && int64_t(R) * p.head_groups >= 2 * int64_t(target) && 2 * int64_t(R) > target &&
           splits == 1;
  p.ws_bytes = splits > 1 ? size_t(R) * splits * H * (kValueDim + 2) * sizeof(float) : 0;
  p.ws_bytes = (p.ws_bytes + 255) / 256 * 256;
  return p;
}

hipError_t launch_sparse_mla(const AttnArgs& a, const AttnPlan& plan, hipStream_t stream) {
  if (a.R == 0) return hipSuccess;
  if (plan.wide && a.dtype == kBF16 && a.latent_dtype == kBF16) {
    sparse_mla_wide_kernel<<<dim3(unsigned(a.R)), kWideThreads, 0, stream>>>(a, plan.keys_per_split);
    return hipGetLastError();
  }
  const dim3 grid(unsigned(a.R) * unsigned(plan.splits) * unsigned(plan.head_groups));
  if (a.latent_dtype == kFP8) sparse_mla_kernel<kFP8><<<grid, kAttnThreads, 0, stream>>>(a, plan.splits, plan.keys_per_split);
  else if (a.dtype == kF32) sparse_mla_kernel<kF32><<<grid, kAttnThreads, 0, stream>>>(a, plan.splits, plan.keys_per_split);
  else sparse_mla_bf16_kernel<<<grid, kAttnWaves8 * 64, 0, stream>>>(a, plan.splits, plan.keys_per_split);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_attn_combine(a, plan, stream);
}

hipError_t launch_attn_combine(const AttnArgs& a, const AttnPlan& plan, hipStream_t stream) {
  if (a.R == 0 || plan.splits == 1) return hipSuccess;
  // P lanes per output float4, SPL splits per lane (splits <= 64), each
  // lane's loads all in flight together; 9-16 splits run as 2 x 8, which
  // measured faster than 4 x 4 and 1 x 16
  const int s = plan.splits;
  const int P = s <= 4 ? 1 : s <= 16 ? 2 : s <= 32 ? 8 : 16;
  const int64_t threads = int64_t(a.R) * a.H * (kValueDim / 4) * P;
  const dim3 cgrid(unsigned((threads + 255) / 256));
  if (s <= 4) combine_kernel<1, 4><<<cgrid, 256, 0, stream>>>(a, s);
  else if (s <= 8) combine_kernel<2, 4><<<cgrid, 256, 0, stream>>>(a, s);
  else if (s <= 16) combine_kernel<2, 8><<<cgrid, 256, 0, stream>>>(a, s);
  else if (s <= 32) combine_kernel<8, 4><<<cgrid, 256, 0, stream>>>(a, s);
  else combine_kernel<16, 4><<<cgrid, 256, 0, stream>>>(a, s);
  return hipGetLastError();
}

}  // namespace dsa
