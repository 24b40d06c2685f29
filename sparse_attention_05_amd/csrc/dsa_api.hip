// C ABI of libdsa.so (declared in include/dsa.h): argument validation on the
// host, workspace layout, and the enqueue order of the fused decode step.
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "dsa.h"
#include "dsa_common.hpp"
#include "dsa_internal.hpp"

namespace dsa {

namespace {
thread_local char g_last_error[256] = "";

dsa_status hip_fail(hipError_t e) {
  snprintf(g_last_error, sizeof(g_last_error), "%s (%d): %s", hipGetErrorName(e), int(e), hipGetErrorString(e));
  return DSA_ERR_HIP;
}

bool aligned16(const void* p) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

size_t align256(size_t x) {
  return (x + 255) / 256 * 256;
}

constexpr int kMaxTopkRow = 1 << 20;  // longest score row the top-k accepts
constexpr int64_t kMaxCacheRows = (int64_t(1) << 31) - 1;  // the attention keeps cache rows in 31 bits

dsa_status check_index_args(const void* q, int q_dtype, const float* w, const void* keys, int k_dtype,
                            const uint16_t* k_scale, int64_t cache_rows, int B, int R, int H_I, int D_I,
                            int max_n) {
  if (!q || !w || !keys) return DSA_ERR_NULL;
  if (k_dtype == DSA_FP8_E4M3 && !k_scale) return DSA_ERR_NULL;
  if (R < 0 || B < 1 || cache_rows < 1 || max_n < 1) return DSA_ERR_SHAPE;
  if (H_I < 1 || H_I > 64) return DSA_ERR_UNSUPPORTED;
  if (D_I != 64 && D_I != 128) return DSA_ERR_UNSUPPORTED;
  const bool ok = (q_dtype == DSA_F32 && k_dtype == DSA_F32) || (q_dtype == DSA_BF16 && k_dtype == DSA_BF16) ||
                  (q_dtype == DSA_BF16 && k_dtype == DSA_FP8_E4M3);
  if (!ok) return DSA_ERR_DTYPE;
  if (!aligned16(q) || !aligned16(keys)) return DSA_ERR_ALIGN;
  if (k_dtype == DSA_FP8_E4M3 && (reinterpret_cast<uintptr_t>(k_scale) & 1u)) return DSA_ERR_ALIGN;
  return DSA_OK;
}

// The latent cache is stored in the activation dtype, or as fp8 codes with a
// float32 row scale next to bf16 queries.
dsa_status check_latent(int dtype, int latent_dtype, const float* latent_scale) {
  if (latent_dtype == DSA_FP8_E4M3) {
    if (dtype != DSA_BF16) return DSA_ERR_DTYPE;
    if (!latent_scale) return DSA_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(latent_scale) & 3u) return DSA_ERR_ALIGN;
    return DSA_OK;
  }
  return latent_dtype == dtype ? DSA_OK : DSA_ERR_DTYPE;
}

dsa_status check_attn_args(const void* q_abs, int dtype, const void* latent, int latent_dtype,
                           const float* latent_scale, int64_t cache_rows, int B, const int32_t* idx, int k, int R,
                           int H, const float* out) {
  if (!q_abs || !latent || !idx || !out) return DSA_ERR_NULL;
  if (dtype != DSA_F32 && dtype != DSA_BF16) return DSA_ERR_DTYPE;
  const dsa_status lt = check_latent(dtype, latent_dtype, latent_scale);
  if (lt != DSA_OK) return lt;
  if (R < 0 || B < 1 || cache_rows < 1) return DSA_ERR_SHAPE;
  if (cache_rows > kMaxCacheRows) return DSA_ERR_UNSUPPORTED;
  if (k < 1 || k > DSA_MAX_TOPK) return DSA_ERR_UNSUPPORTED;
  if (H < 1 || H > 128) return DSA_ERR_UNSUPPORTED;
  if (!aligned16(q_abs) || !aligned16(latent) || !aligned16(out)) return DSA_ERR_ALIGN;
  return DSA_OK;
}

// Where a sequence's cache rows are: consecutive from row_off[b], or in
// pages of 2^page_shift rows named by the block table.
struct CacheMap {
  const int64_t* row_off;
  const int32_t* table;
  int max_pages;
  int page_shift;
};

dsa_status check_cache_map(const CacheMap& m, int64_t cache_rows, int64_t max_len) {
  if (!m.table) return m.row_off ? DSA_OK : DSA_ERR_NULL;
  if (m.page_shift < 6 || m.page_shift > 20) return DSA_ERR_UNSUPPORTED;
  if (m.max_pages < 1 || cache_rows < (int64_t(1) << m.page_shift)) return DSA_ERR_SHAPE;
  if (max_len > (int64_t(m.max_pages) << m.page_shift)) return DSA_ERR_SHAPE;
  return DSA_OK;
}

// log2 of a power-of-two page size, else -1.
int page_shift_of(int32_t page_size) {
  if (page_size < 1 || (page_size & (page_size - 1))) return -1;
  int s = 0;
  while ((1 << s) < page_size) ++s;
  return s;
}

template <typename Args>
void set_map(Args& a, const CacheMap& m) {
  a.table = m.table;
  a.max_pages = m.max_pages;
  a.page_shift = m.page_shift;
}

// Fused-decode workspace, in order: scores [B, ld] fp32, indices [B, k],
// attention partials, score sample [B, ld_sample] fp32, split top-k
// candidates and counts (each part 256-byte aligned).
struct DecodeLayout {
  int64_t ld, ld_sample;
  size_t scores, idx, attn, sample, topk, total;
};
DecodeLayout decode_layout(int B, int max_len, int k, int H) {
  DecodeLayout L{};
  L.ld = (int64_t(max_len) + 3) / 4 * 4;
  L.ld_sample = ((int64_t(max_len) + 15) / 16 + 3) / 4 * 4;
  L.scores = 0;
  L.idx = L.scores + align256(size_t(B) * L.ld * sizeof(float));
  L.attn = L.idx + align256(size_t(B) * k * sizeof(int32_t));
  L.sample = L.attn + align256(plan_attention(B, H, k).ws_bytes);
  L.topk = L.sample + align256(size_t(B) * L.ld_sample * sizeof(float));
  L.total = L.topk + align256(topk_split_ws_bytes(B, max_len));
  return L;
}

size_t decode_ws_bytes(int B, int max_len, int k, int H) {
  return decode_layout(B, max_len, k, H).total;
}


dsa_status decode_fused_impl(const void* q_idx, const float* head_w, const void* k_idx, int32_t k_dtype,
                             const uint16_t* k_scale, const void* q_abs, const void* latent, int32_t act_dtype,
                             int32_t latent_dtype, const float* latent_scale, int64_t cache_rows, const CacheMap& cm,
                             const int32_t* seq_len, int32_t B, int32_t q_per_seq, int32_t max_len, int32_t H_I,
                             int32_t D_I, int32_t H, int32_t k, float scale, float* out, float* lse,
                             int32_t* idx_out, void* workspace, size_t ws_bytes, void* stream) {
  if (q_per_seq < 1 || q_per_seq > DSA_MAX_TOKENS_PER_SEQ) return DSA_ERR_UNSUPPORTED;
  if (B < 1 || int64_t(B) * q_per_seq > (int64_t(1) << 24)) return DSA_ERR_SHAPE;
  const int R = B * q_per_seq;  // query rows: q_per_seq per sequence, sequence-major
  dsa_status st = check_index_args(q_idx, act_dtype, head_w, k_idx, k_dtype, k_scale, cache_rows, B, R, H_I, D_I,
                                   max_len);
  if (st != DSA_OK) return st;
  st = check_cache_map(cm, cache_rows, max_len);
  if (st != DSA_OK) return st;
  if (!seq_len || !q_abs || !latent || !out) return DSA_ERR_NULL;
  if (act_dtype != DSA_F32 && act_dtype != DSA_BF16) return DSA_ERR_DTYPE;
  st = check_latent(act_dtype, latent_dtype, latent_scale);
  if (st != DSA_OK) return st;
  if (max_len > kMaxTopkRow || cache_rows > kMaxCacheRows) return DSA_ERR_UNSUPPORTED;
  if (k < 1 || k > DSA_MAX_TOPK || H < 1 || H > 128) return DSA_ERR_UNSUPPORTED;
  if (!aligned16(q_abs) || !aligned16(latent) || !aligned16(out)) return DSA_ERR_ALIGN;
  const size_t need = decode_ws_bytes(R, max_len, k, H);
  if (!workspace || ws_bytes < need) return DSA_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return DSA_ERR_ALIGN;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const DecodeLayout L = decode_layout(R, max_len, k, H);
  char* ws = static_cast<char*>(workspace);
  float* scores = reinterpret_cast<float*>(ws + L.scores);
  int32_t* idx = idx_out ? idx_out : reinterpret_cast<int32_t*>(ws + L.idx);
  void* attn_ws = ws + L.attn;
  float* sample = reinterpret_cast<float*>(ws + L.sample);
  const bool split = topk_use_split(R, max_len);

  // the indexer also writes the score sample the split top-k takes its pivot from
  IndexArgs ia{q_idx, act_dtype, head_w, k_idx, k_dtype, k_scale, cache_rows, cm.row_off, B, nullptr, nullptr,
               seq_len, R, H_I, D_I, max_len, scores, L.ld, split ? sample : nullptr, L.ld_sample};
  ia.qps = q_per_seq;
  set_map(ia, cm);
  hipError_t e = launch_index_scores(ia, s);
  if (e != hipSuccess) return hip_fail(e);
  TopkArgs ta{scores, L.ld, nullptr, seq_len, R, max_len, k, idx, split ? sample : nullptr, L.ld_sample,
              nullptr, nullptr};
  ta.qps = q_per_seq;
  const AttnPlan plan = plan_attention(R, H, k);
  AttnArgs aa{q_abs, act_dtype, latent, latent_dtype, latent_scale, cache_rows, cm.row_off, B, nullptr, idx, k,
              R, H, scale, out, lse, attn_ws};
  aa.qps = q_per_seq;
  set_map(aa, cm);
  if (split && act_dtype == DSA_BF16) {  // few long rows: selection fused with the attention
    topk_split_carve(ws + L.topk, R, max_len, ta);
    e = launch_topk_attn(ta, aa, plan, s);
    return e == hipSuccess ? DSA_OK : hip_fail(e);
  }
  if (split) topk_split_carve(ws + L.topk, R, max_len, ta);
  e = launch_topk(ta, s);
  if (e != hipSuccess) return hip_fail(e);
  e = launch_sparse_mla(aa, plan, s);
  return e == hipSuccess ? DSA_OK : hip_fail(e);
}

dsa_status sparse_mla_impl(const void* q_abs, int32_t dtype, const void* latent, int32_t latent_dtype,
                           const float* latent_scale, int64_t cache_rows, const CacheMap& cm, int32_t B,
                           const int32_t* q_seq, const int32_t* idx, int32_t k, int32_t R, int32_t H, float scale,
                           float* out, float* lse, void* workspace, size_t ws_bytes, void* stream) {
  dsa_status st = check_attn_args(q_abs, dtype, latent, latent_dtype, latent_scale, cache_rows, B, idx, k, R, H,
                                  out);
  if (st != DSA_OK) return st;
  st = check_cache_map(cm, cache_rows, 0);
  if (st != DSA_OK) return st;
  if (!q_seq && R != B) return DSA_ERR_SHAPE;
  const AttnPlan plan = plan_attention(R, H, k);
  if (plan.ws_bytes && (!workspace || ws_bytes < plan.ws_bytes)) return DSA_ERR_WORKSPACE;
  if (plan.ws_bytes && !aligned16(workspace)) return DSA_ERR_ALIGN;
  AttnArgs a{q_abs, dtype, latent, latent_dtype, latent_scale, cache_rows, cm.row_off, B, q_seq, idx, k, R, H,
             scale, out, lse, workspace};
  set_map(a, cm);
  hipError_t e = launch_sparse_mla(a, plan, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DSA_OK : hip_fail(e);
}

// ---- scratch of the no-allocation decode entry ---------------------------------
// One file-scope device array per GPU, held until the process ends. In host
// code `scratch` names a host-side stand-in, not device memory: its device
// address is looked up once per device (hipGetSymbolAddress, with that device
// current) and only that address is handed to kernels.
constexpr size_t kScratchBytes = size_t(64) << 20;
__device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices] = {};
std::mutex g_scratch_mu;

dsa_status scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= kMaxDevices) return DSA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e);
    if (!p || (reinterpret_cast<uintptr_t>(p) & 255u) != 0) return DSA_ERR_ALIGN;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DSA_OK;
}

}  // namespace

int record_hip_error(hipError_t e) {
  return hip_fail(e);
}

int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

}  // namespace dsa

using namespace dsa;

extern "C" {

dsa_status dsa_index_scores(const void* q_idx, int32_t q_dtype, const float* head_w, const void* k_idx,
                            int32_t k_dtype, const uint16_t* k_scale, int64_t cache_rows,
                            const int64_t* row_off, int32_t B, const int32_t* q_seq, const int32_t* q_pos,
                            int32_t R, int32_t H_I, int32_t D_I, int32_t max_n, float* scores,
                            int64_t ld_scores, void* stream) {
  dsa_status st = check_index_args(q_idx, q_dtype, head_w, k_idx, k_dtype, k_scale, cache_rows, B, R, H_I, D_I,
                                   max_n);
  if (st != DSA_OK) return st;
  if (!q_pos || !scores || !row_off) return DSA_ERR_NULL;
  if (!q_seq && R != B) return DSA_ERR_SHAPE;
  if (ld_scores < max_n || (ld_scores & 3)) return DSA_ERR_SHAPE;
  if (!aligned16(scores)) return DSA_ERR_ALIGN;
  IndexArgs a{q_idx, q_dtype, head_w, k_idx, k_dtype, k_scale, cache_rows, row_off, B, q_seq, q_pos, nullptr,
              R, H_I, D_I, max_n, scores, ld_scores, nullptr, 0};
  hipError_t e = launch_index_scores(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DSA_OK : hip_fail(e);
}

dsa_status dsa_index_scores_decode(const void* q_idx, int32_t q_dtype, const float* head_w, const void* k_idx,
                                   int32_t k_dtype, const uint16_t* k_scale, int64_t cache_rows,
                                   const int64_t* row_off, const int32_t* seq_len, int32_t B, int32_t q_per_seq,
                                   int32_t H_I, int32_t D_I, int32_t max_len, float* scores, int64_t ld_scores,
                                   void* stream) {
  if (q_per_seq < 1 || q_per_seq > DSA_MAX_TOKENS_PER_SEQ) return DSA_ERR_UNSUPPORTED;
  if (B < 1 || int64_t(B) * q_per_seq > (int64_t(1) << 24)) return DSA_ERR_SHAPE;
  const int R = B * q_per_seq;
  dsa_status st = check_index_args(q_idx, q_dtype, head_w, k_idx, k_dtype, k_scale, cache_rows, B, R, H_I, D_I,
                                   max_len);
  if (st != DSA_OK) return st;
  if (!seq_len || !scores || !row_off) return DSA_ERR_NULL;
  if (ld_scores < max_len || (ld_scores & 3)) return DSA_ERR_SHAPE;
  if (!aligned16(scores)) return DSA_ERR_ALIGN;
  IndexArgs a{q_idx, q_dtype, head_w, k_idx, k_dtype, k_scale, cache_rows, row_off, B, nullptr, nullptr, seq_len,
              R, H_I, D_I, max_len, scores, ld_scores, nullptr, 0};
  a.qps = q_per_seq;
  hipError_t e = launch_index_scores(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DSA_OK : hip_fail(e);
}

dsa_status dsa_topk(const float* scores, int64_t ld_scores, const int32_t* q_pos, int32_t R, int32_t max_n,
                    int32_t k, int32_t* idx_out, void* workspace, size_t ws_bytes, void* stream) {
  if (!scores || !q_pos || !idx_out) return DSA_ERR_NULL;
  if (R < 0 || max_n < 1) return DSA_ERR_SHAPE;
  if (max_n > kMaxTopkRow) return DSA_ERR_UNSUPPORTED;
  if (k < 1 || k > DSA_MAX_TOPK) return DSA_ERR_UNSUPPORTED;
  if (ld_scores < max_n || (ld_scores & 3)) return DSA_ERR_SHAPE;
  if (!aligned16(scores)) return DSA_ERR_ALIGN;
  TopkArgs a{scores, ld_scores, q_pos, nullptr, R, max_n, k, idx_out, nullptr, 0, nullptr, nullptr};
  hipStream_t s = static_cast<hipStream_t>(stream);
  // With a large enough workspace, few long rows are split over workgroups.
  if (workspace && topk_use_split(R, max_n) && ws_bytes >= topk_split_ws_bytes(R, max_n)) {
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return DSA_ERR_ALIGN;
    topk_split_carve(workspace, R, max_n, a);
  }
  hipError_t e = launch_topk(a, s);
  return e == hipSuccess ? DSA_OK : hip_fail(e);
}

dsa_status dsa_sparse_mla_attn(const void* q_abs, int32_t dtype, const void* latent, int32_t latent_dtype,
                               const float* latent_scale, int64_t cache_rows, const int64_t* row_off, int32_t B,
                               const int32_t* q_seq, const int32_t* idx, int32_t k, int32_t R, int32_t H,
                               float scale, float* out, float* lse, void* workspace, size_t ws_bytes,
                               void* stream) {
  return sparse_mla_impl(q_abs, dtype, latent, latent_dtype, latent_scale, cache_rows, CacheMap{row_off, nullptr, 0, 0},
                         B, q_seq, idx, k, R, H, scale, out, lse, workspace, ws_bytes, stream);
}

dsa_status dsa_sparse_mla_attn_paged(const void* q_abs, int32_t dtype, const void* latent, int32_t latent_dtype,
                                     const float* latent_scale, int64_t cache_rows, const int32_t* block_table,
                                     int32_t max_pages, int32_t page_size, int32_t B, const int32_t* q_seq,
                                     const int32_t* idx, int32_t k, int32_t R, int32_t H, float scale, float* out,
                                     float* lse, void* workspace, size_t ws_bytes, void* stream) {
  if (!block_table) return DSA_ERR_NULL;
  const int sh = page_shift_of(page_size);
  if (sh < 0) return DSA_ERR_UNSUPPORTED;
  return sparse_mla_impl(q_abs, dtype, latent, latent_dtype, latent_scale, cache_rows,
                         CacheMap{nullptr, block_table, max_pages, sh}, B, q_seq, idx, k, R, H, scale, out, lse,
                         workspace, ws_bytes, stream);
}

dsa_status dsa_decode_fused(const void* q_idx, const float* head_w, const void* k_idx, int32_t k_dtype,
                            const uint16_t* k_scale, const void* q_abs, const void* latent, int32_t act_dtype,
                            int32_t latent_dtype, const float* latent_scale, int64_t cache_rows,
                            const int64_t* row_off, const int32_t* seq_len, int32_t B, int32_t q_per_seq,
                            int32_t max_len, int32_t H_I, int32_t D_I, int32_t H, int32_t k, float scale,
                            float* out, float* lse, int32_t* idx_out, void* workspace, size_t ws_bytes,
                            void* stream) {
  return decode_fused_impl(q_idx, head_w, k_idx, k_dtype, k_scale, q_abs, latent, act_dtype, latent_dtype,
                           latent_scale, cache_rows, CacheMap{row_off, nullptr, 0, 0}, seq_len, B, q_per_seq,
                           max_len, H_I, D_I, H, k, scale, out, lse, idx_out, workspace, ws_bytes, stream);
}

dsa_status dsa_decode_fused_paged(const void* q_idx, const float* head_w, const void* k_idx, int32_t k_dtype,
                                  const uint16_t* k_scale, const void* q_abs, const void* latent,
                                  int32_t act_dtype, int32_t latent_dtype, const float* latent_scale,
                                  int64_t cache_rows, const int32_t* block_table, int32_t max_pages,
                                  int32_t page_size, const int32_t* seq_len, int32_t B, int32_t q_per_seq,
                                  int32_t max_len, int32_t H_I, int32_t D_I, int32_t H, int32_t k, float scale,
                                  float* out, float* lse, int32_t* idx_out, void* workspace, size_t ws_bytes,
                                  void* stream) {
  if (!block_table) return DSA_ERR_NULL;
  const int sh = page_shift_of(page_size);
  if (sh < 0) return DSA_ERR_UNSUPPORTED;
  return decode_fused_impl(q_idx, head_w, k_idx, k_dtype, k_scale, q_abs, latent, act_dtype, latent_dtype,
                           latent_scale, cache_rows, CacheMap{nullptr, block_table, max_pages, sh}, seq_len, B,
                           q_per_seq, max_len, H_I, D_I, H, k, scale, out, lse, idx_out, workspace, ws_bytes,
                           stream);
}

dsa_status dsa_decode_fused_noalloc(const void* q_idx, const float* head_w, const void* k_idx, int32_t k_dtype,
                                    const uint16_t* k_scale, const void* q_abs, const void* latent,
                                    int32_t act_dtype, int32_t latent_dtype, const float* latent_scale,
                                    int64_t cache_rows, const int64_t* row_off, const int32_t* seq_len, int32_t B,
                                    int32_t q_per_seq, int32_t max_len, int32_t H_I, int32_t D_I, int32_t H,
                                    int32_t k, float scale, float* out, float* lse, int32_t* idx_out,
                                    void* stream) {
  // sizes the workspace formula cannot take are rejected by the checks in
  // decode_fused_impl; the formula itself needs R >= 1, max_len >= 1, k, H >= 1
  if (q_per_seq < 1 || q_per_seq > DSA_MAX_TOKENS_PER_SEQ) return DSA_ERR_UNSUPPORTED;
  if (B < 1 || int64_t(B) * q_per_seq > (int64_t(1) << 24) || max_len < 1) return DSA_ERR_SHAPE;
  if (max_len > kMaxTopkRow || k < 1 || k > DSA_MAX_TOPK || H < 1 || H > 128) return DSA_ERR_UNSUPPORTED;
  const size_t need = decode_ws_bytes(B * q_per_seq, max_len, k, H);
  if (need > kScratchBytes) {
    snprintf(g_last_error, sizeof(g_last_error),
             "dsa_decode_fused_noalloc: this step needs %zu bytes of scratch; the library holds %zu per device",
             need, kScratchBytes);
    return DSA_ERR_WORKSPACE;
  }
  void* ws = nullptr;
  const dsa_status st = scratch_ptr(&ws);
  if (st != DSA_OK) return st;
  return decode_fused_impl(q_idx, head_w, k_idx, k_dtype, k_scale, q_abs, latent, act_dtype, latent_dtype,
                           latent_scale, cache_rows, CacheMap{row_off, nullptr, 0, 0}, seq_len, B, q_per_seq,
                           max_len, H_I, D_I, H, k, scale, out, lse, idx_out, ws, kScratchBytes, stream);
}

size_t dsa_decode_noalloc_limit(void) {
  return kScratchBytes;
}

size_t dsa_workspace_size(int32_t entry, int32_t rows, int32_t max_len, int32_t k, int32_t H) {
  if (rows < 0 || k < 1 || H < 1) return 0;
  switch (entry) {
    case DSA_ENTRY_TOPK:
      return topk_use_split(rows, max_len) ? topk_split_ws_bytes(rows, max_len) : 0;
    case DSA_ENTRY_SPARSE_MLA:
      return plan_attention(rows, H, k).ws_bytes;
    case DSA_ENTRY_DECODE:
      return decode_ws_bytes(rows, max_len < 1 ? 1 : max_len, k, H);
    default:
      return 0;
  }
}

const char* dsa_status_string(int32_t status) {
  switch (status) {
    case DSA_OK: return "ok";
    case DSA_ERR_NULL: return "a required pointer is NULL";
    case DSA_ERR_SHAPE: return "a size is out of range or inconsistent";
    case DSA_ERR_DTYPE: return "dtype or dtype combination not provided";
    case DSA_ERR_ALIGN: return "an array is not aligned as required";
    case DSA_ERR_WORKSPACE: return "workspace missing or too small";
    case DSA_ERR_UNSUPPORTED: return "shape not supported by this library";
    case DSA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* dsa_last_error(void) {
  return g_last_error;
}

}  // extern "C"
