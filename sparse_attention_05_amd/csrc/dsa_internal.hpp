// Host-side launchers behind the C ABI (include/dsa.h). Each enqueues its
// kernels on `stream` and returns the launch status; arguments were already
// validated by the entry point.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsa {

struct IndexArgs {
  const void* q;
  int q_dtype;
  const float* w;
  const void* keys;
  int k_dtype;
  const uint16_t* k_scale;
  int64_t cache_rows;
  const int64_t* row_off;
  int B;
  const int32_t* q_seq;  // NULL: query r is sequence r
  const int32_t* q_pos;  // NULL: q_pos[r] = seq_len[r] - 1 (decode form)
  const int32_t* seq_len;
  int R, H_I, D_I, max_n;
  float* scores;
  int64_t ld;
  float* sample;          // NULL, or receives sample[r * ld_sample + i] = scores[r, 16 i]
  int64_t ld_sample;
  int qps = 1;            // decode form (q_seq, q_pos NULL): row r is query r % qps of sequence r / qps,
                          // at position seq_len - qps + r % qps
  const int32_t* table = nullptr;  // paged caches: [B, max_pages] page ids (row_off unused)
  int max_pages = 0;
  int page_shift = 0;              // log2 of the page size (>= 6)
};
hipError_t launch_index_scores(const IndexArgs& a, hipStream_t stream);

struct TopkArgs {
  const float* scores;
  int64_t ld;
  const int32_t* q_pos;    // NULL: use seq_len - 1
  const int32_t* seq_len;
  int R, max_n, k;
  int32_t* idx;
  // Split selection (several workgroups per row), used when state and cand
  // are given and the rows are few and long:
  const float* sample;        // NULL, or sample[r * ld_sample + i] = scores[r, 16 i]
  int64_t ld_sample;
  uint32_t* state;            // [R][slices] uint4: candidate count, largest candidate key, pivot, 0
  unsigned long long* cand;   // [R][slices][slice_tiles * 2048] candidate words
  int slice_tiles;            // 2048-key tiles per slice (set with cand and state)
  int qps = 1;                // decode form (q_pos NULL): queries per sequence, as in IndexArgs
};
hipError_t launch_topk(const TopkArgs& a, hipStream_t stream);
bool topk_use_split(int R, int max_n);
size_t topk_split_ws_bytes(int R, int max_n);
void topk_split_carve(void* ws, int R, int max_n, TopkArgs& a);  // sets a.cand, a.state

struct AttnPlan {
  int splits;           // key splits per query row
  int keys_per_split;   // multiple of 64
  int head_groups;      // ceil(H / 16): one workgroup per (query, head group, split)
  size_t ws_bytes;      // partial-result workspace (0 when splits == 1)
  bool wide;            // many queries, H <= 64, one split: bf16 runs one workgroup per query for all heads
};
AttnPlan plan_attention(int R, int H, int k);

struct AttnArgs {
  const void* q;
  int dtype;
  const void* latent;
  int latent_dtype;            // dtype, or kFP8 (e4m3 codes) with bf16 queries
  const float* latent_scale;   // fp8 latent: one scale per cache row
  int64_t cache_rows;
  const int64_t* row_off;
  int B;
  const int32_t* q_seq;
  const int32_t* idx;
  int k, R, H;
  float scale;
  float* out;
  float* lse;
  void* ws;
  int qps = 1;  // q_seq NULL: row r belongs to sequence r / qps
  const int32_t* table = nullptr;  // paged caches, as in IndexArgs
  int max_pages = 0;
  int page_shift = 0;
};
hipError_t launch_sparse_mla(const AttnArgs& a, const AttnPlan& plan, hipStream_t stream);  // + combine
hipError_t launch_attn_combine(const AttnArgs& a, const AttnPlan& plan, hipStream_t stream);
// Split selection fused with the attention (rows few and long, ta.state and
// ta.cand set, bf16 attention operands): candidates, then selection +
// attention per (row, split, head group), then the combine.
hipError_t launch_topk_attn(const TopkArgs& ta, const AttnArgs& aa, const AttnPlan& plan, hipStream_t stream);

int device_cu_count();
// Records a failed launch's text for dsa_last_error(); returns DSA_ERR_HIP's value.
int record_hip_error(hipError_t e);

}  // namespace dsa
