// Internal launch interfaces between the C ABI layer (api.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hca.h"

namespace hca {

struct CompressArgs {
  const void* raw;
  int64_t raw_stride;  // elements
  const void* logits;
  int64_t logit_row_stride;  // elements
  int64_t logit_col_stride;  // 0 or 1
  const float* bias;         // [w, D]
  int64_t n_rows, first_pos, first_entry, n_entries;
  int m, w, D, d_nope;
  int raw_dtype;   // HCA_F32 / HCA_BF16
  int out_layout;  // HCA_LAYOUT_*
  void* out;
  int64_t out_stride;  // dense: elements; split: bytes
  float* out_scale;
  void* out_rope;
  int64_t out_rope_stride;  // elements
  int64_t out_row0;
};
hipError_t launch_compress(const CompressArgs& a, hipStream_t stream);

struct IndexArgs {
  const void* q;
  const uint8_t* q_scale;
  const float* w;
  int H, d, dtype;
  const void* keys;
  const uint8_t* key_scale;
  int64_t k_rows;
  const int64_t* k_row_begin;
  const int32_t* q_seq;
  const int64_t* q_pos;
  const int64_t* q_lo;  // document starts or nullptr
  int nq;  // queries of this batch (pointers above already offset to the batch)
  int64_t max_visible;
  int m, cw, k;  // cw: the CSA window (document masks)
  int32_t* out;  // [nq, k]
  // workspace views for the batch (set by index_ws_layout)
  int nblk;             // score blocks per query: ceil(max_visible / 1024)
  uint32_t* scores;     // [nq, max_visible] order-preserving score keys
  uint64_t* cand;       // [nq, nblk * 1024] candidate keys (score key << 32 | ~j), a fixed slot
                        // range per score block, 0 = empty slot
  uint64_t* ovf;        // [nq, nblk * 1024 + kMaxTopK] second-round candidates
  uint64_t* blk_thr;    // [nq, nblk] a block emitted exactly its keys >= this threshold
};
constexpr int kHistBins = 2048;
constexpr int kMaxTopK = 2048;
// Lays out the workspace of a batch of nq queries at `ws` (nullptr: only size it); returns bytes.
size_t index_ws_layout(int64_t nq, int64_t max_visible, void* ws, IndexArgs* a);
// scores: the score kernel (the candidates and block thresholds it leaves in the workspace);
// select: the selection kernel that reads them
hipError_t launch_index_topk(const IndexArgs& a, bool scores, bool select, hipStream_t stream);
// Calls taken by the streaming indexer (many queries, MXFP4 keys, 4 indexer heads, k <= 1536):
// one kernel with no workspace, so such a call is never cut into workspace-sized batches.
constexpr int kStreamMaxTopK = 1536;
inline bool index_stream_path(int dtype, int H, int64_t nq, int k) {
  return dtype == HCA_MXFP4 && H == 4 && nq >= 256 && k >= 1 && k <= kStreamMaxTopK;
}
hipError_t index_init();

struct StoreView {
  int layout, d_nope, d_rope;
  int64_t n_rows;
  const void* data;
  int64_t row_stride;
  const float* scale;
  const void* rope;
  int64_t rope_stride;
};

// One decode step (decode_append): inputs [B, D] / [B, d_idx] bf16, rings [B * R, .] bf16.
struct DecodeArgs {
  int B;
  const int64_t* pos;
  const uint16_t *x, *zc, *zh, *ki, *zi;
  int m, w, m_prime, W, R, D, d_idx;
  const float *bias_csa, *bias_hca, *bias_idx;
  uint16_t *ring_x, *ring_zc, *ring_zh, *ring_ki, *ring_zi;
  float* hca_state;  // [B, 3, D]
  StoreView win, csa, hca, idx;
  const int64_t* win_rb;
  int64_t* win_pos0;
  const int64_t *csa_rb, *hca_rb, *idx_rb;
};
hipError_t launch_decode_append(const DecodeArgs& a, hipStream_t stream);

// Grouped output projection: x [n, G Kg] (row stride ldx), w [G, Ng, Kg] bf16, y [n, G Ng] (row
// stride ldy) of y_dtype (HCA_F32 / HCA_BF16).
struct ProjArgs {
  const uint16_t* x;
  int64_t ldx;
  const uint16_t* w;
  void* y;
  int64_t ldy;
  int64_t n;
  int G, Kg, Ng, y_dtype;
};
hipError_t launch_proj(const ProjArgs& a, hipStream_t stream);

struct AttnArgs {
  const void* q;
  int q_dtype;
  int nq, H, D;
  StoreView cache, win;
  const int64_t* cache_row_begin;
  const int32_t* idx;  // CSA: [nq, k]; HCA: nullptr
  int k;               // CSA selection width
  int m_prime;         // HCA
  int64_t max_visible; // HCA
  const int64_t* win_row_begin;
  const int64_t* win_pos0;
  int W;
  const int32_t* q_seq;
  const int64_t* q_pos;
  const int64_t* q_lo;  // document starts or nullptr
  float scale;
  void* o;
  int o_dtype;
  float* lse;
  // split-K
  int n_split;
  int per_split;    // list positions per split
  float* part_o;    // [nq, n_split, H, D]
  float* part_lse;  // [nq, n_split, H]
};
// Chooses the split-K factor for a launch; the workspace query uses the same policy.
void attn_split_policy(int nq, int H, int D, int64_t max_entries, bool mfma, int* n_split,
                       int* per_split);
bool attn_mfma_supported(int q_dtype, int o_dtype, const StoreView& c, const StoreView& w, int H,
                         int D);
// The 64-head FP8 kernel (bf16 queries, split stores of 448 + 64 dims, H a multiple of 64) and its
// split policy.
bool attn_wide_supported(int q_dtype, const StoreView& c, const StoreView& w, int H, int nq);
void attn_split_policy_wide(int nq, int H, int64_t max_entries, int* n_split, int* per_split);
// combine = false leaves a split call's partials for a later launch_merge (deferred merge).
// sel: an index selection (launch_index_topk's select phase) to run with this call: in the same
// grid when the call takes the dense attn_fp8 kernel, else launched just before it
hipError_t launch_attention(const AttnArgs& a, hipStream_t stream, bool combine = true,
                            const IndexArgs* sel = nullptr);
// The LSE merge of one call's split-K partials, or of two calls' in one launch (b may be null).
struct MergeArgs {
  const float* part_o;
  const float* part_lse;
  void* o;
  float* lse;
  int nq, H, D, n_split, o_dtype;
};
hipError_t launch_merge(const MergeArgs& a, const MergeArgs* b, hipStream_t stream);
// The static scratch of hca_dense_mqa_attn_noalloc: its size, and its device address on the
// current device (looked up once per device).
constexpr size_t kNoallocScratchBytes = 16u << 20;
hipError_t noalloc_scratch(void** ptr);
// Dynamic LDS of the float32 attention kernel for H heads of width D, and its ceiling.
constexpr size_t kAttnValuMaxLds = 159 * 1024;  // 160 KiB less room for the static LDS
inline size_t attn_valu_lds_bytes(int H, int D) {
  return sizeof(float) * ((size_t)H * D + 16 * (size_t)D + 16 * (size_t)H + 3 * (size_t)H);
}

}  // namespace hca
