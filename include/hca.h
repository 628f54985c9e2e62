/*
 * hca.h — C ABI of the CSA + HCA hybrid-attention library for AMD MI355X
 * (gfx950).
 *
 * The method: hyper.ai paper page for arXiv 2606.19348 ("DeepSeek-V4"),
 * section 方法 (Method), paragraphs on CSA, HCA and efficiency. CSA
 * compresses every m tokens of KV into one entry with learnable compression
 * weights and a position bias, a lightning indexer picks the top-k
 * compressed entries per query, and MQA core attention with shared keys and
 * values runs over them; HCA merges every m' >> m tokens into one entry
 * without overlap and runs dense attention over all entries; both add a
 * sliding-window branch. KV entries keep BF16 RoPE dims and FP8 for the
 * rest; the indexer runs in FP4. The model card's "Tensor type" list
 * (F8_E4M3, F8_E8M0) fixes FP8 = OCP E4M3FN and FP4 = MX E2M1 with E8M0
 * block scales (block 32).
 *
 * Conventions shared by every entry point:
 *  - Pure, stream-ordered functions. The caller owns every buffer (inputs,
 *    outputs, workspace). The library allocates no device memory and keeps
 *    no state besides its loaded kernels; it is thread-safe.
 *  - All tensor pointers are DEVICE pointers (hipMalloc'd or torch CUDA
 *    tensors); `hca_store` structs themselves live in host memory and are
 *    read during the call only. `stream` is a hipStream_t (NULL = the null
 *    stream). Work is enqueued on `stream`; results are valid once the
 *    caller synchronises it.
 *  - Every argument that the host can check is checked before anything is
 *    enqueued; a failing check returns a negative status and enqueues
 *    nothing. Contents of device arrays (positions, row offsets, indices)
 *    are preconditions stated per function: violating them gives unspecified
 *    values but never an out-of-bounds access, because every kernel clamps
 *    its reads to the `n_rows` of the views it is given.
 *  - Device pointers must be 16-byte aligned, and row strides must keep
 *    every row 16-byte aligned (status HCA_ERR_INVALID_ARG otherwise).
 *  - Positions are absolute token positions (int64). Entry indices are
 *    relative to the first row of their sequence in a store (int32/int64).
 *  - hca_last_error() returns a message for the last failing call on the
 *    calling thread.
 */
#ifndef HCA_H_
#define HCA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HCA_ABI_VERSION 3

/* Status codes. */
#define HCA_OK 0
#define HCA_ERR_INVALID_ARG (-1) /* NULL, range, alignment, raw rows missing  */
#define HCA_ERR_UNSUPPORTED (-2) /* dtype / layout / shape combination        */
#define HCA_ERR_WORKSPACE (-3)   /* workspace smaller than required           */
#define HCA_ERR_HIP (-4)         /* a HIP launch failed                       */

/* Element types. */
#define HCA_F32 0
#define HCA_BF16 1
#define HCA_FP8_E4M3 2
#define HCA_MXFP4 3

/* Layouts of a store of KV rows (compressed entries or raw window tokens). */
#define HCA_LAYOUT_F32 0   /* dense rows of D float32                          */
#define HCA_LAYOUT_BF16 1  /* dense rows of D bf16                             */
#define HCA_LAYOUT_SPLIT 2 /* per row: d_nope E4M3 bytes, one float32 power-of-
                              two scale (value = code * scale), d_rope bf16
                              (the efficiency paragraph: FP8 for the non-RoPE
                              dims, BF16 for the RoPE dims)                   */
#define HCA_LAYOUT_MXFP4 3 /* per row: D/2 bytes of E2M1 codes (element 2i in
                              the low nibble of byte i) and D/32 E8M0 block
                              scales (the efficiency paragraph: FP4 indexer;
                              OCP MX blocks of 32). Written by the
                              compressors only: the indexer-key layout.       */

/*
 * A view of n_rows KV rows of width D = d_nope + d_rope. The first d_nope
 * columns are the non-RoPE dims, the last d_rope the RoPE dims.
 *  dense layouts: row r is `data + r * row_stride` (elements of the layout's
 *                 type); scale/rope/rope_stride are unused.
 *  split layout:  row r's FP8 codes are `data + r * row_stride` (bytes), its
 *                 scale is `scale[r]`, its RoPE dims are
 *                 `rope + r * rope_stride` (bf16 elements).
 *  MXFP4 layout:  d_nope = D (a multiple of 32), d_rope = 0; row r's codes
 *                 are `data + r * row_stride` (bytes), its E8M0 scales are
 *                 the bytes `(uint8_t*)rope + r * rope_stride`; `scale` is
 *                 unused. The scale rows are byte-addressed (no 16-byte
 *                 alignment needed); k_idx / k_idx_scale of
 *                 lightning_index_topk are such a store with row_stride
 *                 d/2 and rope_stride d/32.
 */
typedef struct hca_store {
  int32_t layout;
  int32_t d_nope;
  int32_t d_rope;
  int32_t reserved; /* must be 0 */
  int64_t n_rows;
  void* data;
  int64_t row_stride;
  float* scale;
  void* rope;
  int64_t rope_stride;
} hca_store;

int hca_abi_version(void);
const char* hca_status_string(int status);
const char* hca_last_error(void);

/*
 * csa_compress — CSA compressor (CSA paragraph: every m tokens into one
 * entry with learnable compression weights and a position bias; CSA windows
 * overlap since only HCA is said to compress without overlap).
 *
 * Entry j of a sequence covers the w raw positions [j*m - (w-m), j*m + m)
 * that are >= 0; window position p = t - (j*m - (w-m)). For every channel c:
 *   y[j, c] = sum_p softmax_p(z[t_p, c] + pos_bias[p, c]) * x[t_p, c].
 * Entries first_entry .. first_entry + n_entries - 1 are written to rows
 * out_row0 .. of `out`; a split output gets a per-row scale
 * 2^e, e the smallest integer (>= -126) with max|y[j, :d_nope]| <= 448 * 2^e,
 * and E4M3 codes RNE(y / 2^e); bf16 outputs round to nearest even. An MXFP4
 * output (OCP MX conversion) takes per block of 32 channels the scale 2^e,
 * e = floor(log2 max|y|) - 2 clamped below at -127 (-127 for a zero block),
 * and E2M1 codes of y / 2^e rounded to nearest, ties to the even code,
 * saturating at 6; zero magnitudes encode as +0.
 *
 * raw:     [n_rows, D] of raw_dtype (HCA_F32 or HCA_BF16), row stride
 *          raw_row_stride elements; row r holds absolute position first_pos+r.
 * logits:  same dtype as raw; element (r, c) at
 *          logits + r * logit_row_stride + c * logit_col_stride; a column
 *          stride of 0 means one logit per token (1 is the only other value).
 * pos_bias: float32 [w, D], contiguous.
 * Requires 1 <= m <= w <= 1024; the raw rows must cover every position the
 * requested entries read (HCA_ERR_INVALID_ARG otherwise); D <= 1024 (bf16)
 * or 512 (f32), D a multiple of 8 (bf16) or 4 (f32), d_nope likewise;
 * out_row0 + n_entries <= out->n_rows.
 * Output layouts: HCA_LAYOUT_F32, HCA_LAYOUT_BF16, HCA_LAYOUT_SPLIT,
 * HCA_LAYOUT_MXFP4 (the indexer keys: the efficiency paragraph's FP4
 * indexer applied to compressed 64-dim keys).
 */
int csa_compress(const void* raw, int32_t raw_dtype, int64_t raw_row_stride, int64_t n_rows,
                 int64_t first_pos, const void* logits, int64_t logit_row_stride,
                 int64_t logit_col_stride, const float* pos_bias, int32_t m, int32_t w,
                 int64_t first_entry, int64_t n_entries, const hca_store* out, int64_t out_row0,
                 void* stream);

/*
 * hca_compress — HCA compressor (HCA paragraph: every m' tokens merge into
 * one entry, without overlap). Identical to csa_compress with w = m = m_prime:
 * entry j covers [j*m', (j+1)*m'); pos_bias is float32 [m_prime, D].
 */
int hca_compress(const void* raw, int32_t raw_dtype, int64_t raw_row_stride, int64_t n_rows,
                 int64_t first_pos, const void* logits, int64_t logit_row_stride,
                 int64_t logit_col_stride, const float* pos_bias, int32_t m_prime,
                 int64_t first_entry, int64_t n_entries, const hca_store* out, int64_t out_row0,
                 void* stream);

/*
 * One layer's decode-time state (CSA paragraph: an entry per m tokens and a
 * lightning indexer over the entries; HCA paragraph: an entry per m' tokens,
 * no overlap; both: a sliding window of the last W raw tokens).
 *
 * Raw ring: per sequence b, R rows (R >= w and R >= m_prime) of the raw
 * inputs of its last R tokens, the token at position p in row b * R + p % R
 * of each ring array (bf16, row-contiguous: D elements per row for x and the
 * two logit rings, d_idx for the indexer-key rings).
 * Window store: the last W raw tokens in the store's layout (F32, BF16 or
 * SPLIT), the token at position p written to rows win_row_begin[b] + p % W
 * and win_row_begin[b] + p % W + W, with win_pos0[b] kept at
 * W * floor(max(0, t - W + 1) / W) once the token at t is in: position p of
 * the window is then row win_row_begin[b] + p - win_pos0[b], which is how
 * csa_sparse_mqa_attn / hca_dense_mqa_attn read the window.
 * HCA state: the softmax over an HCA entry's window runs in blocks of 8
 * positions; decode_append folds each block at the step that completes it
 * into hca_state (per channel: running max, sum and weighted sum) and writes
 * the entry at its last block, the same arithmetic as hca_compress.
 * Entry stores: CSA entry j of sequence b goes to row csa_row_begin[b] + j
 * of `csa`, HCA entry j to hca_row_begin[b] + j of `hca`, the indexer key of
 * CSA entry j (the CSA compressor with w, m on d_idx channels, then encoded
 * in `idx`'s layout, normally MXFP4) to idx_row_begin[b] + j of `idx`.
 * All pointers are device pointers; the struct lives in host memory.
 */
typedef struct hca_decode_layer {
  int32_t m, w, m_prime, W;
  int32_t R;             /* ring rows per sequence */
  int32_t d_idx;         /* indexer key width; 0 = no indexer keys */
  const float* bias_csa; /* [w, D] */
  const float* bias_hca; /* [m_prime, D] */
  const float* bias_idx; /* [w, d_idx] */
  void* ring_x;          /* bf16 [B * R, D]: raw KV */
  void* ring_z_csa;      /* bf16 [B * R, D]: CSA compression logits */
  void* ring_z_hca;      /* bf16 [B * R, D]: HCA compression logits */
  void* ring_k_idx;      /* bf16 [B * R, d_idx]: raw indexer keys */
  void* ring_z_idx;      /* bf16 [B * R, d_idx]: indexer-key compression logits */
  float* hca_state;      /* float32 [B, 3, D]: the HCA entry in progress (scratch; no
                            initialisation needed) */
  hca_store window;
  const int64_t* win_row_begin; /* [B] */
  int64_t* win_pos0;            /* [B], written */
  hca_store csa;
  const int64_t* csa_row_begin; /* [B] */
  hca_store hca;
  const int64_t* hca_row_begin; /* [B] */
  hca_store idx;
  const int64_t* idx_row_begin; /* [B] */
} hca_decode_layer;

/*
 * decode_append — one decode step of the layer's compression state: for
 * every sequence b with pos[b] >= 0, the token at t = pos[b] (row b of x,
 * z_csa, z_hca [B, D] and of k_idx, z_idx [B, d_idx], bf16, contiguous) goes
 * into the raw ring and the window store (win_pos0[b] updated); if
 * (t+1) % m == 0 it emits CSA entry j = (t+1)/m - 1 and its indexer key,
 * and if (t+1) % m_prime == 0 HCA entry (t+1)/m_prime - 1, each equal to
 * what csa_compress / hca_compress write for that entry from the whole
 * sequence (same arithmetic in the same order). Sequences with pos[b] < 0
 * are left untouched (an idle slot of the batch).
 * Preconditions (device contents): tokens of a sequence arrive in order,
 * one per call, starting at position 0 or with the ring already holding the
 * previous R - 1 positions and hca_state the blocks of the HCA entry in
 * progress (none when t is a multiple of m_prime). Rows past a store's
 * n_rows are not written (an entry or window row beyond it is dropped).
 * Requires B >= 1; the window, csa and hca stores of one width D (a multiple
 * of 8, <= 1024), window layout F32, BF16 or SPLIT, entry stores in any
 * layout csa_compress writes; d_idx == 0 or a multiple of 8 (of 32 for an
 * MXFP4 idx store) <= 1024; 1 <= m <= w; 1 <= m_prime; R >= max(w, m_prime);
 * W >= 1. k_idx, z_idx, bias_idx, the indexer rings and idx are unused when
 * d_idx == 0.
 */
int decode_append(const hca_decode_layer* layer, int32_t B, const int64_t* pos, const void* x,
                  const void* z_csa, const void* z_hca, const void* k_idx, const void* z_idx,
                  void* stream);

/*
 * lightning_index_topk — the lightning indexer (CSA paragraph: it selects
 * the top-k compressed KV entries for core attention; efficiency paragraph:
 * FP4 indexer).
 *
 * For query i in sequence b = q_seq[i] at position t = q_pos[i], the
 * visible entries are j < n_vis = floor((t+1)/m) (entry j's last raw
 * position (j+1)m-1 must be <= t) and, with a document mask (q_lo not NULL,
 * lo = q_lo[i] > 0: packed sequences, the query's document starting at raw
 * position lo), only entries whose window [j*m - (w-m), (j+1)*m) starts at or
 * after lo, i.e. j >= j_lo = ceil((lo + w - m) / m); and
 *   s[j] = sum_h w_idx[i, h] * max(0, <q_idx[i, h, :], k_idx[k_row_begin[b] + j, :]>).
 * out_idx[i, :] receives the k visible entries with the largest s (ties to
 * the lower j; all of them if at most k are visible) in ascending order of
 * j, padded with -1.
 *
 * idx_dtype HCA_F32 / HCA_BF16: q_idx [nq, H, d] and k_idx [k_rows, d]
 *   elements, contiguous; scores accumulate in float32.
 * idx_dtype HCA_MXFP4: q_idx [nq, H, d/2] and k_idx [k_rows, d/2] packed
 *   E2M1 bytes (element 2i in the low nibble of byte i), q_idx_scale
 *   [nq, H, d/32] and k_idx_scale [k_rows, d/32] E8M0 bytes. Each per-head
 *   dot product is then exact in float32 provided, per head, the summed
 *   block exponents of q and key differ by at most 10 between the two
 *   blocks; the score is defined bit-exactly as s = w0*r0, then
 *   s = s + w_h*r_h in head order, each product and sum rounded to float32
 *   (no fused multiply-add).
 * w_idx: float32 [nq, H]. q_lo: int64 [nq] or NULL (no document mask); w is
 * the CSA window (used with q_lo only). Requires d == 64, 1 <= H <= 8,
 * 1 <= k <= 2048, 1 <= m <= w, 1 <= nq, max_visible <= 2^21
 * (HCA_ERR_UNSUPPORTED beyond).
 * Preconditions: q_seq[i] indexes k_row_begin; every
 * n_vis <= max_visible and k_row_begin[b] + n_vis <= k_rows (reads are
 * clamped to both bounds).
 * Workspace: lightning_index_topk_workspace(nq, max_visible, k) bytes
 * process all queries at once; any ws_bytes >= the value for nq = 1 works
 * (queries are then processed in batches, in order, on `stream`).
 */
size_t lightning_index_topk_workspace(int32_t nq, int64_t max_visible, int32_t k);
int lightning_index_topk(const void* q_idx, const uint8_t* q_idx_scale, const float* w_idx,
                         int32_t n_idx_heads, int32_t d_idx, int32_t idx_dtype, const void* k_idx,
                         const uint8_t* k_idx_scale, int64_t k_rows, const int64_t* k_row_begin,
                         const int32_t* q_seq, const int64_t* q_pos, const int64_t* q_lo,
                         int32_t nq, int64_t max_visible, int32_t m, int32_t w, int32_t k,
                         int32_t* out_idx, void* ws, size_t ws_bytes, void* stream);

/*
 * lightning_index_scores + lightning_index_select — lightning_index_topk in
 * two calls, for callers that run independent work between the scoring and
 * the selection (HCA attention, say, beside the selection and CSA attention
 * on another stream: the selection kernel runs one block per query and
 * leaves most of the GPU free). The two calls take exactly the arguments of
 * lightning_index_topk; lightning_index_scores enqueues the scores and
 * leaves every query's candidates in `ws`, and lightning_index_select,
 * enqueued after it on `stream` with the same arguments and workspace,
 * writes out_idx. Together they equal lightning_index_topk. The workspace
 * must hold all nq queries at once (lightning_index_topk_workspace(nq,
 * max_visible, k) bytes; HCA_ERR_WORKSPACE otherwise), and nothing else may
 * write it between the two calls.
 */
int lightning_index_scores(const void* q_idx, const uint8_t* q_idx_scale, const float* w_idx,
                           int32_t n_idx_heads, int32_t d_idx, int32_t idx_dtype, const void* k_idx,
                           const uint8_t* k_idx_scale, int64_t k_rows, const int64_t* k_row_begin,
                           const int32_t* q_seq, const int64_t* q_pos, const int64_t* q_lo,
                           int32_t nq, int64_t max_visible, int32_t m, int32_t w, int32_t k,
                           int32_t* out_idx, void* ws, size_t ws_bytes, void* stream);
int lightning_index_select(const void* q_idx, const uint8_t* q_idx_scale, const float* w_idx,
                           int32_t n_idx_heads, int32_t d_idx, int32_t idx_dtype, const void* k_idx,
                           const uint8_t* k_idx_scale, int64_t k_rows, const int64_t* k_row_begin,
                           const int32_t* q_seq, const int64_t* q_pos, const int64_t* q_lo,
                           int32_t nq, int64_t max_visible, int32_t m, int32_t w, int32_t k,
                           int32_t* out_idx, void* ws, size_t ws_bytes, void* stream);

/*
 * lightning_index_select_pending — lightning_index_select recorded instead of
 * enqueued (CSA paragraph: the indexer's top-k selection), for a call that
 * runs it inside its own launch: hca_dense_mqa_attn_partials_select. It takes
 * lightning_index_select's arguments (stream unused) plus `out`, a host
 * struct it fills (opaque contents: the validated arguments). Nothing is
 * enqueued. The recorded selection reads the workspace that
 * lightning_index_scores left and writes out_idx when it runs; the workspace,
 * out_idx and the query arrays must stay valid and unchanged until then.
 * Errors as lightning_index_select (out untouched on error; NULL out:
 * HCA_ERR_INVALID_ARG).
 */
typedef struct hca_pending_select {
  uint64_t opaque[48];
} hca_pending_select;
int lightning_index_select_pending(const void* q_idx, const uint8_t* q_idx_scale, const float* w_idx,
                                   int32_t n_idx_heads, int32_t d_idx, int32_t idx_dtype,
                                   const void* k_idx, const uint8_t* k_idx_scale, int64_t k_rows,
                                   const int64_t* k_row_begin, const int32_t* q_seq,
                                   const int64_t* q_pos, const int64_t* q_lo, int32_t nq,
                                   int64_t max_visible, int32_t m, int32_t w, int32_t k,
                                   int32_t* out_idx, void* ws, size_t ws_bytes, void* stream,
                                   hca_pending_select* out);

/*
 * csa_sparse_mqa_attn — CSA core attention (CSA paragraph: MQA with shared
 * keys and values over the selected entries; HCA paragraph: plus a
 * sliding-window branch).
 *
 * For query i (sequence b, position t) and every head h, one softmax over
 * the set E = {cache row cache_row_begin[b] + idx[i, r] : r < k, idx >= 0}
 * U {window row win_row_begin[b] + (p - win_pos0[b]) :
 *     max(0, lo, t-W+1) <= p <= t}, with K = V = the stored row (all D dims);
 * lo = q_lo[i] is the first raw position of the query's document in a packed
 * sequence (q_lo NULL: no document mask, lo = 0):
 *   o[i, h] = sum_e softmax_e(scale * <q[i, h], e>) e,
 *   lse[i, h] = log sum_e exp(scale * <q[i, h], e>)  (natural log).
 * An empty set gives o = 0, lse = -inf.
 *
 * q: [nq, n_heads, D] of q_dtype, contiguous. o: [nq, n_heads, D] of o_dtype,
 * contiguous. lse: float32 [nq, n_heads].
 * Supported: q, o, cache, window all F32 with D <= 512, n_heads * D <= 8192
 * and 4 * (n_heads * D + 16 * D + 19 * n_heads) <= 162816 (the vector path's
 * LDS; e.g. 16 heads of 512); or q BF16, o BF16 or F32, cache and window
 * BF16 or SPLIT with D = 512, n_heads a multiple of 16. Anything else:
 * HCA_ERR_UNSUPPORTED. k == 0 selects no compressed entry (idx is not read).
 * Preconditions: idx entries are distinct and < the sequence's stored entry
 * count; win_pos0[b] <= max(0, t-W+1); the window rows exist.
 * Workspace: mqa_attn_workspace(q_dtype, nq, n_heads, D, k + W) bytes (the
 * split-K partials; 0 when one block per query and head group suffices).
 */
size_t mqa_attn_workspace(int32_t q_dtype, int32_t nq, int32_t n_heads, int32_t d,
                          int64_t max_entries);
int csa_sparse_mqa_attn(const void* q, int32_t q_dtype, int32_t nq, int32_t n_heads,
                        const hca_store* cache, const int64_t* cache_row_begin,
                        const int32_t* idx, int32_t k, const hca_store* window,
                        const int64_t* win_row_begin, const int64_t* win_pos0, int32_t W,
                        const int32_t* q_seq, const int64_t* q_pos, const int64_t* q_lo, float scale,
                        void* o, int32_t o_dtype, float* lse, void* ws, size_t ws_bytes,
                        void* stream);

/*
 * hca_dense_mqa_attn — HCA core attention (HCA paragraph: dense attention
 * over all heavily compressed entries plus the sliding-window branch).
 * As csa_sparse_mqa_attn, with the compressed part of E being every visible
 * entry j < n_vis = min(floor((t+1)/m_prime), max_visible) whose window
 * [j*m_prime, (j+1)*m_prime) starts at or after lo (j >= ceil(lo / m_prime)):
 * cache rows cache_row_begin[b] + j.
 * Workspace: mqa_attn_workspace(q_dtype, nq, n_heads, D, max_visible + W) bytes.
 */
int hca_dense_mqa_attn(const void* q, int32_t q_dtype, int32_t nq, int32_t n_heads,
                       const hca_store* cache, const int64_t* cache_row_begin, int32_t m_prime,
                       int64_t max_visible, const hca_store* window, const int64_t* win_row_begin,
                       const int64_t* win_pos0, int32_t W, const int32_t* q_seq,
                       const int64_t* q_pos, const int64_t* q_lo, float scale, void* o,
                       int32_t o_dtype, float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * Deferred merge of the split-K partials (both mechanisms end in one joint
 * softmax per query and head; CSA and HCA paragraphs: the compressed part and
 * the sliding-window branch). A call may split each query's entry list into
 * ranges whose normalised partial outputs and log-sum-exps are merged by
 * log-sum-exp. csa_sparse_mqa_attn_partials / hca_dense_mqa_attn_partials
 * take the same arguments as csa_sparse_mqa_attn / hca_dense_mqa_attn plus
 * `out`, run the attention and stop before that merge: when the call splits
 * (out->n_split > 1) its partials stay in ws and o/lse are not written until
 * mqa_attn_merge runs; otherwise o/lse are final and the merge skips the call.
 * mqa_attn_merge(a, b, stream) merges one call (b NULL) or two calls in one
 * launch, giving the same o/lse bits as the undeferred calls. It must run
 * after the partial calls (same stream, or ordered by events) and before
 * their workspaces are reused. hca_attn_partials holds device pointers and
 * sizes filled by the partial calls; the caller keeps it in host memory.
 * Errors as the undeferred calls; bad sizes or NULL pointers in a or b:
 * HCA_ERR_INVALID_ARG.
 */
typedef struct hca_attn_partials {
  float* part_o;    /* [nq][n_split][n_heads][d] float32, inside the call's ws */
  float* part_lse;  /* [nq][n_split][n_heads] float32 */
  void* o;          /* the call's o and lse */
  float* lse;
  int32_t nq, n_heads, d, n_split, o_dtype;
} hca_attn_partials;
int csa_sparse_mqa_attn_partials(const void* q, int32_t q_dtype, int32_t nq, int32_t n_heads,
                                 const hca_store* cache, const int64_t* cache_row_begin,
                                 const int32_t* idx, int32_t k, const hca_store* window,
                                 const int64_t* win_row_begin, const int64_t* win_pos0, int32_t W,
                                 const int32_t* q_seq, const int64_t* q_pos, const int64_t* q_lo,
                                 float scale, void* o, int32_t o_dtype, float* lse, void* ws,
                                 size_t ws_bytes, void* stream, hca_attn_partials* out);
int hca_dense_mqa_attn_partials(const void* q, int32_t q_dtype, int32_t nq, int32_t n_heads,
                                const hca_store* cache, const int64_t* cache_row_begin,
                                int32_t m_prime, int64_t max_visible, const hca_store* window,
                                const int64_t* win_row_begin, const int64_t* win_pos0, int32_t W,
                                const int32_t* q_seq, const int64_t* q_pos, const int64_t* q_lo,
                                float scale, void* o, int32_t o_dtype, float* lse, void* ws,
                                size_t ws_bytes, void* stream, hca_attn_partials* out);
int mqa_attn_merge(const hca_attn_partials* a, const hca_attn_partials* b, void* stream);

/*
 * hca_dense_mqa_attn_partials_select — hca_dense_mqa_attn_partials and a
 * recorded top-k selection (lightning_index_select_pending) enqueued as one
 * unit on `stream` (HCA paragraph: dense attention over the heavily
 * compressed entries; CSA paragraph: the indexer's top-k, which only the
 * later CSA call reads). For a decode step whose HCA call does not depend on
 * the selection: when the HCA call takes the FP8 split-store kernel or the
 * bf16-store MFMA kernel (bf16 queries), the selection's blocks run in the
 * same grid as the attention's (one launch instead of two streams joined by
 * events); otherwise the selection is launched first on the stream. Results are bit-identical to the two calls
 * made separately: out_idx as lightning_index_select writes it, o/lse and the
 * partials as hca_dense_mqa_attn_partials. The selection must not read what
 * the attention writes (its workspace and out_idx are disjoint from the HCA
 * call's ws, o and lse). Errors as hca_dense_mqa_attn_partials; sel NULL or
 * not filled by lightning_index_select_pending: HCA_ERR_INVALID_ARG. An
 * inactive selection (no query, or the streaming indexer path) adds nothing.
 */
int hca_dense_mqa_attn_partials_select(const void* q, int32_t q_dtype, int32_t nq, int32_t n_heads,
                                       const hca_store* cache, const int64_t* cache_row_begin,
                                       int32_t m_prime, int64_t max_visible, const hca_store* window,
                                       const int64_t* win_row_begin, const int64_t* win_pos0,
                                       int32_t W, const int32_t* q_seq, const int64_t* q_pos,
                                       const int64_t* q_lo, float scale, void* o, int32_t o_dtype,
                                       float* lse, void* ws, size_t ws_bytes, void* stream,
                                       const hca_pending_select* sel, hca_attn_partials* out);

/*
 * hca_dense_mqa_attn_noalloc — hca_dense_mqa_attn for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). Same arguments and results as
 * hca_dense_mqa_attn without the workspace: the split-K partials go to a
 * static device array of 16 MiB that the library holds on every GPU it runs
 * on until the process ends. Calls needing more than that
 * (mqa_attn_workspace(q_dtype, nq, n_heads, D, max_visible + W) > 16 MiB)
 * return HCA_ERR_WORKSPACE before anything is enqueued. The call allocates
 * nothing. Every call on one GPU shares that GPU's array: calls that overlap
 * on one GPU (other streams, other threads) race and give unspecified
 * results; calls ordered on one stream do not.
 */
int hca_dense_mqa_attn_noalloc(const void* q, int32_t q_dtype, int32_t nq, int32_t n_heads,
                               const hca_store* cache, const int64_t* cache_row_begin,
                               int32_t m_prime, int64_t max_visible, const hca_store* window,
                               const int64_t* win_row_begin, const int64_t* win_pos0, int32_t W,
                               const int32_t* q_seq, const int64_t* q_pos, const int64_t* q_lo,
                               float scale, void* o, int32_t o_dtype, float* lse, void* stream);

/*
 * grouped_out_proj — the grouped output projection after core attention
 * (CSA paragraph: core attention is followed by a grouped output projection
 * to manage the computational cost). The heads are split into `groups`
 * equal groups of consecutive heads; group g's concatenated head outputs are
 * the k_group = (h / groups) * D values x[r, g*k_group .. (g+1)*k_group - 1]
 * (the attention output [n, h, D] is such an x with ldx = h * D), and
 *   y[r, g*n_group + c] = sum_k x[r, g*k_group + k] * w[g, c, k]
 * with w bf16 [groups, n_group, k_group] (out-features by in-features, per
 * group, contiguous), float32 accumulation, y of y_dtype (HCA_BF16, rounded
 * to nearest even, or HCA_F32) with row stride ldy. x: bf16, row stride ldx
 * (elements). The result is deterministic (fixed summation order).
 * Requires n >= 0, n <= 2^22, 1 <= groups <= 65535, k_group a multiple of 32,
 * n_group a multiple of 16, ldx >= groups * k_group and ldx a multiple of 8,
 * ldy >= groups * n_group, x and w 16-byte aligned, y aligned to its element.
 */
int grouped_out_proj(const void* x, int64_t n, int64_t ldx, int32_t groups, int32_t k_group,
                     const void* w, int32_t n_group, void* y, int32_t y_dtype, int64_t ldy,
                     void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HCA_H_ */
