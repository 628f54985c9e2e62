// C ABI of the hybrid-attention library: argument validation and kernel dispatch.
// Every host-checkable argument is validated before anything is enqueued.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "hca.h"
#include "internal.h"

namespace hca {
hipError_t attention_init();
}

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fn, const char* msg) {
  g_last_error = std::string(fn) + ": " + msg;
  return status;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int ensure_init(const char* fn) {
  static std::once_flag once;
  static hipError_t err = hipSuccess;
  std::call_once(once, [] {
    err = hca::attention_init();
    if (err == hipSuccess) err = hca::index_init();
  });
  if (err != hipSuccess) {
    g_last_error = std::string(fn) + ": HIP init failed: " + hipGetErrorString(err);
    return HCA_ERR_HIP;
  }
  return HCA_OK;
}

int launched(const char* fn, hipError_t e) {
  if (e == hipSuccess) return HCA_OK;
  g_last_error = std::string(fn) + ": launch failed: " + hipGetErrorString(e);
  return HCA_ERR_HIP;
}

// Validates a store view; `what` names it in messages.
int check_store(const char* fn, const hca_store* s, const char* what, std::string* msg) {
  char buf[256];
  auto bad = [&](const char* m) {
    snprintf(buf, sizeof buf, "%s: %s", what, m);
    *msg = buf;
    return HCA_ERR_INVALID_ARG;
  };
  (void)fn;
  if (!s) return bad("NULL store");
  if (s->reserved != 0) return bad("reserved field must be 0");
  if (s->d_nope < 0 || s->d_rope < 0 || s->d_nope + s->d_rope <= 0) return bad("bad d_nope/d_rope");
  if (s->n_rows < 0) return bad("negative n_rows");
  const int64_t D = (int64_t)s->d_nope + s->d_rope;
  switch (s->layout) {
    case HCA_LAYOUT_F32:
    case HCA_LAYOUT_BF16: {
      const int64_t es = s->layout == HCA_LAYOUT_F32 ? 4 : 2;
      if (s->n_rows > 0 && !s->data) return bad("NULL data");
      if (!aligned16(s->data)) return bad("data not 16-byte aligned");
      if (s->row_stride < D) return bad("row_stride < D");
      if ((s->row_stride * es) % 16) return bad("rows not 16-byte aligned");
      return HCA_OK;
    }
    case HCA_LAYOUT_SPLIT:
      if (s->n_rows > 0 && (!s->data || !s->scale || !s->rope)) return bad("NULL data/scale/rope");
      if (!aligned16(s->data) || !aligned16(s->rope)) return bad("data/rope not 16-byte aligned");
      if (s->row_stride < s->d_nope || s->row_stride % 16) return bad("bad FP8 row_stride");
      if (s->rope_stride < s->d_rope || (s->rope_stride * 2) % 16) return bad("bad rope_stride");
      if (s->d_nope % 8 || s->d_rope % 8) return bad("d_nope and d_rope must be multiples of 8");
      return HCA_OK;
    case HCA_LAYOUT_MXFP4:
      if (s->d_rope != 0 || s->d_nope % 32) return bad("MXFP4 rows need d_rope == 0 and d_nope a multiple of 32");
      if (s->n_rows > 0 && (!s->data || !s->rope)) return bad("NULL data/scales (rope)");
      if (!aligned16(s->data)) return bad("data not 16-byte aligned");
      if (s->row_stride < s->d_nope / 2 || s->row_stride % 16) return bad("bad MXFP4 row_stride");
      if (s->rope_stride < s->d_nope / 32) return bad("bad MXFP4 scale stride (rope_stride)");
      return HCA_OK;
    default:
      return bad("unknown layout");
  }
}

hca::StoreView view_of(const hca_store* s) {
  hca::StoreView v;
  v.layout = s->layout;
  v.d_nope = s->d_nope;
  v.d_rope = s->d_rope;
  v.n_rows = s->n_rows;
  v.data = s->data;
  v.row_stride = s->row_stride;
  v.scale = s->scale;
  v.rope = s->rope;
  v.rope_stride = s->rope_stride;
  return v;
}

int compress_impl(const char* fn, const void* raw, int32_t raw_dtype, int64_t raw_row_stride, int64_t n_rows,
                  int64_t first_pos, const void* logits, int64_t logit_row_stride, int64_t logit_col_stride,
                  const float* pos_bias, int32_t m, int32_t w, int64_t first_entry, int64_t n_entries,
                  const hca_store* out, int64_t out_row0, void* stream) {
  if (!raw || !logits || !pos_bias) return fail(HCA_ERR_INVALID_ARG, fn, "NULL raw/logits/pos_bias");
  if (raw_dtype != HCA_F32 && raw_dtype != HCA_BF16) return fail(HCA_ERR_UNSUPPORTED, fn, "raw dtype must be F32 or BF16");
  std::string msg;
  if (check_store(fn, out, "out", &msg) != HCA_OK) return fail(HCA_ERR_INVALID_ARG, fn, msg.c_str());
  if (m < 1 || w < m || w > 1024) return fail(HCA_ERR_INVALID_ARG, fn, "need 1 <= m <= w <= 1024");
  if (n_rows < 0 || first_pos < 0 || first_entry < 0 || n_entries < 0 || out_row0 < 0)
    return fail(HCA_ERR_INVALID_ARG, fn, "negative size or offset");
  const int64_t D = (int64_t)out->d_nope + out->d_rope;
  const int64_t es = raw_dtype == HCA_F32 ? 4 : 2;
  const int64_t vec = 16 / es;
  if (D % vec || out->d_nope % vec) return fail(HCA_ERR_UNSUPPORTED, fn, "D and d_nope must be multiples of 16 bytes of raw");
  if (D > 2 * 64 * vec) return fail(HCA_ERR_UNSUPPORTED, fn, "D too large (1024 bf16 / 512 f32 max)");
  if (raw_row_stride < D || (raw_row_stride * es) % 16) return fail(HCA_ERR_INVALID_ARG, fn, "bad raw_row_stride");
  if (!aligned16(raw) || !aligned16(pos_bias)) return fail(HCA_ERR_INVALID_ARG, fn, "raw/pos_bias not 16-byte aligned");
  if (logit_col_stride != 0 && logit_col_stride != 1) return fail(HCA_ERR_INVALID_ARG, fn, "logit_col_stride must be 0 or 1");
  if (logit_col_stride == 1) {
    if (!aligned16(logits) || logit_row_stride < D || (logit_row_stride * es) % 16)
      return fail(HCA_ERR_INVALID_ARG, fn, "bad logits alignment or row stride");
  } else if (logit_row_stride < 1) {
    return fail(HCA_ERR_INVALID_ARG, fn, "bad logit_row_stride");
  }
  if (out_row0 + n_entries > out->n_rows) return fail(HCA_ERR_INVALID_ARG, fn, "output rows out of range");
  if (n_entries > 0) {
    const int64_t lo = std::max<int64_t>(0, first_entry * m - (w - m));
    const int64_t hi = (first_entry + n_entries) * m;  // exclusive
    if (lo < first_pos || hi > first_pos + n_rows)
      return fail(HCA_ERR_INVALID_ARG, fn, "raw rows do not cover the windows of the requested entries");
  }
  hca::CompressArgs a;
  a.raw = raw; a.raw_stride = raw_row_stride;
  a.logits = logits; a.logit_row_stride = logit_row_stride; a.logit_col_stride = logit_col_stride;
  a.bias = pos_bias;
  a.n_rows = n_rows; a.first_pos = first_pos; a.first_entry = first_entry; a.n_entries = n_entries;
  a.m = m; a.w = w; a.D = (int)D; a.d_nope = out->d_nope;
  a.raw_dtype = raw_dtype; a.out_layout = out->layout;
  a.out = out->data; a.out_stride = out->row_stride; a.out_scale = out->scale;
  a.out_rope = out->rope; a.out_rope_stride = out->rope_stride; a.out_row0 = out_row0;
  return launched(fn, hca::launch_compress(a, static_cast<hipStream_t>(stream)));
}


int decode_impl(const char* fn, const hca_decode_layer* L, int32_t B, const int64_t* pos, const void* x,
                const void* z_csa, const void* z_hca, const void* k_idx, const void* z_idx, void* stream) {
  if (!L || !pos || !x || !z_csa || !z_hca) return fail(HCA_ERR_INVALID_ARG, fn, "NULL argument");
  if (B < 1) return fail(HCA_ERR_INVALID_ARG, fn, "B < 1");
  if (L->m < 1 || L->w < L->m || L->m_prime < 1 || L->W < 1)
    return fail(HCA_ERR_INVALID_ARG, fn, "need 1 <= m <= w, m_prime >= 1, W >= 1");
  if (L->R < L->w || L->R < L->m_prime) return fail(HCA_ERR_INVALID_ARG, fn, "ring rows R < max(w, m_prime)");
  if (L->w > 1024 || L->m_prime > 1024) return fail(HCA_ERR_INVALID_ARG, fn, "window longer than 1024");
  std::string msg;
  if (check_store(fn, &L->window, "window", &msg) != HCA_OK || check_store(fn, &L->csa, "csa", &msg) != HCA_OK ||
      check_store(fn, &L->hca, "hca", &msg) != HCA_OK)
    return fail(HCA_ERR_INVALID_ARG, fn, msg.c_str());
  if (L->window.layout == HCA_LAYOUT_MXFP4) return fail(HCA_ERR_UNSUPPORTED, fn, "window layout must be F32, BF16 or SPLIT");
  const int64_t D = (int64_t)L->csa.d_nope + L->csa.d_rope;
  if ((int64_t)L->window.d_nope + L->window.d_rope != D || (int64_t)L->hca.d_nope + L->hca.d_rope != D)
    return fail(HCA_ERR_INVALID_ARG, fn, "window, csa and hca widths differ");
  for (const hca_store* s : {&L->window, &L->csa, &L->hca})
    if (s->d_nope % 8) return fail(HCA_ERR_UNSUPPORTED, fn, "d_nope must be a multiple of 8");
  if (D % 8 || D > 1024) return fail(HCA_ERR_UNSUPPORTED, fn, "D must be a multiple of 8, at most 1024");
  const int64_t di = L->d_idx;
  if (di < 0 || di % 8 || di > 1024) return fail(HCA_ERR_UNSUPPORTED, fn, "d_idx must be 0 or a multiple of 8 <= 1024");
  if (!L->bias_csa || !L->bias_hca || !L->ring_x || !L->ring_z_csa || !L->ring_z_hca || !L->hca_state || !L->win_row_begin ||
      !L->win_pos0 || !L->csa_row_begin || !L->hca_row_begin)
    return fail(HCA_ERR_INVALID_ARG, fn, "NULL field of the layer");
  for (const void* p : {(const void*)L->bias_csa, (const void*)L->bias_hca, (const void*)L->ring_x,
                        (const void*)L->ring_z_csa, (const void*)L->ring_z_hca, (const void*)L->hca_state, x,
                        z_csa, z_hca})
    if (!aligned16(p)) return fail(HCA_ERR_INVALID_ARG, fn, "inputs, rings and biases must be 16-byte aligned");
  if (di > 0) {
    if (!k_idx || !z_idx || !L->bias_idx || !L->ring_k_idx || !L->ring_z_idx || !L->idx_row_begin)
      return fail(HCA_ERR_INVALID_ARG, fn, "NULL indexer-key argument");
    if (check_store(fn, &L->idx, "idx", &msg) != HCA_OK) return fail(HCA_ERR_INVALID_ARG, fn, msg.c_str());
    if ((int64_t)L->idx.d_nope + L->idx.d_rope != di) return fail(HCA_ERR_INVALID_ARG, fn, "idx width != d_idx");
    if (L->idx.d_nope % 8) return fail(HCA_ERR_UNSUPPORTED, fn, "idx d_nope must be a multiple of 8");
    for (const void* p : {(const void*)L->bias_idx, (const void*)L->ring_k_idx, (const void*)L->ring_z_idx, k_idx, z_idx})
      if (!aligned16(p)) return fail(HCA_ERR_INVALID_ARG, fn, "indexer inputs, rings and bias must be 16-byte aligned");
  }
  hca::DecodeArgs a;
  a.B = B;
  a.pos = pos;
  a.x = static_cast<const uint16_t*>(x);
  a.zc = static_cast<const uint16_t*>(z_csa);
  a.zh = static_cast<const uint16_t*>(z_hca);
  a.ki = static_cast<const uint16_t*>(k_idx);
  a.zi = static_cast<const uint16_t*>(z_idx);
  a.m = L->m; a.w = L->w; a.m_prime = L->m_prime; a.W = L->W; a.R = L->R; a.D = (int)D; a.d_idx = (int)di;
  a.bias_csa = L->bias_csa; a.bias_hca = L->bias_hca; a.bias_idx = L->bias_idx;
  a.ring_x = static_cast<uint16_t*>(L->ring_x);
  a.ring_zc = static_cast<uint16_t*>(L->ring_z_csa);
  a.ring_zh = static_cast<uint16_t*>(L->ring_z_hca);
  a.ring_ki = static_cast<uint16_t*>(L->ring_k_idx);
  a.ring_zi = static_cast<uint16_t*>(L->ring_z_idx);
  a.hca_state = L->hca_state;
  a.win = view_of(&L->window);
  a.csa = view_of(&L->csa);
  a.hca = view_of(&L->hca);
  a.idx = di > 0 ? view_of(&L->idx) : a.csa;
  a.win_rb = L->win_row_begin;
  a.win_pos0 = L->win_pos0;
  a.csa_rb = L->csa_row_begin;
  a.hca_rb = L->hca_row_begin;
  a.idx_rb = di > 0 ? L->idx_row_begin : L->csa_row_begin;
  return launched(fn, hca::launch_decode_append(a, static_cast<hipStream_t>(stream)));
}

size_t index_ws(int64_t nq, int64_t max_visible) { return hca::index_ws_layout(nq, max_visible, nullptr, nullptr); }

uint8_t* align256(uint8_t* p) { return reinterpret_cast<uint8_t*>((reinterpret_cast<uintptr_t>(p) + 255) & ~uintptr_t(255)); }

// Split-K workspace of a launch: partial outputs [nq, n_split, H, D] and lse [nq, n_split, H]
// (float32). `wide`: the 64-head kernel's policy, else the other kernels'.
size_t attn_ws(int q_dtype, int64_t nq, int H, int D, int64_t max_entries, bool wide, int* n_split, int* per) {
  if (wide) hca::attn_split_policy_wide((int)nq, H, max_entries, n_split, per);
  else hca::attn_split_policy((int)nq, H, D, max_entries, q_dtype == HCA_BF16, n_split, per);
  if (*n_split <= 1) return 0;
  return 512 + (size_t)nq * (size_t)(*n_split) * (size_t)H * ((size_t)D + 1) * 4;
}

// Workspace for any store layout: the larger of the two policies where the 64-head kernel may run.
size_t attn_ws_any(int q_dtype, int64_t nq, int H, int D, int64_t max_entries) {
  int n_split, per;
  size_t need = attn_ws(q_dtype, nq, H, D, max_entries, false, &n_split, &per);
  if (q_dtype == HCA_BF16 && H % 64 == 0 && nq >= 64)
    need = std::max(need, attn_ws(q_dtype, nq, H, D, max_entries, true, &n_split, &per));
  return need;
}

int attn_impl(const char* fn, bool csa, const void* q, int32_t q_dtype, int32_t nq, int32_t n_heads,
              const hca_store* cache, const int64_t* cache_row_begin, const int32_t* idx, int32_t k,
              int32_t m_prime, int64_t max_visible, const hca_store* window, const int64_t* win_row_begin,
              const int64_t* win_pos0, int32_t W, const int32_t* q_seq, const int64_t* q_pos,
              const int64_t* q_lo, float scale,
              void* o, int32_t o_dtype, float* lse, void* ws, size_t ws_bytes, void* stream,
              bool static_scratch = false, hca_attn_partials* defer = nullptr,
              const hca::IndexArgs* sel = nullptr) {
  if (!q || !cache_row_begin || !win_row_begin || !win_pos0 || !q_seq || !q_pos || !o || !lse)
    return fail(HCA_ERR_INVALID_ARG, fn, "NULL argument");
  if (csa && k > 0 && !idx) return fail(HCA_ERR_INVALID_ARG, fn, "NULL idx");
  if (nq < 0 || n_heads < 1 || W < 0) return fail(HCA_ERR_INVALID_ARG, fn, "bad nq/n_heads/W");
  if (csa && (k < 0 || k > 65536)) return fail(HCA_ERR_INVALID_ARG, fn, "k out of range");
  if (!csa && (m_prime < 1 || max_visible < 0)) return fail(HCA_ERR_INVALID_ARG, fn, "bad m_prime/max_visible");
  if (!std::isfinite(scale)) return fail(HCA_ERR_INVALID_ARG, fn, "non-finite scale");
  std::string msg;
  if (check_store(fn, cache, "cache", &msg) != HCA_OK) return fail(HCA_ERR_INVALID_ARG, fn, msg.c_str());
  if (check_store(fn, window, "window", &msg) != HCA_OK) return fail(HCA_ERR_INVALID_ARG, fn, msg.c_str());
  if (cache->d_nope != window->d_nope || cache->d_rope != window->d_rope)
    return fail(HCA_ERR_INVALID_ARG, fn, "cache and window widths differ");
  if (!aligned16(q) || !aligned16(o) || (reinterpret_cast<uintptr_t>(lse) & 3))
    return fail(HCA_ERR_INVALID_ARG, fn, "q/o not 16-byte aligned");
  const int D = cache->d_nope + cache->d_rope;
  const hca::StoreView cv = view_of(cache), wv = view_of(window);
  const bool mfma = hca::attn_mfma_supported(q_dtype, o_dtype, cv, wv, n_heads, D);
  if (!mfma) {
    const bool valu = q_dtype == HCA_F32 && o_dtype == HCA_F32 && cache->layout == HCA_LAYOUT_F32 &&
                      window->layout == HCA_LAYOUT_F32 && D <= 512 && (int64_t)n_heads * D <= 8192 &&
                      hca::attn_valu_lds_bytes(n_heads, D) <= hca::kAttnValuMaxLds;
    if (!valu) return fail(HCA_ERR_UNSUPPORTED, fn, "unsupported dtype/layout/shape combination");
  }
  if (defer) *defer = hca_attn_partials{nullptr, nullptr, o, lse, 0, n_heads, D, 1, o_dtype};
  if (nq == 0) {
    if (!sel) return HCA_OK;
    const int st = ensure_init(fn);
    if (st != HCA_OK) return st;
    return launched(fn, hca::launch_index_topk(*sel, false, true, static_cast<hipStream_t>(stream)));
  }
  const int64_t max_entries = (csa ? (int64_t)k : max_visible) + W;
  int n_split = 1, per = 1;
  const bool wide = hca::attn_wide_supported(q_dtype, cv, wv, n_heads, nq);
  const size_t need = attn_ws(q_dtype, nq, n_heads, D, max_entries, wide, &n_split, &per);
  if (static_scratch) {
    // the library's static device scratch stands in for the workspace (no allocation)
    if (need > hca::kNoallocScratchBytes)
      return fail(HCA_ERR_WORKSPACE, fn, "the call needs more than the 16 MiB static scratch (mqa_attn_workspace)");
    ws = nullptr;
    ws_bytes = 0;
    if (need > 0) {
      const hipError_t e = hca::noalloc_scratch(&ws);
      if (e != hipSuccess) {
        g_last_error = std::string(fn) + ": static scratch lookup failed: " + hipGetErrorString(e);
        return HCA_ERR_HIP;
      }
      ws_bytes = hca::kNoallocScratchBytes;
    }
  }
  if (need > 0 && (!ws || ws_bytes < need)) return fail(HCA_ERR_WORKSPACE, fn, "workspace too small");
  int st = ensure_init(fn);
  if (st != HCA_OK) return st;
  hca::AttnArgs a;
  a.q = q; a.q_dtype = q_dtype; a.nq = nq; a.H = n_heads; a.D = D;
  a.cache = cv; a.win = wv;
  a.cache_row_begin = cache_row_begin;
  // k == 0 selects nothing: the call runs as the dense path over no compressed entries (the
  // window only), so no kernel ever reads idx, whatever the pointer
  a.idx = (csa && k > 0) ? idx : nullptr;
  a.k = (csa && k > 0) ? k : 0;
  a.m_prime = csa ? 1 : m_prime;
  a.max_visible = csa ? 0 : max_visible;
  a.win_row_begin = win_row_begin; a.win_pos0 = win_pos0; a.W = W;
  a.q_seq = q_seq; a.q_pos = q_pos; a.q_lo = q_lo; a.scale = scale;
  a.o = o; a.o_dtype = o_dtype; a.lse = lse;
  a.n_split = n_split; a.per_split = per;
  a.part_o = nullptr; a.part_lse = nullptr;
  if (n_split > 1) {
    uint8_t* p = align256(static_cast<uint8_t*>(ws));
    a.part_o = reinterpret_cast<float*>(p);
    a.part_lse = a.part_o + (size_t)nq * n_split * n_heads * D;
  }
  if (defer) *defer = hca_attn_partials{a.part_o, a.part_lse, o, lse, nq, n_heads, D, n_split, o_dtype};
  return launched(fn, hca::launch_attention(a, static_cast<hipStream_t>(stream), /*combine=*/defer == nullptr, sel));
}

int check_partials(const char* fn, const hca_attn_partials* p, const char* which) {
  std::string m = std::string(which) + ": ";
  if (p->nq < 0 || p->n_heads < 1 || p->d < 1 || p->n_split < 1) return fail(HCA_ERR_INVALID_ARG, fn, (m + "bad sizes").c_str());
  if (p->o_dtype != HCA_BF16 && p->o_dtype != HCA_F32) return fail(HCA_ERR_INVALID_ARG, fn, (m + "bad o_dtype").c_str());
  if (p->nq > 0 && (!p->o || !p->lse)) return fail(HCA_ERR_INVALID_ARG, fn, (m + "NULL output").c_str());
  if (p->nq > 0 && p->n_split > 1 && (!p->part_o || !p->part_lse))
    return fail(HCA_ERR_INVALID_ARG, fn, (m + "NULL partials").c_str());
  return HCA_OK;
}

hca::MergeArgs merge_of(const hca_attn_partials* p) {
  hca::MergeArgs m;
  m.part_o = p->part_o;
  m.part_lse = p->part_lse;
  m.o = p->o;
  m.lse = p->lse;
  m.nq = p->nq;
  m.H = p->n_heads;
  m.D = p->d;
  m.n_split = p->n_split;
  m.o_dtype = p->o_dtype;
  return m;
}

}  // namespace

extern "C" {
#define HCA_EXPORT __attribute__((visibility("default")))

HCA_EXPORT int hca_abi_version(void) { return HCA_ABI_VERSION; }

HCA_EXPORT int grouped_out_proj(const void* x, int64_t n, int64_t ldx, int32_t groups, int32_t k_group, const void* w,
                                int32_t n_group, void* y, int32_t y_dtype, int64_t ldy, void* stream) {
  const char* fn = "grouped_out_proj";
  if (!x || !w || !y) return fail(HCA_ERR_INVALID_ARG, fn, "NULL argument");
  if (n < 0 || n > ((int64_t)1 << 22)) return fail(HCA_ERR_INVALID_ARG, fn, "n out of range");
  if (groups < 1 || groups > 65535) return fail(HCA_ERR_INVALID_ARG, fn, "groups out of range");
  if (k_group < 32 || k_group % 32) return fail(HCA_ERR_UNSUPPORTED, fn, "k_group must be a multiple of 32");
  if (n_group < 16 || n_group % 16) return fail(HCA_ERR_UNSUPPORTED, fn, "n_group must be a multiple of 16");
  if (y_dtype != HCA_BF16 && y_dtype != HCA_F32) return fail(HCA_ERR_UNSUPPORTED, fn, "y dtype must be BF16 or F32");
  if (ldx < (int64_t)groups * k_group || ldx % 8) return fail(HCA_ERR_INVALID_ARG, fn, "bad ldx");
  if (ldy < (int64_t)groups * n_group) return fail(HCA_ERR_INVALID_ARG, fn, "bad ldy");
  if (!aligned16(x) || !aligned16(w)) return fail(HCA_ERR_INVALID_ARG, fn, "x/w not 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(y) % (y_dtype == HCA_F32 ? 4 : 2)) return fail(HCA_ERR_INVALID_ARG, fn, "y misaligned");
  if (n == 0) return HCA_OK;
  hca::ProjArgs a;
  a.x = static_cast<const uint16_t*>(x);
  a.ldx = ldx;
  a.w = static_cast<const uint16_t*>(w);
  a.y = y;
  a.ldy = ldy;
  a.n = n;
  a.G = groups;
  a.Kg = k_group;
  a.Ng = n_group;
  a.y_dtype = y_dtype;
  return launched(fn, hca::launch_proj(a, static_cast<hipStream_t>(stream)));
}

HCA_EXPORT int decode_append(const hca_decode_layer* layer, int32_t B, const int64_t* pos, const void* x,
                             const void* z_csa, const void* z_hca, const void* k_idx, const void* z_idx,
                             void* stream) {
  return decode_impl("decode_append", layer, B, pos, x, z_csa, z_hca, k_idx, z_idx, stream);
}

HCA_EXPORT const char* hca_status_string(int status) {
  switch (status) {
    case HCA_OK: return "ok";
    case HCA_ERR_INVALID_ARG: return "invalid argument";
    case HCA_ERR_UNSUPPORTED: return "unsupported dtype/layout/shape combination";
    case HCA_ERR_WORKSPACE: return "workspace too small";
    case HCA_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

HCA_EXPORT const char* hca_last_error(void) { return g_last_error.c_str(); }

HCA_EXPORT int csa_compress(const void* raw, int32_t raw_dtype, int64_t raw_row_stride, int64_t n_rows, int64_t first_pos,
                 const void* logits, int64_t logit_row_stride, int64_t logit_col_stride, const float* pos_bias,
                 int32_t m, int32_t w, int64_t first_entry, int64_t n_entries, const hca_store* out,
                 int64_t out_row0, void* stream) {
  return compress_impl("csa_compress", raw, raw_dtype, raw_row_stride, n_rows, first_pos, logits, logit_row_stride,
                       logit_col_stride, pos_bias, m, w, first_entry, n_entries, out, out_row0, stream);
}

HCA_EXPORT int hca_compress(const void* raw, int32_t raw_dtype, int64_t raw_row_stride, int64_t n_rows, int64_t first_pos,
                 const void* logits, int64_t logit_row_stride, int64_t logit_col_stride, const float* pos_bias,
                 int32_t m_prime, int64_t first_entry, int64_t n_entries, const hca_store* out,
                 int64_t out_row0, void* stream) {
  return compress_impl("hca_compress", raw, raw_dtype, raw_row_stride, n_rows, first_pos, logits, logit_row_stride,
                       logit_col_stride, pos_bias, m_prime, m_prime, first_entry, n_entries, out, out_row0, stream);
}

HCA_EXPORT size_t lightning_index_topk_workspace(int32_t nq, int64_t max_visible, int32_t k) {
  (void)k;
  if (nq < 0 || max_visible < 0) return 0;
  return index_ws(nq, max_visible);
}

}  // extern "C"

namespace {

// The indexer's two phases: kIndexBoth (lightning_index_topk), kIndexScores or kIndexSelect
// (the split calls, which keep every query's intermediate state in the workspace in between
// and so need the workspace of all nq queries at once).
enum IndexPhase { kIndexBoth = 0, kIndexScores = 1, kIndexSelect = 2, kIndexPending = 3 };

// What lightning_index_select_pending records in a hca_pending_select.
struct PendingSelect {
  uint64_t magic;  // kPendingMagic once recorded
  int32_t active;  // 0: the selection has nothing to launch (no query, or the streaming path)
  int32_t pad;
  hca::IndexArgs a;
};
constexpr uint64_t kPendingMagic = 0x5345'4c45'4354'3031ull;
static_assert(sizeof(PendingSelect) <= sizeof(hca_pending_select), "hca_pending_select too small");

int index_impl(const char* fn, int phase, const void* q_idx, const uint8_t* q_idx_scale, const float* w_idx,
               int32_t n_idx_heads, int32_t d_idx, int32_t idx_dtype, const void* k_idx,
               const uint8_t* k_idx_scale, int64_t k_rows, const int64_t* k_row_begin, const int32_t* q_seq,
               const int64_t* q_pos, const int64_t* q_lo, int32_t nq, int64_t max_visible, int32_t m, int32_t w,
               int32_t k, int32_t* out_idx, void* ws, size_t ws_bytes, void* stream,
               PendingSelect* pending = nullptr) {
  if (!q_idx || !w_idx || !k_idx || !k_row_begin || !q_seq || !q_pos || !out_idx)
    return fail(HCA_ERR_INVALID_ARG, fn, "NULL argument");
  if (idx_dtype != HCA_F32 && idx_dtype != HCA_BF16 && idx_dtype != HCA_MXFP4)
    return fail(HCA_ERR_UNSUPPORTED, fn, "indexer dtype must be F32, BF16 or MXFP4");
  if (idx_dtype == HCA_MXFP4 && (!q_idx_scale || !k_idx_scale)) return fail(HCA_ERR_INVALID_ARG, fn, "NULL MXFP4 scales");
  if (d_idx != 64) return fail(HCA_ERR_UNSUPPORTED, fn, "indexer dim must be 64");
  if (n_idx_heads < 1 || n_idx_heads > 8) return fail(HCA_ERR_UNSUPPORTED, fn, "indexer heads must be 1..8");
  if (k < 1 || k > 2048) return fail(HCA_ERR_INVALID_ARG, fn, "k must be 1..2048");
  if (m < 1 || nq < 0 || max_visible < 0 || k_rows < 0) return fail(HCA_ERR_INVALID_ARG, fn, "bad m/nq/max_visible/k_rows");
  if (w < m || w > (1 << 20)) return fail(HCA_ERR_INVALID_ARG, fn, "need m <= w <= 2^20");
  if (max_visible > ((int64_t)1 << 21)) return fail(HCA_ERR_UNSUPPORTED, fn, "max_visible above 2^21");
  if (!aligned16(q_idx) || !aligned16(k_idx)) return fail(HCA_ERR_INVALID_ARG, fn, "q_idx/k_idx not 16-byte aligned");
  if (nq == 0) return HCA_OK;
  if (!ws || ws_bytes < index_ws(1, max_visible)) return fail(HCA_ERR_WORKSPACE, fn, "workspace too small");
  if (phase != kIndexBoth && ws_bytes < index_ws(nq, max_visible))
    return fail(HCA_ERR_WORKSPACE, fn, "the split calls need the workspace of all nq queries");
  int64_t batch = nq;
  if (!hca::index_stream_path(idx_dtype, n_idx_heads, nq, k))
    while (batch > 1 && index_ws(batch, max_visible) > ws_bytes) batch = std::max<int64_t>(1, batch / 2);
  const int64_t q_row = idx_dtype == HCA_MXFP4 ? (int64_t)n_idx_heads * d_idx / 2
                                               : (int64_t)n_idx_heads * d_idx * (idx_dtype == HCA_F32 ? 4 : 2);
  if (phase != kIndexPending) {  // recording a selection touches no device
    const int st = ensure_init(fn);
    if (st != HCA_OK) return st;
  }
  for (int64_t q0 = 0; q0 < nq; q0 += batch) {
    const int64_t nb = std::min<int64_t>(batch, nq - q0);
    hca::IndexArgs a;
    hca::index_ws_layout(nb, max_visible, ws, &a);
    a.q = static_cast<const uint8_t*>(q_idx) + q0 * q_row;
    a.q_scale = idx_dtype == HCA_MXFP4 ? q_idx_scale + q0 * n_idx_heads * (d_idx / 32) : nullptr;
    a.w = w_idx + q0 * n_idx_heads;
    a.H = n_idx_heads;
    a.d = d_idx;
    a.dtype = idx_dtype;
    a.keys = k_idx;
    a.key_scale = k_idx_scale;
    a.k_rows = k_rows;
    a.k_row_begin = k_row_begin;
    a.q_seq = q_seq + q0;
    a.q_pos = q_pos + q0;
    a.q_lo = q_lo ? q_lo + q0 : nullptr;
    a.cw = w;
    a.nq = (int)nb;
    a.max_visible = max_visible;
    a.m = m;
    a.k = k;
    a.out = out_idx + q0 * k;
    if (phase == kIndexPending) {
      // the split calls take every query in one batch; the streaming path's selection phase has
      // nothing to launch
      pending->a = a;
      pending->active = hca::index_stream_path(idx_dtype, n_idx_heads, nq, k) ? 0 : 1;
      return HCA_OK;
    }
    hipError_t e = hca::launch_index_topk(a, phase != kIndexSelect, phase != kIndexScores,
                                          static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return launched(fn, e);
  }
  return HCA_OK;
}

}  // namespace

extern "C" {

#define HCA_INDEX_ARGS                                                                                           \
  const void *q_idx, const uint8_t *q_idx_scale, const float *w_idx, int32_t n_idx_heads, int32_t d_idx,         \
      int32_t idx_dtype, const void *k_idx, const uint8_t *k_idx_scale, int64_t k_rows,                          \
      const int64_t *k_row_begin, const int32_t *q_seq, const int64_t *q_pos, const int64_t *q_lo, int32_t nq,   \
      int64_t max_visible, int32_t m, int32_t w, int32_t k, int32_t *out_idx, void *ws, size_t ws_bytes,         \
      void *stream
#define HCA_INDEX_PASS                                                                                           \
  q_idx, q_idx_scale, w_idx, n_idx_heads, d_idx, idx_dtype, k_idx, k_idx_scale, k_rows, k_row_begin, q_seq,      \
      q_pos, q_lo, nq, max_visible, m, w, k, out_idx, ws, ws_bytes, stream

HCA_EXPORT int lightning_index_topk(HCA_INDEX_ARGS) {
  return index_impl("lightning_index_topk", kIndexBoth, HCA_INDEX_PASS);
}

HCA_EXPORT int lightning_index_scores(HCA_INDEX_ARGS) {
  return index_impl("lightning_index_scores", kIndexScores, HCA_INDEX_PASS);
}

HCA_EXPORT int lightning_index_select(HCA_INDEX_ARGS) {
  return index_impl("lightning_index_select", kIndexSelect, HCA_INDEX_PASS);
}

HCA_EXPORT int lightning_index_select_pending(HCA_INDEX_ARGS, hca_pending_select* out) {
  const char* fn = "lightning_index_select_pending";
  if (!out) return fail(HCA_ERR_INVALID_ARG, fn, "NULL out");
  PendingSelect ps{};
  const int st = index_impl(fn, kIndexPending, HCA_INDEX_PASS, &ps);
  if (st != HCA_OK) return st;
  ps.magic = kPendingMagic;
  std::memset(out, 0, sizeof(*out));
  std::memcpy(out, &ps, sizeof(ps));
  return HCA_OK;
}

HCA_EXPORT size_t mqa_attn_workspace(int32_t q_dtype, int32_t nq, int32_t n_heads, int32_t d, int64_t max_entries) {
  if (nq <= 0 || n_heads < 1 || d < 1 || max_entries < 0) return 0;
  return attn_ws_any(q_dtype, nq, n_heads, d, max_entries);
}

HCA_EXPORT int csa_sparse_mqa_attn(const void* q, int32_t q_dtype, int32_t nq, int32_t n_heads, const hca_store* cache,
                        const int64_t* cache_row_begin, const int32_t* idx, int32_t k, const hca_store* window,
                        const int64_t* win_row_begin, const int64_t* win_pos0, int32_t W, const int32_t* q_seq,
                        const int64_t* q_pos, const int64_t* q_lo, float scale, void* o, int32_t o_dtype, float* lse,
                        void* ws, size_t ws_bytes, void* stream) {
  return attn_impl("csa_sparse_mqa_attn", true, q, q_dtype, nq, n_heads, cache, cache_row_begin, idx, k, 1, 0,
                   window, win_row_begin, win_pos0, W, q_seq, q_pos, q_lo, scale, o, o_dtype, lse, ws, ws_bytes,
                   stream);
}

HCA_EXPORT int hca_dense_mqa_attn_noalloc(const void* q, int32_t q_dtype, int32_t nq, int32_t n_heads,
                                          const hca_store* cache, const int64_t* cache_row_begin, int32_t m_prime,
                                          int64_t max_visible, const hca_store* window, const int64_t* win_row_begin,
                                          const int64_t* win_pos0, int32_t W, const int32_t* q_seq,
                                          const int64_t* q_pos, const int64_t* q_lo, float scale, void* o,
                                          int32_t o_dtype, float* lse, void* stream) {
  return attn_impl("hca_dense_mqa_attn_noalloc", false, q, q_dtype, nq, n_heads, cache, cache_row_begin, nullptr, 0,
                   m_prime, max_visible, window, win_row_begin, win_pos0, W, q_seq, q_pos, q_lo, scale, o, o_dtype,
                   lse, nullptr, 0, stream, /*static_scratch=*/true);
}

HCA_EXPORT int csa_sparse_mqa_attn_partials(const void* q, int32_t q_dtype, int32_t nq, int32_t n_heads,
                                            const hca_store* cache, const int64_t* cache_row_begin, const int32_t* idx,
                                            int32_t k, const hca_store* window, const int64_t* win_row_begin,
                                            const int64_t* win_pos0, int32_t W, const int32_t* q_seq,
                                            const int64_t* q_pos, const int64_t* q_lo, float scale, void* o,
                                            int32_t o_dtype, float* lse, void* ws, size_t ws_bytes, void* stream,
                                            hca_attn_partials* out) {
  const char* fn = "csa_sparse_mqa_attn_partials";
  if (!out) return fail(HCA_ERR_INVALID_ARG, fn, "NULL out");
  return attn_impl(fn, true, q, q_dtype, nq, n_heads, cache, cache_row_begin, idx, k, 1, 0, window, win_row_begin,
                   win_pos0, W, q_seq, q_pos, q_lo, scale, o, o_dtype, lse, ws, ws_bytes, stream, false, out);
}

HCA_EXPORT int hca_dense_mqa_attn_partials(const void* q, int32_t q_dtype, int32_t nq, int32_t n_heads,
                                           const hca_store* cache, const int64_t* cache_row_begin, int32_t m_prime,
                                           int64_t max_visible, const hca_store* window, const int64_t* win_row_begin,
                                           const int64_t* win_pos0, int32_t W, const int32_t* q_seq,
                                           const int64_t* q_pos, const int64_t* q_lo, float scale, void* o,
                                           int32_t o_dtype, float* lse, void* ws, size_t ws_bytes, void* stream,
                                           hca_attn_partials* out) {
  const char* fn = "hca_dense_mqa_attn_partials";
  if (!out) return fail(HCA_ERR_INVALID_ARG, fn, "NULL out");
  return attn_impl(fn, false, q, q_dtype, nq, n_heads, cache, cache_row_begin, nullptr, 0, m_prime, max_visible,
                   window, win_row_begin, win_pos0, W, q_seq, q_pos, q_lo, scale, o, o_dtype, lse, ws, ws_bytes,
                   stream, false, out);
}

HCA_EXPORT int hca_dense_mqa_attn_partials_select(const void* q, int32_t q_dtype, int32_t nq, int32_t n_heads,
                                                  const hca_store* cache, const int64_t* cache_row_begin,
                                                  int32_t m_prime, int64_t max_visible, const hca_store* window,
                                                  const int64_t* win_row_begin, const int64_t* win_pos0, int32_t W,
                                                  const int32_t* q_seq, const int64_t* q_pos, const int64_t* q_lo,
                                                  float scale, void* o, int32_t o_dtype, float* lse, void* ws,
                                                  size_t ws_bytes, void* stream, const hca_pending_select* sel,
                                                  hca_attn_partials* out) {
  const char* fn = "hca_dense_mqa_attn_partials_select";
  if (!out || !sel) return fail(HCA_ERR_INVALID_ARG, fn, "NULL out or sel");
  PendingSelect ps;
  std::memcpy(&ps, sel, sizeof(ps));
  if (ps.magic != kPendingMagic) return fail(HCA_ERR_INVALID_ARG, fn, "sel was not filled by lightning_index_select_pending");
  return attn_impl(fn, false, q, q_dtype, nq, n_heads, cache, cache_row_begin, nullptr, 0, m_prime, max_visible,
                   window, win_row_begin, win_pos0, W, q_seq, q_pos, q_lo, scale, o, o_dtype, lse, ws, ws_bytes,
                   stream, false, out, ps.active ? &ps.a : nullptr);
}

HCA_EXPORT int mqa_attn_merge(const hca_attn_partials* a, const hca_attn_partials* b, void* stream) {
  const char* fn = "mqa_attn_merge";
  if (!a) return fail(HCA_ERR_INVALID_ARG, fn, "NULL a");
  int st = check_partials(fn, a, "a");
  if (st != HCA_OK) return st;
  if (b && (st = check_partials(fn, b, "b")) != HCA_OK) return st;
  if ((a->n_split > 1 ? a->nq : 0) + (b && b->n_split > 1 ? b->nq : 0) == 0) return HCA_OK;
  st = ensure_init(fn);
  if (st != HCA_OK) return st;
  const hca::MergeArgs ma = merge_of(a);
  hca::MergeArgs mb;
  if (b) mb = merge_of(b);
  return launched(fn, hca::launch_merge(ma, b ? &mb : nullptr, static_cast<hipStream_t>(stream)));
}

HCA_EXPORT int hca_dense_mqa_attn(const void* q, int32_t q_dtype, int32_t nq, int32_t n_heads, const hca_store* cache,
                       const int64_t* cache_row_begin, int32_t m_prime, int64_t max_visible, const hca_store* window,
                       const int64_t* win_row_begin, const int64_t* win_pos0, int32_t W, const int32_t* q_seq,
                       const int64_t* q_pos, const int64_t* q_lo, float scale, void* o, int32_t o_dtype, float* lse,
                       void* ws, size_t ws_bytes, void* stream) {
  return attn_impl("hca_dense_mqa_attn", false, q, q_dtype, nq, n_heads, cache, cache_row_begin, nullptr, 0,
                   m_prime, max_visible, window, win_row_begin, win_pos0, W, q_seq, q_pos, q_lo, scale, o, o_dtype,
                   lse, ws, ws_bytes, stream);
}

}  // extern "C"
