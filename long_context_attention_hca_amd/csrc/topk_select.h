// Exact top-k selection of the lightning indexer: the shared helpers of the score kernels and
// the selection that one block runs per query over the candidates the score kernels leave in
// the workspace. Included by the indexer and by the attention library, which launches the
// selection beside HCA attention in one grid.
//
// Method: hyper.ai paper page for arXiv 2606.19348 ("DeepSeek-V4"), section 方法 (Method),
// CSA paragraph (a lightning indexer selects the top-k compressed KV entries; ties go to the
// lower entry index). The selection works on the 64-bit key (order-preserving score bits << 32
// | ~j), which is unique per entry; its design is described in the indexer's header.
#pragma once
#include "common.h"
#include "internal.h"

namespace hca {
namespace {

constexpr int kBlockKeys = 1024;        // entries per score block
constexpr int kFinThreads = 512;        // finalize block
constexpr int kCandCap = 8192;          // candidates finalize holds in registers
constexpr int kMaxBlk = 2048;           // score blocks per query (max_visible <= 2^21)
constexpr int kBpt = kMaxBlk / kFinThreads;  // score blocks per finalize thread


// The visible entries of query qi are the rows *row0 + j, j < the returned count, which are
// entries *j0 + j of its sequence: with a document mask the entries before j_lo (their window
// starts before the document) are cut off the front, so the kernels work on the shifted range
// and add *j0 to the indices they output.
__device__ __forceinline__ int64_t visible_keys(const IndexArgs& a, int qi, int64_t* row0, int64_t* j0 = nullptr) {
  const int b = a.q_seq[qi];
  const int64_t t = a.q_pos[qi];
  const int64_t lo = a.q_lo ? a.q_lo[qi] : 0;
  const int64_t j_lo = lo > 0 ? (lo + a.cw - 1) / a.m : 0;  // ceil((lo + cw - m) / m)
  const int64_t rb = a.k_row_begin[b] + j_lo;
  int64_t nv = t >= 0 ? (t + 1) / a.m : 0;
  nv = min(nv, a.max_visible) - j_lo;
  nv = min(nv, a.k_rows - rb);
  if (rb < 0 || nv < 0) nv = 0;
  *row0 = rb;
  if (j0) *j0 = j_lo;
  return nv;
}

// ---------------------------------------------------------------------------------------
// Block-wide helpers (blockDim.x = NT, a multiple of 64).

// Exclusive prefix sum of v over the block (thread order); *total gets the block sum.
template <int NT>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* lds_tmp, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t x = wave_incl_scan_add(v);
  if (lane == 63) lds_tmp[wave] = x;
  __syncthreads();
  uint32_t wbase = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const uint32_t t = lds_tmp[w];
    wbase += w < wave ? t : 0;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return wbase + x - v;
}

// Over counters c[0..256*PER) in LDS: the largest index d with sum_{i >= d} c[i] >= rem, and
// above = sum_{i > d} c[i]. Wave 0 must call it; one lane writes the result to *d_out /
// *above_out (LDS). Requires sum c >= rem >= 1.
template <int PER>
__device__ __forceinline__ void find_crossing(const uint32_t* c, uint32_t rem, int* d_out, uint32_t* above_out) {
  const int lane = threadIdx.x & 63;
  constexpr int G = 4 * PER;  // counters per lane
  uint32_t v[G];
  uint32_t own = 0;
  const uint4* c4 = reinterpret_cast<const uint4*>(c);
#pragma unroll
  for (int i = 0; i < G / 4; ++i) {
    const uint4 q = c4[(G / 4) * lane + i];
    v[4 * i] = q.x;
    v[4 * i + 1] = q.y;
    v[4 * i + 2] = q.z;
    v[4 * i + 3] = q.w;
    own += q.x + q.y + q.z + q.w;
  }
  const uint32_t pre = wave_incl_scan_add(own);
  const uint32_t nxt = (uint32_t)__builtin_amdgcn_readlane((int)pre, 63) - pre;  // sum over lanes > lane
  const uint32_t suf = nxt + own;                                                 // sum over lanes >= lane
  if (suf >= rem && nxt < rem) {
    uint32_t acc = nxt;
    int d = G * lane;
#pragma unroll
    for (int i = G - 1; i >= 0; --i) {
      if (acc + v[i] >= rem) { d = G * lane + i; break; }
      acc += v[i];
    }
    *d_out = d;
    *above_out = acc;
  }
}

struct CrossLds {
  int dc, d;
  uint32_t ac, above;
};

// Over 2048 counters h in LDS with NT threads: *d = the largest bin with
// sum_{i >= d} h[i] >= rem and *above = sum_{i > d} h[i]. Requires sum >= rem >= 1; part is
// NT words of LDS. Reads are 16-byte vectors so that the threads hit distinct LDS banks.
// Ends with the block synchronised.
template <int NT>
__device__ __forceinline__ void crossing2048(const uint32_t* h, uint32_t* part, uint32_t rem, CrossLds& x, int* d,
                                             uint32_t* above) {
  constexpr int B = kHistBins / NT;  // bins per thread
  const int tid = threadIdx.x;
  const uint4* h4 = reinterpret_cast<const uint4*>(h);
  uint32_t s = 0;
#pragma unroll
  for (int i = 0; i < B / 4; ++i) {
    const uint4 q = h4[(B / 4) * tid + i];
    s += q.x + q.y + q.z + q.w;
  }
  part[tid] = s;
  __syncthreads();
  if (tid < 64) find_crossing<NT / 256>(part, rem, &x.dc, &x.ac);
  __syncthreads();
  if (tid == x.dc) {
    uint32_t acc = x.ac;
    int b = B * tid + B - 1;
    for (; b > B * tid; --b) {
      if (acc + h[b] >= rem) break;
      acc += h[b];
    }
    x.d = b;
    x.above = acc;
  }
  __syncthreads();
  *d = x.d;
  *above = x.above;
}

// Candidates of a block: L = max(16, ceil(2 k 1024 / n_vis)), about twice the block's share of
// the top-k when the top-k is spread evenly over the blocks.
__device__ __forceinline__ uint32_t block_quota(int k, int64_t nv) {
  return (uint32_t)max<int64_t>(16, (2 * (int64_t)k * kBlockKeys + nv - 1) / nv);
}
// Candidate slots per block: a block emits at most 2L keys (and at most its 1024 entries).
__device__ __forceinline__ uint32_t region_slots(uint32_t L) { return min(2 * L, (uint32_t)kBlockKeys); }

// Wave-wide minimum and maximum of 64-bit keys.
__device__ __forceinline__ uint64_t wave_min_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)v, off, 64), hi = __shfl_xor((uint32_t)(v >> 32), off, 64);
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    v = o < v ? o : v;
  }
  return v;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)v, off, 64), hi = __shfl_xor((uint32_t)(v >> 32), off, 64);
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

// ---------------------------------------------------------------------------------------
// Finalisation: one block of NT threads per query (NT = kFinThreads = 512 for finalize_kernel
// and HCA attention's FP8 grid, 256 for the bf16-store attention grid).

constexpr int kListCap = kHistBins / 2;         // keys of one bin ranked exactly (the histogram's LDS)

template <int NT>
struct FinLdsT {
  uint32_t h[kHistBins];  // histogram; keys of the crossing bin (as u64); flagged blocks; output
  uint64_t sel[kMaxTopK];  // keys of the selected entries
  uint64_t sel_sink[64];   // per-lane targets of writes that select nothing (branch-free code)
  uint64_t list_sink[64];
  uint32_t part[NT];
  uint32_t tmp[32];
  CrossLds cx;
  uint64_t kmin, kmax, T;
  uint32_t smin, smax, nsel, nflag, novf;
};
using FinLds = FinLdsT<kFinThreads>;

// The candidates of one query: ns slots of the score blocks (0 = empty) and novf rescanned keys.
struct CandSet {
  const uint64_t* slots;
  uint32_t ns;
  const uint64_t* ovf;
  uint32_t novf;
};

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ int32_t key_entry(uint64_t key) { return (int32_t)(0xFFFFFFFFu - (uint32_t)key); }

// The score whose float_key is k (the top half of a candidate key).
__device__ __forceinline__ float key_score(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// f.kmin / f.kmax <- the smallest and largest of the per-thread extremes lo / hi.
template <int NT>
__device__ __forceinline__ void block_min_max(uint64_t lo, uint64_t hi, FinLdsT<NT>& f) {
  lo = wave_min_u64(lo);
  hi = wave_max_u64(hi);
  if (threadIdx.x == 0) {
    f.kmin = ~0ull;
    f.kmax = 0;
  }
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
    atomicMin(reinterpret_cast<unsigned long long*>(&f.kmin), (unsigned long long)lo);
    atomicMax(reinterpret_cast<unsigned long long*>(&f.kmax), (unsigned long long)hi);
  }
  __syncthreads();
}

// Monotone map of a candidate key to one of 2048 equal-width bins of the score range between
// the score keys k0 < k1.
struct ScoreBins {
  float s0, inv;
  __device__ __forceinline__ ScoreBins(uint32_t k0, uint32_t k1) {
    s0 = key_score(k0);
    inv = 2047.0f / (key_score(k1) - s0);
  }
  __device__ __forceinline__ int operator()(uint64_t key) const {
    return (int)fminf(fmaxf(__fmul_rn(__fsub_rn(key_score((uint32_t)(key >> 32)), s0), inv), 0.f), 2047.f);
  }
};

// Appends x to list[] (counter *n) with one LDS atomic per wave; p says whether this lane appends.
template <class Tv>
__device__ __forceinline__ void wave_append(bool p, Tv x, Tv* list, uint32_t* n, uint32_t cap) {
  const uint64_t m = __ballot(p);
  if (m == 0) return;
  const int lane = threadIdx.x & 63, leader = __ffsll((long long)m) - 1;
  uint32_t base = 0;
  if (lane == leader) base = atomicAdd(n, (uint32_t)__popcll(m));
  base = (uint32_t)__builtin_amdgcn_readlane((int)base, leader);
  const uint32_t slot = base + lanes_below(m);
  if (p && slot < cap) list[slot] = x;
}

// Selection with the candidates in registers (v[i], 0 = empty; at least K non-empty, unique).
// Returns T, the K-th largest key (exactly K keys are >= T); with kSel it also writes those K
// keys to f.sel (unordered). First pass: a histogram over 2048 equal-width bins of the
// candidates' score range; the keys of the bin holding the K-th key are then ranked exactly
// among themselves (gathered by per-wave appends when only T is wanted; with kSel every
// selected key is placed by a block scan or by its rank). Equal scores throughout, or a
// crossing bin with more than kListCap keys (heavy ties), are resolved by 11-bit radix passes
// below the bits all candidates share.
template <bool kSel, int NT>
__device__ __forceinline__ uint64_t select_regs(const uint64_t (&v)[kCandCap / NT], uint32_t K, FinLdsT<NT>& f) {
  constexpr int kPer = kCandCap / NT;
  const int tid = threadIdx.x;
  // Elementwise steps below are written without branches (selects, sink addresses): in this
  // one-pass kernel every taken branch is a likely instruction-cache miss.
  const int lane = tid & 63;
  uint32_t lo = 0xFFFFFFFFu, hi = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const uint32_t k = (uint32_t)(v[i] >> 32);  // 0 for an empty slot
    lo = min(lo, v[i] ? k : 0xFFFFFFFFu);
    hi = max(hi, k);
  }
  lo = wave_min_u32(lo);
  hi = wave_max_u32(hi);
  if (tid == 0) {
    f.smin = 0xFFFFFFFFu;
    f.smax = 0;
  }
  for (int i = tid; i < kHistBins; i += NT) f.h[i] = 0;
  __syncthreads();
  if ((tid & 63) == 0) {
    atomicMin(&f.smin, lo);
    atomicMax(&f.smax, hi);
  }
  __syncthreads();
  if (f.smin != f.smax) {
    const ScoreBins bin(f.smin, f.smax);
    int bn[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int b = bin(v[i]);
      bn[i] = v[i] ? b : -1;
      atomicAdd(v[i] ? &f.h[b] : &f.part[tid], 1u);  // part[] is rewritten by the crossing search
    }
    __syncthreads();
    int d;
    uint32_t above;
    crossing2048<NT>(f.h, f.part, K, f.cx, &d, &above);
    const uint32_t rem = K - above, cd = f.h[d];
    if (tid == 0) f.nsel = 0;
    __syncthreads();
    if (cd <= (uint32_t)kListCap && !kSel) {
      // the crossing bin's keys, in any order (one LDS atomic per wave and slot)
      uint64_t* list = reinterpret_cast<uint64_t*>(f.h);
#pragma unroll
      for (int i = 0; i < kPer; ++i) wave_append<uint64_t>(bn[i] == d, v[i], list, &f.nsel, (uint32_t)kListCap);
      __syncthreads();
      for (uint32_t i = tid; i < cd; i += NT) {
        const uint64_t x = list[i];
        uint32_t g = 0;
        for (uint32_t j = 0; j < cd; ++j) g += list[j] > x;
        if (g == rem - 1) f.T = x;
      }
      __syncthreads();
      return f.T;
    }
    if (cd <= (uint32_t)kListCap) {
      uint64_t* list = reinterpret_cast<uint64_t*>(f.h);
      uint32_t na = 0, nl = 0;
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        na += bn[i] > d;
        nl += bn[i] == d;
      }
      uint32_t tot;
      const uint32_t off = block_exclusive_scan<NT>(na | (nl << 16), f.tmp, &tot);
      uint32_t oa = off & 0xFFFFu, ol = off >> 16;
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const bool a = bn[i] > d, l = bn[i] == d;
        if (kSel) *(a ? &f.sel[min(oa, K - 1)] : &f.sel_sink[lane]) = v[i];
        *(l ? &list[min(ol, (uint32_t)kListCap - 1)] : &f.list_sink[lane]) = v[i];
        oa += a;
        ol += l;
      }
      __syncthreads();
      // rank within the bin: a key with g larger keys is selected iff g < rem
      for (uint32_t i = tid; i < cd; i += NT) {
        const uint64_t x = list[i];
        uint32_t g = 0;
        for (uint32_t j = 0; j < cd; ++j) g += list[j] > x;
        if (kSel && g < rem) f.sel[above + g] = x;
        if (g == rem - 1) f.T = x;
      }
      __syncthreads();
      return f.T;
    }
  }
  // radix passes (heavy ties, or a single candidate)
  uint64_t klo = ~0ull, khi = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    if (v[i]) klo = v[i] < klo ? v[i] : klo;
    khi = v[i] > khi ? v[i] : khi;
  }
  block_min_max(klo, khi, f);
  const uint64_t kmin = f.kmin, kmax = f.kmax;
  uint64_t T = kmin;
  if (kmin != kmax) {
    int lb = 64 - __clzll((long long)(kmin ^ kmax));  // bits >= lb are common to all candidates
    uint64_t prefix = lb >= 64 ? 0ull : (kmax >> lb) << lb;
    uint32_t rem = K;
    while (true) {
      const int hb = lb, width = min(11, lb);
      lb -= width;
      for (int i = tid; i < kHistBins; i += NT) f.h[i] = 0;
      __syncthreads();
      const uint64_t want = hb >= 64 ? 0ull : prefix >> hb;
      const uint32_t dmask = (1u << width) - 1u;
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const bool m = v[i] && (hb >= 64 || (v[i] >> hb) == want);
        atomicAdd(m ? &f.h[(uint32_t)(v[i] >> lb) & dmask] : &f.part[tid], 1u);
      }
      __syncthreads();
      int d;
      uint32_t above;
      crossing2048<NT>(f.h, f.part, rem, f.cx, &d, &above);
      rem -= above;
      prefix |= (uint64_t)d << lb;
      const bool done = f.h[d] == rem || lb == 0;
      __syncthreads();
      if (done) break;
    }
    T = prefix;
  }
  if (!kSel) return T;
  uint32_t n = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) n += v[i] >= T;  // T > 0, so empty slots never count
  uint32_t tot;
  uint32_t o = block_exclusive_scan<NT>(n, f.tmp, &tot);
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const bool s = v[i] >= T;
    *(s ? &f.sel[min(o, K - 1)] : &f.sel_sink[tid & 63]) = v[i];
    o += s;
  }
  __syncthreads();
  return T;
}

// Calls fn(key) for every candidate held in global memory (empty slots skipped).
template <int NT, class F>
__device__ __forceinline__ void for_each_global(const CandSet& cs, F fn) {
  for (uint32_t i = threadIdx.x; i < cs.ns; i += NT) {
    const uint64_t key = cs.slots[i];
    if (key) fn(key);
  }
  for (uint32_t i = threadIdx.x; i < cs.novf; i += NT) fn(cs.ovf[i]);
}

// Selection over more candidates than the registers hold: the same steps as select_regs, with
// every pass reading the candidates from global memory and LDS atomics for the appends.
template <int NT>
__device__ uint64_t select_global(const CandSet& cs, uint32_t K, FinLdsT<NT>& f) {
  const int tid = threadIdx.x;
  uint64_t lo = ~0ull, hi = 0;
  for_each_global<NT>(cs, [&](uint64_t x) {
    lo = x < lo ? x : lo;
    hi = x > hi ? x : hi;
  });
  block_min_max(lo, hi, f);
  const uint64_t kmin = f.kmin, kmax = f.kmax;
  if (tid == 0) f.nsel = 0;
  uint64_t T = kmin;
  if (kmin != kmax) {
    int lb = 64 - __clzll((long long)(kmin ^ kmax));
    uint64_t prefix = lb >= 64 ? 0ull : (kmax >> lb) << lb;
    uint32_t rem = K;
    while (true) {
      const int hb = lb, width = min(11, lb);
      lb -= width;
      for (int i = tid; i < kHistBins; i += NT) f.h[i] = 0;
      __syncthreads();
      const uint64_t want = hb >= 64 ? 0ull : prefix >> hb;
      const uint32_t dmask = (1u << width) - 1u;
      for_each_global<NT>(cs, [&](uint64_t key) {
        if (hb >= 64 || (key >> hb) == want) atomicAdd(&f.h[(uint32_t)(key >> lb) & dmask], 1u);
      });
      __syncthreads();
      int d;
      uint32_t above;
      crossing2048<NT>(f.h, f.part, rem, f.cx, &d, &above);
      rem -= above;
      prefix |= (uint64_t)d << lb;
      const bool done = f.h[d] == rem || lb == 0;
      __syncthreads();
      if (done) break;
    }
    T = prefix;
  }
  __syncthreads();
  for_each_global<NT>(cs, [&](uint64_t key) { wave_append<uint64_t>(key >= T, key, f.sel, &f.nsel, K); });
  __syncthreads();
  return T;
}

// Candidates tid + NT * i of cs into registers (0 past the end). Unconditional loads
// from clamped slots stay in flight together.
template <int NT>
__device__ __forceinline__ void load_candidates(const CandSet& cs, uint64_t (&v)[kCandCap / NT]) {
  constexpr int kPer = kCandCap / NT;
  const int tid = threadIdx.x;
  const uint32_t n = cs.ns + cs.novf;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const uint32_t s = min((uint32_t)(tid + NT * i), n - 1);
    v[i] = *(s < cs.ns ? cs.slots + s : cs.ovf + (s - cs.ns));
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i)
    if (tid + NT * i >= (int)n) v[i] = 0;
}

// Score blocks whose unemitted keys (all below the block's threshold) may reach T; their
// numbers go to f.h. Returns how many.
template <int NT>
__device__ __forceinline__ uint32_t flag_blocks(const uint64_t (&tq)[kMaxBlk / NT], uint64_t T, FinLdsT<NT>& f) {
  constexpr int kBpt = kMaxBlk / NT;
  const int tid = threadIdx.x;
  if (tid == 0) f.nflag = 0;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kBpt; ++i)
    if (tq[i] > T) f.h[atomicAdd(&f.nflag, 1u)] = (uint32_t)(kBpt * tid + i);
  __syncthreads();
  return f.nflag;
}

// Output of the K keys >= T when they are all among the emitted candidates. The candidate slots
// are in ascending entry order (score blocks in order, each block's keys ascending, empty slots
// 0 < T), so compacting the selected slots in slot order gives the ascending answer. Slot
// tid + NT * i is position (i, wave, lane) in row-major order: per-wave ballots give
// the lane offsets, a scan of the kPer x (NT / 64) wave counts the rest.
template <int NT>
__device__ __forceinline__ void ordered_output(const uint64_t (&v)[kCandCap / NT], uint64_t T, int K, int32_t* out,
                                               int32_t j0, FinLdsT<NT>& f) {
  constexpr int kPer = kCandCap / NT, kW = NT / 64;
  static_assert(kPer * kW == 128, "two counts per lane of one wave");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t* cnt = f.h;  // [kPer][kW] wave counts, then their exclusive prefix
  uint32_t mb[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const uint64_t bal = __ballot(v[i] >= T);
    mb[i] = lanes_below(bal);
    if (lane == 0) cnt[i * kW + wave] = (uint32_t)__popcll(bal);
  }
  __syncthreads();
  if (wave == 0) {
    const uint32_t c0 = cnt[2 * lane], c1 = cnt[2 * lane + 1];
    const uint32_t incl = wave_incl_scan_add(c0 + c1);
    cnt[2 * lane] = incl - c0 - c1;
    cnt[2 * lane + 1] = incl - c1;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kPer; ++i)
    if (v[i] >= T) out[min(cnt[i * kW + wave] + mb[i], (uint32_t)K - 1)] = key_entry(v[i]) + j0;
}

// Output LDS: per-block counts (then their prefix), per-block cursors, entries bucketed by block.
struct OutLds {
  uint32_t pre[kMaxBlk + 1];
  uint32_t cur[kMaxBlk];
  alignas(16) int32_t bucket[kMaxTopK];
};

// The selection of query qi by one block of NT threads; f and ol are its LDS.
template <int NT>
__device__ __forceinline__ void finalize_block(const IndexArgs& a, int qi, FinLdsT<NT>& f, OutLds& ol) {
  constexpr int kPer = kCandCap / NT, kBpt = kMaxBlk / NT;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int K = a.k;
  const int64_t q_blk = (int64_t)qi * a.nblk;
  const uint64_t* thr = a.blk_thr + q_blk;
  const uint64_t* slots = a.cand + q_blk * kBlockKeys;
  // The candidate slots and block thresholds lie in this query's workspace region, so their
  // loads go out first (clamped to the region) and are masked once the visible count is known.
  uint64_t v[kPer], tq[kBpt];
  {
    const uint32_t region = (uint32_t)a.nblk * kBlockKeys;
#pragma unroll
    for (int i = 0; i < kPer; ++i) v[i] = slots[min((uint32_t)(tid + NT * i), region - 1)];
#pragma unroll
    for (int i = 0; i < kBpt; ++i) tq[i] = thr[min(kBpt * tid + i, a.nblk - 1)];
  }
  int64_t rb, j0;
  const int64_t nv = visible_keys(a, qi, &rb, &j0);
  const int32_t jo = (int32_t)j0;  // entry index of visible key 0
  int32_t* out = a.out + (int64_t)qi * K;
  if (nv <= K) {  // every visible entry is selected, ascending; pad with -1
    for (int j = tid; j < K; j += NT) out[j] = j < nv ? j + jo : -1;
    return;
  }
  const int nb = (int)((nv + kBlockKeys - 1) / kBlockKeys);
  const uint32_t* sk = a.scores + q_blk * kBlockKeys;
  const int64_t ovf_cap = (int64_t)a.nblk * kBlockKeys + kMaxTopK;  // >= k + n_vis
  uint64_t* ovf = a.ovf + (int64_t)qi * ovf_cap;
  CandSet cs;
  cs.slots = slots;
  cs.ns = (uint32_t)nb * region_slots(block_quota(K, nv));
  cs.ovf = ovf;
  cs.novf = 0;
  // thresholds of blocks kBpt * tid + i
#pragma unroll
  for (int i = 0; i < kBpt; ++i)
    if (kBpt * tid + i >= nb) tq[i] = 0ull;
  if (tid == 0) f.novf = 0;
  // round 1 over the emitted candidates
  uint64_t T;
  uint32_t nflag;
  if (cs.ns <= (uint32_t)kCandCap) {
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      if ((uint32_t)(tid + NT * i) >= cs.ns) v[i] = 0;
    T = select_regs<false>(v, (uint32_t)K, f);
    nflag = flag_blocks(tq, T, f);
    if (nflag == 0) {
      ordered_output(v, T, K, out, jo, f);
      return;
    }
    // the round-1 winners (the K keys >= T) seed the overflow list of round 2
    uint32_t c = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) c += v[i] >= T;
    uint32_t tot;
    uint32_t o = block_exclusive_scan<NT>(c, f.tmp, &tot);
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      if (v[i] >= T) ovf[min(o++, (uint32_t)K - 1)] = v[i];
  } else {
    T = select_global(cs, (uint32_t)K, f);
    nflag = flag_blocks(tq, T, f);
    if (nflag > 0)
      for (int i = tid; i < K; i += NT) ovf[i] = f.sel[i];
  }
  if (nflag > 0) {
    // round 2 selects among the round-1 winners (every candidate >= T) and the unemitted keys
    // >= T of the flagged blocks (one wave per block), all gathered in the overflow list:
    // together they hold every key >= T, hence the whole top-k
    if (tid == 0) f.novf = (uint32_t)K;
    __syncthreads();
    // Each wave takes flagged blocks wave, wave + W, ... (W waves), two per step, with the next
    // two blocks' keys already in flight; a block's keys >= T that it did not emit (those below
    // its threshold) are appended with one LDS atomic per wave and block.
    constexpr int kR = kBlockKeys / 64, kW = NT / 64;
    struct Blk {
      uint32_t kv[kR];
      uint64_t tb;
      int b;
    };
    auto load_blk = [&](uint32_t fi, Blk& x) {
      x.b = (int)f.h[min(fi, nflag - 1)];
      x.tb = thr[x.b];
#pragma unroll
      for (int r = 0; r < kR; ++r) x.kv[r] = sk[min<int64_t>((int64_t)x.b * kBlockKeys + lane + 64 * r, nv - 1)];
    };
    auto append_blk = [&](const Blk& x) {
      const int64_t jb = (int64_t)x.b * kBlockKeys;
      uint64_t k64[kR];
      uint32_t pm = 0, c = 0;
#pragma unroll
      for (int r = 0; r < kR; ++r) {
        const int64_t j = jb + lane + 64 * r;
        k64[r] = ((uint64_t)x.kv[r] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)j);
        const bool p = j < nv && k64[r] < x.tb && k64[r] >= T;
        pm |= (uint32_t)p << r;
        c += p;
      }
      const uint32_t incl = wave_incl_scan_add(c);
      const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
      if (total == 0) return;
      uint32_t base = 0;
      if (lane == 0) base = atomicAdd(&f.novf, total);
      uint32_t o = (uint32_t)__builtin_amdgcn_readlane((int)base, 0) + incl - c;
#pragma unroll
      for (int r = 0; r < kR; ++r) {
        if ((pm >> r) & 1u) {
          if (o < (uint32_t)ovf_cap) ovf[o] = k64[r];
          ++o;
        }
      }
    };
    uint32_t fi = wave;
    Blk c0, c1;
    load_blk(fi, c0);
    load_blk(fi + kW, c1);
    while (fi < nflag) {
      Blk n0, n1;
      load_blk(fi + 2 * kW, n0);
      load_blk(fi + 3 * kW, n1);
      append_blk(c0);
      if (fi + kW < nflag) append_blk(c1);
      fi += 2 * kW;
      c0 = n0;
      c1 = n1;
    }
    __threadfence_block();
    __syncthreads();
    cs.ns = 0;
    cs.novf = f.novf;
    __syncthreads();
    if (cs.novf <= (uint32_t)kCandCap) {
      uint64_t v[kPer];
      load_candidates<NT>(cs, v);
      T = select_regs<true>(v, (uint32_t)K, f);
    } else {
      T = select_global(cs, (uint32_t)K, f);
    }
  }
  // ascending order: bucket the K entries by score block, then rank each within its bucket
  const uint64_t* sel = f.sel;
  for (int b = tid; b < nb; b += NT) ol.pre[b] = 0;
  __syncthreads();
  const uint32_t last = (uint32_t)nb - 1;
  for (int i = tid; i < K; i += NT) atomicAdd(&ol.pre[min((uint32_t)key_entry(sel[i]) >> 10, last)], 1u);
  __syncthreads();
  {
    uint32_t c[kBpt], sum = 0;
#pragma unroll
    for (int i = 0; i < kBpt; ++i) {
      const int b = kBpt * tid + i;
      c[i] = b < nb ? ol.pre[b] : 0u;
      sum += c[i];
    }
    uint32_t tot;
    uint32_t off = block_exclusive_scan<NT>(sum, f.tmp, &tot);
#pragma unroll
    for (int i = 0; i < kBpt; ++i) {
      const int b = kBpt * tid + i;
      if (b <= nb) ol.pre[b] = off;  // b == nb receives the total K
      if (b < nb) ol.cur[b] = off;
      off += c[i];
    }
    if (tid == 0) ol.pre[nb] = tot;
  }
  __syncthreads();
  for (int i = tid; i < K; i += NT) {
    const int32_t j = key_entry(sel[i]);
    ol.bucket[min(atomicAdd(&ol.cur[min((uint32_t)j >> 10, last)], 1u), (uint32_t)K - 1)] = j;
  }
  __syncthreads();
  int32_t* sorted = reinterpret_cast<int32_t*>(f.h);
  for (int i = tid; i < K; i += NT) {
    const int32_t j = ol.bucket[i];
    const uint32_t b = min((uint32_t)j >> 10, last);
    const uint32_t s0 = ol.pre[b], s1 = ol.pre[b + 1];
    // rank among the bucket's entries, read four at a time from the aligned words covering it
    uint32_t r = 0;
    for (uint32_t s = s0 & ~3u; s < s1; s += 4) {
      const int4 w = *reinterpret_cast<const int4*>(ol.bucket + s);
      r += (s >= s0 && w.x < j) + (s + 1 >= s0 && s + 1 < s1 && w.y < j) + (s + 2 >= s0 && s + 2 < s1 && w.z < j) +
           (s + 3 >= s0 && s + 3 < s1 && w.w < j);
    }
    sorted[min(s0 + r, (uint32_t)K - 1)] = j;
  }
  __syncthreads();
  for (int i = tid; i < K; i += NT) out[i] = sorted[i] + jo;
}

}  // namespace
}  // namespace hca
