// Arg-top-k per row of scores (ACRE §2.4 Eq. 16; InfoFlow §4.2 global budget).
//
// Order: score descending, ties by smaller index.  Scores become 32-bit keys
// whose unsigned order is the float order (-0 folded onto +0), so selection
// is exact integer work.  One workgroup per row:
//  1. the k-th largest key K*, and how many keys equal to K* are kept
//     (need_eq), from histograms over the row's own key range [lo, hi]:
//     2048 bins, bin = (key - base) >> shift (monotone in the key); each pass
//     narrows the range to the bin that holds the k-th largest key, until
//     that bin holds at most 256 keys (then ranked exactly against each
//     other) or a single key value.  At most three passes.
//  2. each thread counts keys > K* and == K* over a contiguous slice of
//     indices; a block-wide exclusive scan of both counts gives every kept
//     index its output slot, so the kept set is written in ascending index
//     order with no sort.
// Rows of up to 64 * 1024 scores keep each thread's slice in registers and
// read the scores once, with 16-byte loads that are all in flight together;
// longer rows read them again for every pass (coalesced reads of a row the L2
// holds), since their slices would not fit in the registers of a 1024-thread
// workgroup.
#include "common.h"
#include "internal.h"

namespace kvsel {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kFastBits = 11;
constexpr int kFastBins = 1 << kFastBits;
constexpr int kFastCand = 256;
constexpr int kRegKeys = 64;   // keys per thread held in registers, at most
static_assert(kFastBins == 2 * kThreads, "two bins per thread in the bin scan");
static_assert(kFastCand <= kThreads, "one candidate per thread in the ranking");

__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;  // -0 ranks with +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

struct TopkShared {
  uint32_t hist[kFastBins];
  uint32_t scan_a[kWaves], scan_b[kWaves];
  uint32_t lo[kWaves], hi[kWaves];
  uint32_t bin, rank, count, ncand, kstar, need;
  uint32_t tot[2];
  uint32_t cand[kFastCand];
};

// Exclusive scan of (a, b) over the block; returns the prefix of this thread
// (and, where tot is given, the block totals in tot[0], tot[1]).
__device__ __forceinline__ void block_exclusive_scan2(uint32_t a, uint32_t b, uint32_t& pa,
                                                      uint32_t& pb, uint32_t* sa, uint32_t* sb,
                                                      uint32_t* tot = nullptr) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  uint32_t ia = a, ib = b;  // inclusive within the wave
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t ta = __shfl_up(ia, off, 64);
    const uint32_t tb = __shfl_up(ib, off, 64);
    if (lane >= off) { ia += ta; ib += tb; }
  }
  if (lane == 63) { sa[wave] = ia; sb[wave] = ib; }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t ca = 0, cb = 0;
    for (int w = 0; w < kWaves; ++w) {
      const uint32_t xa = sa[w], xb = sb[w];
      sa[w] = ca; sb[w] = cb;
      ca += xa; cb += xb;
    }
    if (tot != nullptr) { tot[0] = ca; tot[1] = cb; }
  }
  __syncthreads();
  pa = sa[wave] + ia - a;
  pb = sb[wave] + ib - b;
}

// Row indices stay below 2^31 (the int32 output), so a slice's indices and
// counts are 32-bit: 64-bit index arithmetic per unrolled key would cost
// registers.  The number of a slice's KPT indices from i0 that lie in a row
// of M:
template <int KPT>
__device__ __forceinline__ int slice_valid(uint32_t i0, uint32_t M) {
  return i0 >= M ? 0 : static_cast<int>(min(static_cast<uint32_t>(KPT), M - i0));
}

// Keys of a row held in registers: this thread's slice of KPT indices, the
// first nv of them inside the row.
template <int KPT>
struct RegKeys {
  uint32_t key[KPT];
  int nv;
  template <typename F>
  __device__ __forceinline__ void each(F f) const {
#pragma unroll
    for (int e = 0; e < KPT; ++e) f(e < nv, key[e]);
  }
};

// Loads issued together before their keys are used: a thread's reads are
// independent, so kBatch of them are in flight instead of one.
constexpr int kBatch = 16;

// Keys of a row read for every pass: indices threadIdx.x + r * kThreads.
struct StreamKeys {
  const float* s;
  uint32_t M;
  template <typename F>
  __device__ __forceinline__ void each(F f) const {
    for (uint32_t i0 = threadIdx.x; i0 < M; i0 += kBatch * kThreads) {
      uint32_t key[kBatch];
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const uint32_t i = i0 + static_cast<uint32_t>(b) * kThreads;
        key[b] = i < M ? order_key(s[i]) : 0u;
      }
#pragma unroll
      for (int b = 0; b < kBatch; ++b) f(i0 + static_cast<uint32_t>(b) * kThreads < M, key[b]);
    }
  }
};

// Step 1: K* and need_eq of the k-th largest key (1 <= k <= M).  Every
// thread of the block calls it and gets the same two values.
template <typename Keys>
__device__ __forceinline__ void range_select(const Keys& keys, uint32_t k, TopkShared& sm,
                                             uint32_t& kstar, uint32_t& need_eq) {
  const int wave = threadIdx.x >> 6;
  uint32_t lo = 0xffffffffu, hi = 0u;
  keys.each([&](bool valid, uint32_t key) {
    if (valid) {
      lo = min(lo, key);
      hi = max(hi, key);
    }
  });
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    lo = min(lo, static_cast<uint32_t>(__shfl_xor(static_cast<int>(lo), off, 64)));
    hi = max(hi, static_cast<uint32_t>(__shfl_xor(static_cast<int>(hi), off, 64)));
  }
  if ((threadIdx.x & 63) == 0) { sm.lo[wave] = lo; sm.hi[wave] = hi; }
  if (threadIdx.x == 0) sm.ncand = 0;
  __syncthreads();
  lo = sm.lo[0];
  hi = sm.hi[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) {
    lo = min(lo, sm.lo[w]);
    hi = max(hi, sm.hi[w]);
  }
  // The current range holds the keys with base <= key and key - base < span
  // (span = 2^bits, then the previous pass's bin width); its bins are
  // (key - base) >> sh, kFastBins of them at most.
  const uint32_t range = hi - lo;
  const int bits = range == 0u ? 0 : 32 - __clz(static_cast<int>(range));
  uint32_t base = lo;
  uint64_t span = uint64_t{1} << bits;
  int sh = bits > kFastBits ? bits - kFastBits : 0;
  uint32_t rank = k, fbin = 0, fcount = 0;
  for (;;) {
    for (int i = threadIdx.x; i < kFastBins; i += kThreads) sm.hist[i] = 0;
    __syncthreads();
    keys.each([&](bool valid, uint32_t key) {
      const uint32_t d = key - base;
      if (valid && key >= base && d < span) atomicAdd(&sm.hist[d >> sh], 1u);
    });
    __syncthreads();
    // bins from the top: thread t owns bins 2047 - 2t and 2046 - 2t; exactly
    // one bin b has above(b) < rank <= above(b) + count(b), since the range
    // holds at least `rank` keys
    const uint32_t c0 = sm.hist[kFastBins - 1 - 2 * threadIdx.x];
    const uint32_t c1 = sm.hist[kFastBins - 2 - 2 * threadIdx.x];
    uint32_t above, unused;
    block_exclusive_scan2(c0 + c1, 0u, above, unused, sm.scan_a, sm.scan_b);
    if (above < rank && rank <= above + c0) {
      sm.bin = kFastBins - 1 - 2 * threadIdx.x;
      sm.rank = rank - above;
      sm.count = c0;
    } else if (above + c0 < rank && rank <= above + c0 + c1) {
      sm.bin = kFastBins - 2 - 2 * threadIdx.x;
      sm.rank = rank - above - c0;
      sm.count = c1;
    }
    __syncthreads();
    fbin = sm.bin;
    rank = sm.rank;
    fcount = sm.count;
    if (fcount <= kFastCand || sh == 0) break;
    base += fbin << sh;
    span = uint64_t{1} << sh;
    sh = sh > kFastBits ? sh - kFastBits : 0;
    __syncthreads();               // every thread has read hist and sm.* before they change
  }
  if (sh == 0) {
    // the bin is one key value
    kstar = base + fbin;
    need_eq = rank;
    return;
  }
  // at most kFastCand keys: each one's exact rank among them; K* is the key
  // with (# greater) < rank <= (# greater or equal)
  keys.each([&](bool valid, uint32_t key) {
    const uint32_t d = key - base;
    if (valid && key >= base && d < span && (d >> sh) == fbin)
      sm.cand[atomicAdd(&sm.ncand, 1u)] = key;
  });
  __syncthreads();
  if (threadIdx.x < fcount) {
    const uint32_t x = sm.cand[threadIdx.x];
    uint32_t gt = 0, ge = 0;
    for (uint32_t j = 0; j < fcount; ++j) {
      const uint32_t y = sm.cand[j];
      gt += y > x;
      ge += y >= x;
    }
    // keys equal to K* all write the same two values
    if (gt < rank && rank <= ge) { sm.kstar = x; sm.need = rank - gt; }
  }
  __syncthreads();
  kstar = sm.kstar;
  need_eq = sm.need;
}

// KPT consecutive keys of indices i0 .. i0 + KPT - 1, the first nv inside the
// row (the rest read as 0).
template <int KPT>
__device__ __forceinline__ void load_slice(const float* s, uint32_t i0, int nv,
                                           uint32_t (&key)[KPT]) {
  if (KPT % 4 == 0 && nv == KPT && (reinterpret_cast<uintptr_t>(s + i0) & 15u) == 0) {
    // a whole 16-byte aligned slice: vector loads (a quarter of the requests)
#pragma unroll
    for (int e = 0; e < KPT; e += 4) {
      const float4 v = *reinterpret_cast<const float4*>(s + i0 + e);
      key[e] = order_key(v.x);
      if constexpr (KPT % 4 == 0) {
        key[e + 1] = order_key(v.y);
        key[e + 2] = order_key(v.z);
        key[e + 3] = order_key(v.w);
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < KPT; ++e) key[e] = e < nv ? order_key(s[i0 + e]) : 0u;
  }
}

// Step 2 for one tile of kThreads * KPT indices starting at tile0: thread t
// owns the slice tile0 + t * KPT .. + KPT - 1.  gt_run / eq_run count the kept
// keys (> K*, == K*) of earlier tiles and are advanced past this one.
template <int KPT>
__device__ __forceinline__ void write_tile(const uint32_t (&key)[KPT], uint32_t tile0, int nv,
                                           uint32_t kstar, uint32_t need_eq, uint32_t& gt_run,
                                           uint32_t& eq_run, TopkShared& sm, const float* s,
                                           int32_t* out_i, float* out_v) {
  const uint32_t i0 = tile0 + threadIdx.x * KPT;
  uint32_t n_gt = 0, n_eq = 0;
#pragma unroll
  for (int e = 0; e < KPT; ++e) {
    const bool in = e < nv;
    n_gt += in && key[e] > kstar;
    n_eq += in && key[e] == kstar;
  }
  uint32_t gt_before, eq_before;
  block_exclusive_scan2(n_gt, n_eq, gt_before, eq_before, sm.scan_a, sm.scan_b, sm.tot);
  const uint32_t tile_gt = sm.tot[0], tile_eq = sm.tot[1];
  gt_before += gt_run;
  eq_before += eq_run;
#pragma unroll
  for (int e = 0; e < KPT; ++e) {   // a fixed trip count, so the keys stay in registers
    const bool in = e < nv;
    if (in && key[e] > kstar) {
      const uint32_t pos = gt_before + min(eq_before, need_eq);
      out_i[pos] = static_cast<int32_t>(i0 + e);
      if (out_v) out_v[pos] = s[i0 + e];
      ++gt_before;
    } else if (in && key[e] == kstar) {
      if (eq_before < need_eq) {
        const uint32_t pos = gt_before + eq_before;
        out_i[pos] = static_cast<int32_t>(i0 + e);
        if (out_v) out_v[pos] = s[i0 + e];
      }
      ++eq_before;
    }
  }
  gt_run += tile_gt;
  eq_run += tile_eq;
  __syncthreads();                 // scan_a/b and tot are free for the next tile
}

// Rows of up to KPT * 1024 scores (KPT <= kRegKeys): each thread keeps its
// contiguous slice of KPT keys in registers, so the scores are read once and
// compacted in one tile.
template <int KPT>
__global__ void __launch_bounds__(kThreads)
topk_reg_kernel(const float* __restrict__ score, int64_t M, int64_t k, int32_t* __restrict__ idx,
                float* __restrict__ val) {
  __shared__ TopkShared sm;
  const float* s = score + static_cast<int64_t>(blockIdx.x) * M;
  int32_t* out_i = idx + static_cast<int64_t>(blockIdx.x) * k;
  float* out_v = val ? val + static_cast<int64_t>(blockIdx.x) * k : nullptr;
  RegKeys<KPT> keys;
  const uint32_t i0 = threadIdx.x * KPT;
  keys.nv = slice_valid<KPT>(i0, static_cast<uint32_t>(M));
  load_slice<KPT>(s, i0, keys.nv, keys.key);
  uint32_t kstar, need_eq;
  range_select(keys, static_cast<uint32_t>(k), sm, kstar, need_eq);
  uint32_t gt_run = 0, eq_run = 0;
  write_tile<KPT>(keys.key, 0u, keys.nv, kstar, need_eq, gt_run, eq_run, sm, s, out_i, out_v);
}

// Longer rows: the selection reads the row again for every pass; the
// compaction walks tiles of kThreads * kRegKeys scores, each read once.
__global__ void __launch_bounds__(kThreads)
topk_stream_kernel(const float* __restrict__ score, int64_t M, int64_t k,
                   int32_t* __restrict__ idx, float* __restrict__ val) {
  __shared__ TopkShared sm;
  const float* s = score + static_cast<int64_t>(blockIdx.x) * M;
  int32_t* out_i = idx + static_cast<int64_t>(blockIdx.x) * k;
  float* out_v = val ? val + static_cast<int64_t>(blockIdx.x) * k : nullptr;
  uint32_t kstar, need_eq;
  const uint32_t m = static_cast<uint32_t>(M);
  range_select(StreamKeys{s, m}, static_cast<uint32_t>(k), sm, kstar, need_eq);

  // tiles of kThreads * kRegKeys indices, in ascending order
  uint32_t gt_run = 0, eq_run = 0;
  for (uint32_t tile0 = 0; tile0 < m; tile0 += kThreads * kRegKeys) {
    uint32_t key[kRegKeys];
    const uint32_t i0 = tile0 + threadIdx.x * kRegKeys;
    const int nv = slice_valid<kRegKeys>(i0, m);
    load_slice<kRegKeys>(s, i0, nv, key);
    write_tile<kRegKeys>(key, tile0, nv, kstar, need_eq, gt_run, eq_run, sm, s, out_i, out_v);
  }
}

// out[g][j] = src[g][idx[g][j]]: composes two index lists, e.g. the
// positions kept in the current list with the list itself (CacheFocus §2.4:
// the cache IDs left after a pruning layer).  Indices outside [0, m) give -1.
constexpr int kTakeThreads = 256;

__global__ void __launch_bounds__(kTakeThreads)
take_kernel(const int32_t* __restrict__ src, int64_t m, const int32_t* __restrict__ idx,
            int64_t k, int64_t total, int32_t* __restrict__ out) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * kTakeThreads + threadIdx.x;
  if (e >= total) return;
  const int64_t g = e / k;
  const int32_t i = idx[e];
  out[e] = (i >= 0 && i < m) ? src[g * m + i] : -1;
}

// Lists the k given indices of each row by their scores (CacheFocus §2.5,
// attention-guided "sort" placement): an entry's rank is the number of
// entries before it in the order (score descending, index ascending,
// position in the list ascending), which is a permutation of 0..k-1; rank r
// goes to slot r (descending) or k-1-r (ascending).  Every thread ranks one
// entry against all k of its row, read through LDS tiles: O(k^2) compares,
// exact integer work on the same keys as the top-k.  Indices outside [0, M)
// rank as the lowest key and get value 0.
constexpr int kOrderThreads = 256;
constexpr int kOrderTile = 1024;

__global__ void __launch_bounds__(kOrderThreads)
order_kernel(const float* __restrict__ score, int64_t M, const int32_t* __restrict__ idx,
             int64_t k, int64_t jblocks, int descending, int32_t* __restrict__ idx_out,
             float* __restrict__ val_out) {
  __shared__ uint32_t skey[kOrderTile];
  __shared__ int32_t sidx[kOrderTile];
  const int64_t g = blockIdx.x / static_cast<uint32_t>(jblocks);   // 32-bit: the grid is below 2^32 workgroups
  const int64_t j = static_cast<int64_t>(blockIdx.x % static_cast<uint32_t>(jblocks)) * kOrderThreads + threadIdx.x;
  const int32_t* in = idx + g * k;
  const float* sc = score + g * M;
  auto key_of = [&](int32_t i) -> uint32_t { return (i >= 0 && i < M) ? order_key(sc[i]) : 0u; };
  const bool mine = j < k;
  const int32_t my_i = mine ? in[j] : 0;
  const uint32_t my_key = mine ? key_of(my_i) : 0u;
  int64_t rank = 0;
  for (int64_t t0 = 0; t0 < k; t0 += kOrderTile) {
    const int n = static_cast<int>(min<int64_t>(kOrderTile, k - t0));
    __syncthreads();  // previous tile fully read
    for (int e = threadIdx.x; e < n; e += kOrderThreads) {
      const int32_t i = in[t0 + e];
      sidx[e] = i;
      skey[e] = key_of(i);
    }
    __syncthreads();
    if (mine) {
      for (int e = 0; e < n; ++e) {
        const uint32_t ke = skey[e];
        const int32_t ie = sidx[e];
        rank += (ke > my_key) || (ke == my_key && (ie < my_i || (ie == my_i && t0 + e < j)));
      }
    }
  }
  if (mine) {
    const int64_t pos = g * k + (descending ? rank : k - 1 - rank);
    idx_out[pos] = my_i;
    if (val_out) val_out[pos] = (my_i >= 0 && my_i < M) ? sc[my_i] : 0.0f;
  }
}

// r[g][u] = |sel_g ∩ unit u| / unit_len (InfoFlow §4.3, the share of chunk
// u's tokens in a selection): one work-item per (row, unit) counts the
// ascending index list between the unit's bounds with two binary searches.
constexpr int kFracThreads = 256;

__device__ __forceinline__ int64_t lower_bound_i32(const int32_t* a, int64_t n, int64_t x) {
  int64_t lo = 0, hi = n;
  while (lo < hi) {
    const int64_t mid = (lo + hi) >> 1;
    if (a[mid] < x) lo = mid + 1; else hi = mid;
  }
  return lo;
}

__global__ void __launch_bounds__(kFracThreads)
unit_fractions_kernel(const int32_t* __restrict__ sel, int64_t k, int64_t unit_len, int64_t M,
                      int64_t total, float* __restrict__ r) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * kFracThreads + threadIdx.x;
  if (e >= total) return;
  const int64_t g = e / M, u = e % M;
  const int32_t* s = sel + g * k;
  const int64_t n = lower_bound_i32(s, k, (u + 1) * unit_len) - lower_bound_i32(s, k, u * unit_len);
  r[e] = static_cast<float>(n) / static_cast<float>(unit_len);
}

// delta[g * rep + i][order[g][p]] = base + p * unit_len for i < rep: the start
// of each unit once the units are concatenated in `order` (InfoFlow §4.3,
// GLOBAL positions rebuilt for the new order).  Entries outside [0, M) are
// skipped.
__global__ void __launch_bounds__(kFracThreads)
slot_starts_kernel(const int32_t* __restrict__ order, int64_t M, int64_t unit_len, int64_t base,
                   int64_t rep, int64_t total, int64_t* __restrict__ delta) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * kFracThreads + threadIdx.x;
  if (e >= total) return;
  const int64_t g = e / M, p = e % M;
  const int32_t c = order[e];
  if (c < 0 || c >= M) return;
  for (int64_t i = 0; i < rep; ++i) delta[(g * rep + i) * M + c] = base + p * unit_len;
}

}  // namespace

int launch_unit_fractions(const int32_t* sel, int64_t G, int64_t k, int64_t unit_len, int64_t M,
                          float* r, hipStream_t s) {
  const int64_t total = G * M;
  hipLaunchKernelGGL(unit_fractions_kernel, dim3(static_cast<unsigned>((total + kFracThreads - 1) / kFracThreads)),
                     dim3(kFracThreads), 0, s, sel, k, unit_len, M, total, r);
  return check_launch("kvsel_unit_fractions");
}

int launch_slot_starts(const int32_t* order, int64_t G, int64_t M, int64_t unit_len, int64_t base,
                       int64_t rep, int64_t* delta, hipStream_t s) {
  const int64_t total = G * M;
  hipLaunchKernelGGL(slot_starts_kernel, dim3(static_cast<unsigned>((total + kFracThreads - 1) / kFracThreads)),
                     dim3(kFracThreads), 0, s, order, M, unit_len, base, rep, total, delta);
  return check_launch("kvsel_slot_starts");
}

int launch_take(const int32_t* src, int64_t G, int64_t m, const int32_t* idx, int64_t k,
                int32_t* out, hipStream_t s) {
  const int64_t total = G * k;
  const int64_t blocks = (total + kTakeThreads - 1) / kTakeThreads;
  hipLaunchKernelGGL(take_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kTakeThreads), 0, s,
                     src, m, idx, k, total, out);
  return check_launch("kvsel_take");
}

int launch_order(const float* score, int64_t G, int64_t M, const int32_t* idx, int64_t k,
                 int descending, int32_t* idx_out, float* val_out, hipStream_t s) {
  const int64_t jblocks = (k + kOrderThreads - 1) / kOrderThreads;
  hipLaunchKernelGGL(order_kernel, dim3(static_cast<unsigned>(G * jblocks)), dim3(kOrderThreads),
                     0, s, score, M, idx, k, jblocks, descending, idx_out, val_out);
  return check_launch("kvsel_order");
}

int launch_topk(const float* score, int64_t G, int64_t M, int64_t k, int32_t* idx, float* val,
                hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(G)), block(kThreads);
  const int64_t per = (M + kThreads - 1) / kThreads;
#define KVSEL_TK(KPT) \
  if (per <= KPT) { hipLaunchKernelGGL(topk_reg_kernel<KPT>, grid, block, 0, s, score, M, k, idx, val); return check_launch("kvsel_topk"); }
  KVSEL_TK(1) KVSEL_TK(2) KVSEL_TK(4) KVSEL_TK(8) KVSEL_TK(16) KVSEL_TK(32) KVSEL_TK(64)
#undef KVSEL_TK
  static_assert(kRegKeys == 64, "the register variants above end at kRegKeys");
  hipLaunchKernelGGL(topk_stream_kernel, grid, block, 0, s, score, M, k, idx, val);
  return check_launch("kvsel_topk");
}

}  // namespace kvsel
