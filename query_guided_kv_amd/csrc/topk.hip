// Arg-top-k per row of scores (ACRE §2.4 Eq. 16; InfoFlow §4.2 global budget).
//
// Order: score descending, ties by smaller index.  Scores become 32-bit keys
// whose unsigned order is the float order (-0 folded onto +0), so selection
// is exact integer work.  One workgroup per row:
//  1. radix select, 4 passes of 8 bits with an LDS histogram, finds the k-th
//     largest key K* and how many keys equal to K* are kept (need_eq);
//  2. each thread counts keys > K* and == K* over a contiguous slice of
//     indices; a block-wide exclusive scan of both counts gives every kept
//     index its output slot, so the kept set is written in ascending index
//     order with no sort.
#include "common.h"
#include "internal.h"

namespace kvsel {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;

__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;  // -0 ranks with +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive scan of (a, b) over the block; returns the prefix of this thread.
__device__ __forceinline__ void block_exclusive_scan2(uint32_t a, uint32_t b, uint32_t& pa,
                                                      uint32_t& pb, uint32_t* sa, uint32_t* sb) {
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
  }
  __syncthreads();
  pa = sa[wave] + ia - a;
  pb = sb[wave] + ib - b;
}

// Pick the digit of the k-th largest key from a 256-bin histogram (one wave,
// threadIdx.x < 64): lane l owns bins 255-4l .. 252-4l (high to low); an
// exclusive scan of the lanes' counts gives the number of keys in higher bins,
// and the one bin with above < rank <= above + count publishes the new prefix
// and the rank left inside that bin.
__device__ __forceinline__ void select_bin(const uint32_t* h, uint32_t rank, uint32_t prefix,
                                           int shift, uint32_t* sh_prefix, uint32_t* sh_rank) {
  const int lane = threadIdx.x;
  uint32_t c[4], tot = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    c[j] = h[255 - 4 * lane - j];
    tot += c[j];
  }
  uint32_t incl = tot;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t t = __shfl_up(incl, off, 64);
    if (lane >= off) incl += t;
  }
  uint32_t above = incl - tot;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (above < rank && rank <= above + c[j]) {
      *sh_prefix = prefix | (static_cast<uint32_t>(255 - 4 * lane - j) << shift);
      *sh_rank = rank - above;
    }
    above += c[j];
  }
}

// Count `bin` into this wave's histogram.  Scores of one row share most of
// their leading bits, so the lanes of a wave mostly hit the same bin: the
// lanes with the first active lane's bin add their count once (ballot +
// popcount), the rest add one by one.  Integer counts: exact in any order.
__device__ __forceinline__ void count_bin(uint32_t* hist, uint32_t bin, bool active) {
  const uint64_t act = __ballot(active);
  if (act == 0) return;
  const int first = __builtin_ctzll(act);
  const uint32_t lead = __shfl(bin, first, 64);
  const bool same = active && bin == lead;
  const uint64_t grp = __ballot(same);
  const int lane = threadIdx.x & 63;
  if (lane == first) atomicAdd(&hist[lead], static_cast<uint32_t>(__popcll(grp)));
  if (active && !same) atomicAdd(&hist[bin], 1u);
}

__global__ void __launch_bounds__(kThreads)
topk_kernel(const float* __restrict__ score, int64_t M, int64_t k, int32_t* __restrict__ idx,
            float* __restrict__ val) {
  __shared__ uint32_t hist[kWaves][256];
  __shared__ uint32_t sh_prefix, sh_rank;
  __shared__ uint32_t scan_a[kWaves], scan_b[kWaves];
  const float* s = score + static_cast<int64_t>(blockIdx.x) * M;
  int32_t* out_i = idx + static_cast<int64_t>(blockIdx.x) * k;
  float* out_v = val ? val + static_cast<int64_t>(blockIdx.x) * k : nullptr;
  const int wave = threadIdx.x >> 6;

  // 1. radix select of the k-th largest key, 8 bits per pass, one histogram
  //    per wave merged in a fixed order
  uint32_t prefix = 0, mask = 0, rank = static_cast<uint32_t>(k);
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < kWaves * 256; i += kThreads) (&hist[0][0])[i] = 0;
    __syncthreads();
    const int64_t rounds = (M + kThreads - 1) / kThreads;
    for (int64_t rd = 0; rd < rounds; ++rd) {
      const int64_t i = rd * kThreads + threadIdx.x;
      uint32_t key = 0;
      bool act = false;
      if (i < M) {
        key = order_key(s[i]);
        act = (key & mask) == prefix;
      }
      count_bin(hist[wave], (key >> shift) & 255u, act);
    }
    __syncthreads();
    if (threadIdx.x < 256) {
      uint32_t t = 0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) t += hist[w][threadIdx.x];
      hist[0][threadIdx.x] = t;   // each thread reads and writes its own bin only
    }
    __syncthreads();
    if (threadIdx.x < 64) select_bin(hist[0], rank, prefix, shift, &sh_prefix, &sh_rank);
    __syncthreads();
    rank = sh_rank;
    prefix = sh_prefix;
    mask |= 255u << shift;
  }
  const uint32_t kstar = prefix;
  const uint32_t need_eq = rank;  // keys equal to K* that are kept

  // 2. ordered compaction over contiguous index slices
  const int64_t per = (M + kThreads - 1) / kThreads;
  const int64_t i0 = min(M, threadIdx.x * per);
  const int64_t i1 = min(M, i0 + per);
  uint32_t n_gt = 0, n_eq = 0;
  for (int64_t i = i0; i < i1; ++i) {
    const uint32_t key = order_key(s[i]);
    n_gt += key > kstar;
    n_eq += key == kstar;
  }
  uint32_t gt_before, eq_before;
  block_exclusive_scan2(n_gt, n_eq, gt_before, eq_before, scan_a, scan_b);
  for (int64_t i = i0; i < i1; ++i) {
    const float x = s[i];
    const uint32_t key = order_key(x);
    if (key > kstar) {
      const uint32_t pos = gt_before + min(eq_before, need_eq);
      out_i[pos] = static_cast<int32_t>(i);
      if (out_v) out_v[pos] = x;
      ++gt_before;
    } else if (key == kstar) {
      if (eq_before < need_eq) {
        const uint32_t pos = gt_before + eq_before;
        out_i[pos] = static_cast<int32_t>(i);
        if (out_v) out_v[pos] = x;
      }
      ++eq_before;
    }
  }
}

// Rows of up to 64 * 1024 scores: each thread keeps its contiguous slice of
// KPT keys in registers, so the four radix passes and the ordered compaction
// read the scores once.
template <int KPT>
__global__ void __launch_bounds__(kThreads)
topk_reg_kernel(const float* __restrict__ score, int64_t M, int64_t k, int32_t* __restrict__ idx,
                float* __restrict__ val) {
  __shared__ uint32_t hist[kWaves][256];
  __shared__ uint32_t sh_prefix, sh_rank;
  __shared__ uint32_t scan_a[kWaves], scan_b[kWaves];
  const float* s = score + static_cast<int64_t>(blockIdx.x) * M;
  int32_t* out_i = idx + static_cast<int64_t>(blockIdx.x) * k;
  float* out_v = val ? val + static_cast<int64_t>(blockIdx.x) * k : nullptr;
  const int wave = threadIdx.x >> 6;
  const int64_t i0 = static_cast<int64_t>(threadIdx.x) * KPT;

  uint32_t key[KPT];
#pragma unroll
  for (int e = 0; e < KPT; ++e) key[e] = i0 + e < M ? order_key(s[i0 + e]) : 0u;

  uint32_t prefix = 0, mask = 0, rank = static_cast<uint32_t>(k);
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < kWaves * 256; i += kThreads) (&hist[0][0])[i] = 0;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < KPT; ++e)
      count_bin(hist[wave], (key[e] >> shift) & 255u, i0 + e < M && (key[e] & mask) == prefix);
    __syncthreads();
    if (threadIdx.x < 256) {
      uint32_t t = 0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) t += hist[w][threadIdx.x];
      hist[0][threadIdx.x] = t;
    }
    __syncthreads();
    if (threadIdx.x < 64) select_bin(hist[0], rank, prefix, shift, &sh_prefix, &sh_rank);
    __syncthreads();
    rank = sh_rank;
    prefix = sh_prefix;
    mask |= 255u << shift;
  }
  const uint32_t kstar = prefix;
  const uint32_t need_eq = rank;

  uint32_t n_gt = 0, n_eq = 0;
#pragma unroll
  for (int e = 0; e < KPT; ++e) {
    const bool in = i0 + e < M;
    n_gt += in && key[e] > kstar;
    n_eq += in && key[e] == kstar;
  }
  uint32_t gt_before, eq_before;
  block_exclusive_scan2(n_gt, n_eq, gt_before, eq_before, scan_a, scan_b);
#pragma unroll
  for (int e = 0; e < KPT; ++e) {
    if (i0 + e >= M) break;
    if (key[e] > kstar) {
      const uint32_t pos = gt_before + min(eq_before, need_eq);
      out_i[pos] = static_cast<int32_t>(i0 + e);
      if (out_v) out_v[pos] = s[i0 + e];
      ++gt_before;
    } else if (key[e] == kstar) {
      if (eq_before < need_eq) {
        const uint32_t pos = gt_before + eq_before;
        out_i[pos] = static_cast<int32_t>(i0 + e);
        if (out_v) out_v[pos] = s[i0 + e];
      }
      ++eq_before;
    }
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
  const int64_t g = blockIdx.x / jblocks;
  const int64_t j = (blockIdx.x % jblocks) * kOrderThreads + threadIdx.x;
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
  hipLaunchKernelGGL(topk_kernel, grid, block, 0, s, score, M, k, idx, val);
  return check_launch("kvsel_topk");
}

}  // namespace kvsel
