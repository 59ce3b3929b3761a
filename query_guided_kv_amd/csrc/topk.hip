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

__global__ void __launch_bounds__(kThreads)
topk_kernel(const float* __restrict__ score, int64_t M, int64_t k, int32_t* __restrict__ idx,
            float* __restrict__ val) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sh_prefix, sh_rank;
  __shared__ uint32_t scan_a[kWaves], scan_b[kWaves];
  const float* s = score + static_cast<int64_t>(blockIdx.x) * M;
  int32_t* out_i = idx + static_cast<int64_t>(blockIdx.x) * k;
  float* out_v = val ? val + static_cast<int64_t>(blockIdx.x) * k : nullptr;

  // 1. radix select of the k-th largest key
  uint32_t prefix = 0, mask = 0, rank = static_cast<uint32_t>(k);
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (threadIdx.x < 256) hist[threadIdx.x] = 0;
    __syncthreads();
    for (int64_t i = threadIdx.x; i < M; i += kThreads) {
      const uint32_t key = order_key(s[i]);
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t above = 0;
      int bin = 255;
      for (; bin > 0; --bin) {
        if (above + hist[bin] >= rank) break;
        above += hist[bin];
      }
      sh_rank = rank - above;
      sh_prefix = prefix | (static_cast<uint32_t>(bin) << shift);
    }
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

}  // namespace

int launch_topk(const float* score, int64_t G, int64_t M, int64_t k, int32_t* idx, float* val,
                hipStream_t s) {
  hipLaunchKernelGGL(topk_kernel, dim3(static_cast<unsigned>(G)), dim3(kThreads), 0, s, score, M,
                     k, idx, val);
  return check_launch("kvsel_topk");
}

}  // namespace kvsel
