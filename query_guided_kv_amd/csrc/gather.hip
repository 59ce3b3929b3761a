// Gather / refill of the kept units (ACRE §2.4 Eq. 18-19; CacheFocus §2.4
// final cache, §2.5 "align" re-positioning).
//
// gather_kernel: one workgroup copies a chunk of rows of one kept unit of one
// instance, as 16-byte vectors.  Compact layout puts the r-th kept unit at
// rows [r*U, (r+1)*U); the nested layout of Eq. 18-19 puts it right before its
// proxy entry j, i.e. at rows [j + r*U, j + (r+1)*U).  With `align`, keys are
// rotated on the way so that unit r lands at positions align_base + r*U + t.
//
// proxy_copy_kernel (nested layout only): proxy entry j goes to row
// j + U * (number of kept entries <= j), found by binary search in the
// ascending index list.
#include "common.h"
#include "internal.h"

#include <algorithm>

namespace kvsel {
namespace {

constexpr int kThreads = 256;

template <typename T, int D, int STYLE, bool ALIGN, bool NESTED>
__global__ void __launch_bounds__(kThreads)
gather_kernel(const T* __restrict__ ksrc, const T* __restrict__ vsrc, int H, int64_t stride_b,
              int64_t stride_n, int64_t U, const int32_t* __restrict__ idx, int64_t k,
              int64_t idx_group, const int64_t* __restrict__ src_start, int64_t align_base,
              RopeTheta th, int64_t chunks, int64_t rows_per_chunk, int64_t dst_rows,
              int64_t M, T* __restrict__ kdst, T* __restrict__ vdst) {
  constexpr int V = Elem<T>::kPerVec;
  constexpr int HALF = D / 2;
  __shared__ double2 cs[ALIGN ? HALF : 1];

  const int64_t chunk = blockIdx.x % static_cast<uint32_t>(chunks);   // 32-bit: the grid is below 2^32 workgroups
  const uint32_t br = blockIdx.x / static_cast<uint32_t>(chunks);
  const int64_t r = br % static_cast<uint32_t>(k);
  const int64_t b = br / static_cast<uint32_t>(k);
  const int64_t u = idx[(b / idx_group) * k + r];
  if (u < 0 || u >= M) return;  // invalid index: leave the slot untouched
  const int64_t t0 = chunk * rows_per_chunk;
  const int rows = static_cast<int>(min<int64_t>(rows_per_chunk, U - t0));
  const int64_t dst_row0 = (NESTED ? u + r * U : r * U) + t0;
  const int64_t row_elems = static_cast<int64_t>(H) * D;

  if constexpr (ALIGN) {
    const int64_t delta = align_base + r * U - (src_start ? src_start[u] : 0);
    for (int i = threadIdx.x; i < HALF; i += kThreads) cs[i] = rope_cs(delta, th.t[i]);
    __syncthreads();
  }

  const T* ks = ksrc + b * stride_b + (u * U + t0) * stride_n;
  T* kd = kdst + (b * dst_rows + dst_row0) * row_elems;
  const int vecs_per_row = static_cast<int>(row_elems / V);
  if constexpr (!ALIGN) {
    const int items = rows * vecs_per_row;
    for (int it = threadIdx.x; it < items; it += kThreads) {
      const int rr = it / vecs_per_row, c = it % vecs_per_row;
      *reinterpret_cast<uint4*>(kd + rr * row_elems + c * V) =
          *reinterpret_cast<const uint4*>(ks + rr * stride_n + c * V);
    }
  } else if constexpr (STYLE == KVSEL_ROPE_HALF) {
    constexpr int VPH = HALF / V;
    const int items = rows * H * VPH;
    for (int it = threadIdx.x; it < items; it += kThreads) {
      const int c = it % VPH;
      const int rh = it / VPH;
      const int h = rh % H, rr = rh / H;
      const int64_t so = rr * stride_n + static_cast<int64_t>(h) * D + c * V;
      const int64_t dof = rr * row_elems + static_cast<int64_t>(h) * D + c * V;
      uint4 ra = *reinterpret_cast<const uint4*>(ks + so);
      uint4 rb = *reinterpret_cast<const uint4*>(ks + so + HALF);
      rope_rotate16<T, KVSEL_ROPE_HALF>(ra, rb, c * V, cs);
      *reinterpret_cast<uint4*>(kd + dof) = ra;
      *reinterpret_cast<uint4*>(kd + dof + HALF) = rb;
    }
  } else {
    const int items = rows * vecs_per_row;
    for (int it = threadIdx.x; it < items; it += kThreads) {
      const int rr = it / vecs_per_row, c = it % vecs_per_row;
      const int d0 = (c * V) % D;
      uint4 ra = *reinterpret_cast<const uint4*>(ks + rr * stride_n + c * V);
      uint4 unused;
      rope_rotate16<T, KVSEL_ROPE_INTERLEAVED>(ra, unused, d0, cs);
      *reinterpret_cast<uint4*>(kd + rr * row_elems + c * V) = ra;
    }
  }
  if (vsrc != nullptr) {
    const T* vs = vsrc + b * stride_b + (u * U + t0) * stride_n;
    T* vd = vdst + (b * dst_rows + dst_row0) * row_elems;
    const int items = rows * vecs_per_row;
    for (int it = threadIdx.x; it < items; it += kThreads) {
      const int rr = it / vecs_per_row, c = it % vecs_per_row;
      *reinterpret_cast<uint4*>(vd + rr * row_elems + c * V) =
          *reinterpret_cast<const uint4*>(vs + rr * stride_n + c * V);
    }
  }
}

constexpr int kProxyRows = 16;

template <typename T>
__global__ void __launch_bounds__(kThreads)
proxy_copy_kernel(const T* __restrict__ kp, const T* __restrict__ vp, int64_t m, int64_t row_elems,
                  int64_t pstride_b, int64_t pstride_n, int64_t U, const int32_t* __restrict__ idx,
                  int64_t k, int64_t idx_group, int64_t tiles, int64_t dst_rows,
                  T* __restrict__ kdst, T* __restrict__ vdst) {
  constexpr int V = Elem<T>::kPerVec;
  __shared__ int64_t dst_row[kProxyRows];
  const int64_t b = blockIdx.x / static_cast<uint32_t>(tiles);   // 32-bit: the grid is below 2^32 workgroups
  const int64_t j0 = static_cast<int64_t>(blockIdx.x % static_cast<uint32_t>(tiles)) * kProxyRows;
  const int rows = static_cast<int>(min<int64_t>(kProxyRows, m - j0));
  const int32_t* sel = idx + (b / idx_group) * k;
  if (threadIdx.x < rows) {
    const int64_t j = j0 + threadIdx.x;
    int64_t lo = 0, hi = k;  // number of kept indices <= j
    while (lo < hi) {
      const int64_t mid = (lo + hi) >> 1;
      if (sel[mid] <= j) lo = mid + 1; else hi = mid;
    }
    dst_row[threadIdx.x] = j + U * lo;
  }
  __syncthreads();
  const int vpr = static_cast<int>(row_elems / V);
  const int items = rows * vpr;
  for (int it = threadIdx.x; it < items; it += kThreads) {
    const int rr = it / vpr, c = it % vpr;
    const int64_t so = b * pstride_b + (j0 + rr) * pstride_n + c * V;
    const int64_t dof = (b * dst_rows + dst_row[rr]) * row_elems + c * V;
    *reinterpret_cast<uint4*>(kdst + dof) = *reinterpret_cast<const uint4*>(kp + so);
    if (vp != nullptr)
      *reinterpret_cast<uint4*>(vdst + dof) = *reinterpret_cast<const uint4*>(vp + so);
  }
}

template <typename T, int D, int STYLE, bool ALIGN, bool NESTED>
void launch_g(const void* k_src, const void* v_src, const kvsel_cache& kc, int64_t U,
              const int32_t* idx, int64_t k, int64_t idx_group, const int64_t* src_start,
              int64_t align_base, double base, int64_t dst_rows, void* k_dst, void* v_dst,
              hipStream_t s) {
  const int64_t row_bytes = kc.H * kc.D * static_cast<int64_t>(sizeof(T));
  // 32 KiB per workgroup; with "align" 8 KiB but at least two rows (measured
  // on 1 KiB rows: 32 KiB 0.884 ms, 8 KiB 0.838, 4 KiB 1.13; rows of 8 KiB
  // gain nothing below 16 KiB)
  const int64_t fit = ALIGN ? std::max<int64_t>(2, 8192 / row_bytes) : 32768 / row_bytes;
  const int64_t rows_per_chunk = std::min<int64_t>(U, fit > 1 ? fit : 1);
  const int64_t chunks = (U + rows_per_chunk - 1) / rows_per_chunk;
  hipLaunchKernelGGL((gather_kernel<T, D, STYLE, ALIGN, NESTED>),
                     dim3(static_cast<unsigned>(kc.B * k * chunks)), dim3(kThreads), 0, s,
                     static_cast<const T*>(k_src), static_cast<const T*>(v_src),
                     static_cast<int>(kc.H), kc.stride_b, kc.stride_n, U, idx, k, idx_group,
                     src_start, align_base, ALIGN ? rope_theta(base, D) : RopeTheta{}, chunks,
                     rows_per_chunk, dst_rows, kc.N / U,
                     static_cast<T*>(k_dst), static_cast<T*>(v_dst));
}

template <typename T, int D>
void dispatch_g(const void* k_src, const void* v_src, const kvsel_cache& kc, int64_t U,
                const int32_t* idx, int64_t k, int64_t idx_group, const int64_t* src_start,
                int64_t align_base, double base, int style, int nested, int64_t dst_rows,
                void* k_dst, void* v_dst, hipStream_t s) {
#define KVSEL_G(ST, AL, NE) launch_g<T, D, ST, AL, NE>(k_src, v_src, kc, U, idx, k, idx_group, src_start, align_base, base, dst_rows, k_dst, v_dst, s)
  if (align_base >= 0) {
    if (style == KVSEL_ROPE_HALF) KVSEL_G(0, true, false); else KVSEL_G(1, true, false);
  } else if (nested) {
    KVSEL_G(0, false, true);
  } else {
    KVSEL_G(0, false, false);
  }
#undef KVSEL_G
}

}  // namespace

int launch_gather(const void* k_src, const void* v_src, const kvsel_cache& kc, int64_t unit_len,
                  const int32_t* idx, int64_t k, int64_t idx_group, const int64_t* src_start,
                  int64_t align_base, double base, int style, int nested, int64_t dst_rows,
                  void* k_dst, void* v_dst, hipStream_t s) {
  if (kc.dtype == KVSEL_BF16) {
    if (kc.D == 128) dispatch_g<bf16_t, 128>(k_src, v_src, kc, unit_len, idx, k, idx_group, src_start, align_base, base, style, nested, dst_rows, k_dst, v_dst, s);
    else dispatch_g<bf16_t, 64>(k_src, v_src, kc, unit_len, idx, k, idx_group, src_start, align_base, base, style, nested, dst_rows, k_dst, v_dst, s);
  } else {
    if (kc.D == 128) dispatch_g<float, 128>(k_src, v_src, kc, unit_len, idx, k, idx_group, src_start, align_base, base, style, nested, dst_rows, k_dst, v_dst, s);
    else dispatch_g<float, 64>(k_src, v_src, kc, unit_len, idx, k, idx_group, src_start, align_base, base, style, nested, dst_rows, k_dst, v_dst, s);
  }
  return check_launch("kvsel_gather");
}

int launch_proxy_copy(const void* k_proxy, const void* v_proxy, const kvsel_cache& proxy,
                      int64_t unit_len, const int32_t* idx, int64_t k, int64_t idx_group,
                      int64_t dst_rows, void* k_dst, void* v_dst, hipStream_t s) {
  const int64_t tiles = (proxy.N + kProxyRows - 1) / kProxyRows;
  const dim3 grid(static_cast<unsigned>(proxy.B * tiles));
  const int64_t re = proxy.H * proxy.D;
  if (proxy.dtype == KVSEL_BF16)
    hipLaunchKernelGGL(proxy_copy_kernel<bf16_t>, grid, dim3(kThreads), 0, s,
                       static_cast<const bf16_t*>(k_proxy), static_cast<const bf16_t*>(v_proxy),
                       proxy.N, re, proxy.stride_b, proxy.stride_n, unit_len, idx, k, idx_group,
                       tiles, dst_rows, static_cast<bf16_t*>(k_dst), static_cast<bf16_t*>(v_dst));
  else
    hipLaunchKernelGGL(proxy_copy_kernel<float>, grid, dim3(kThreads), 0, s,
                       static_cast<const float*>(k_proxy), static_cast<const float*>(v_proxy),
                       proxy.N, re, proxy.stride_b, proxy.stride_n, unit_len, idx, k, idx_group,
                       tiles, dst_rows, static_cast<float*>(k_dst), static_cast<float*>(v_dst));
  return check_launch("kvsel_gather (proxy rows)");
}

}  // namespace kvsel
