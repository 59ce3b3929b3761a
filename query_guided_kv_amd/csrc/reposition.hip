// Cache re-positioning: rotate every cached key of unit u by delta[u]
// positions (CacheFocus §2.3; InfoFlow §4.2 global position reconstruction).
//
// One workgroup owns kRows consecutive rows of one instance.  It forms the
// cos/sin of delta[u] * theta_i for the units it touches in fp64 and keeps
// them in LDS; every thread then streams 16-byte vectors of the key rows,
// rotates in fp64 and stores the correctly rounded result.  HBM-bound: one
// read and one write of each key byte (the fp64 work hides under the loads).
#include "common.h"
#include "internal.h"

namespace kvsel {
namespace {

constexpr int kRows = 16;
constexpr int kThreads = 256;

template <typename T, int D, int STYLE>
__global__ void __launch_bounds__(kThreads)
reposition_kernel(const T* kin, T* kout, int64_t N, int H, int64_t stride_b,
                  int64_t stride_n, int64_t unit_len, const int64_t* __restrict__ delta,
                  int64_t delta_stride_b, int64_t tiles, RopeTheta th) {
  constexpr int V = Elem<T>::kPerVec;
  constexpr int HALF = D / 2;
  __shared__ double2 cs[kRows][HALF];

  const int64_t b = blockIdx.x / static_cast<uint32_t>(tiles);   // 32-bit: the grid is below 2^32 workgroups
  const int64_t r0 = static_cast<int64_t>(blockIdx.x % static_cast<uint32_t>(tiles)) * kRows;
  const int rows = static_cast<int>(min<int64_t>(kRows, N - r0));
  const int64_t u0 = r0 / unit_len;
  const int nu = static_cast<int>((r0 + rows - 1) / unit_len - u0 + 1);
  const int64_t* db = delta + b * delta_stride_b;
  for (int e = threadIdx.x; e < nu * HALF; e += kThreads) {
    const int uu = e / HALF, i = e - uu * HALF;
    cs[uu][i] = rope_cs(db[u0 + uu], th.t[i]);
  }
  __syncthreads();

  const T* src = kin + b * stride_b;
  T* dst = kout + b * stride_b;
  if constexpr (STYLE == KVSEL_ROPE_HALF) {
    constexpr int VPH = HALF / V;  // vector pairs per head
    const int items = rows * H * VPH;
    for (int it = threadIdx.x; it < items; it += kThreads) {
      const int c = it % VPH;
      const int rh = it / VPH;
      const int h = rh % H;
      const int r = rh / H;
      const int64_t row = r0 + r;
      const int uu = static_cast<int>(row / unit_len - u0);
      const int64_t off = row * stride_n + static_cast<int64_t>(h) * D + c * V;
      uint4 ra = *reinterpret_cast<const uint4*>(src + off);
      uint4 rb = *reinterpret_cast<const uint4*>(src + off + HALF);
      rope_rotate16<T, KVSEL_ROPE_HALF>(ra, rb, c * V, cs[uu]);
      *reinterpret_cast<uint4*>(dst + off) = ra;
      *reinterpret_cast<uint4*>(dst + off + HALF) = rb;
    }
  } else {
    constexpr int VPR = D / V;  // vectors per head
    const int items = rows * H * VPR;
    for (int it = threadIdx.x; it < items; it += kThreads) {
      const int c = it % VPR;
      const int rh = it / VPR;
      const int h = rh % H;
      const int r = rh / H;
      const int64_t row = r0 + r;
      const int uu = static_cast<int>(row / unit_len - u0);
      const int64_t off = row * stride_n + static_cast<int64_t>(h) * D + c * V;
      uint4 ra = *reinterpret_cast<const uint4*>(src + off);
      uint4 unused;
      rope_rotate16<T, KVSEL_ROPE_INTERLEAVED>(ra, unused, c * V, cs[uu]);
      *reinterpret_cast<uint4*>(dst + off) = ra;
    }
  }
}

template <typename T, int D, int STYLE>
void launch_t(const void* k_in, void* k_out, const kvsel_cache& kc, int64_t unit_len,
              const int64_t* delta, int per_instance, double base, hipStream_t s) {
  const int64_t tiles = (kc.N + kRows - 1) / kRows;
  const int64_t M = kc.N / unit_len;
  hipLaunchKernelGGL((reposition_kernel<T, D, STYLE>), dim3(static_cast<unsigned>(kc.B * tiles)),
                     dim3(kThreads), 0, s, static_cast<const T*>(k_in), static_cast<T*>(k_out),
                     kc.N, static_cast<int>(kc.H), kc.stride_b, kc.stride_n, unit_len, delta,
                     per_instance ? M : int64_t{0}, tiles, rope_theta(base, D));
}

}  // namespace

int launch_reposition(const void* k_in, void* k_out, const kvsel_cache& kc, int64_t unit_len,
                      const int64_t* delta, int per_instance, double base, int style,
                      hipStream_t s) {
#define KVSEL_REPOS(T, D, ST) launch_t<T, D, ST>(k_in, k_out, kc, unit_len, delta, per_instance, base, s)
  const bool half = style == KVSEL_ROPE_HALF;
  if (kc.dtype == KVSEL_BF16) {
    if (kc.D == 128) { if (half) KVSEL_REPOS(bf16_t, 128, 0); else KVSEL_REPOS(bf16_t, 128, 1); }
    else             { if (half) KVSEL_REPOS(bf16_t, 64, 0);  else KVSEL_REPOS(bf16_t, 64, 1); }
  } else {
    if (kc.D == 128) { if (half) KVSEL_REPOS(float, 128, 0); else KVSEL_REPOS(float, 128, 1); }
    else             { if (half) KVSEL_REPOS(float, 64, 0);  else KVSEL_REPOS(float, 64, 1); }
  }
#undef KVSEL_REPOS
  return check_launch("kvsel_reposition");
}

}  // namespace kvsel
