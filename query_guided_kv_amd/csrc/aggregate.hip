// Per-unit relevance from the softmax-normalised attention.
//   mass:  S[g,u] = sum_{b in g} sum_h sum_j sum_{t in u} alpha        (ACRE §2.4 Eq. 15,
//          as a sum; CacheFocus §2.4 footnote 3)
//   vnorm: S[g,u] = sum ... alpha * ||v[b,t,kv(h)]||_2                  (InfoFlow §4.2)
// with alpha = exp(l - row_max) / row_sum.
//
// Chunk path: units are the score segments, so the per-unit sums follow from
// the partials (m_u, S_u) without touching the cache again:
//   sum_{t in u} alpha = S_u * exp(m_u - row_max) / row_sum.
// Token path: the logits are recomputed from Q and K (a second streaming pass
// over the keys, plus the values for the norm); each lane group owns one
// cached row and loops over the query rows, so the sum over rows stays in
// registers and needs no atomics.  Reductions have a fixed order, so results
// are bitwise reproducible from run to run.
#include "common.h"
#include "internal.h"

namespace kvsel {
namespace {

constexpr int kThreads = 256;

// Chunk path, stage 1: workgroup (g, row chunk, unit chunk); 64 units x 4 row
// lanes; each lane sums every 4th row of the chunk, the four lanes merge in
// LDS.  Writes out[g][u] directly when one chunk covers the group's rows
// (added to the value there with `accumulate`), else a partial
// ws[(g * n_rc + rc) * M + u] for stage 2.
constexpr int kAggUnits = 64;
constexpr int kAggRowLanes = kThreads / kAggUnits;
constexpr int kAggChunkRows = 64;

// DERIVE: no row statistics are given; the workgroup derives (row_max,
// row_sum) of its 64 rows from their partials first (4 lanes per row, merged
// in a fixed order), in the log2 domain.
template <bool DERIVE>
__global__ void __launch_bounds__(kThreads)
agg_chunk_kernel(const float* __restrict__ part, const float* __restrict__ row_max,
                 const float* __restrict__ row_sum, int64_t rows_per_g, int64_t M, int64_t n_rc,
                 int64_t n_uc, int accumulate, float* __restrict__ dst) {
  static_assert(kThreads == 4 * kAggChunkRows, "4 lanes per row derive its statistics");
  __shared__ float red[kAggRowLanes][kAggUnits];
  __shared__ float s_m[DERIVE ? kAggChunkRows : 1], s_iz[DERIVE ? kAggChunkRows : 1];
  const int64_t uc = blockIdx.x % static_cast<uint32_t>(n_uc);   // 32-bit: the grid is below 2^32 workgroups
  const int64_t rc = (blockIdx.x / static_cast<uint32_t>(n_uc)) % static_cast<uint32_t>(n_rc);
  const int64_t gi = blockIdx.x / static_cast<uint32_t>(n_uc * n_rc);
  const int ul = threadIdx.x % kAggUnits, rl = threadIdx.x / kAggUnits;
  const int64_t u = uc * kAggUnits + ul;
  const int64_t r0 = rc * kAggChunkRows;
  const int64_t r1 = min(rows_per_g, r0 + kAggChunkRows);
  if constexpr (DERIVE) {
    const int sr = threadIdx.x / 4, sq = threadIdx.x % 4;
    float m = -INFINITY, z = 0.0f;
    if (r0 + sr < r1) {
      const float* pr = part + (gi * rows_per_g + r0 + sr) * M * 2;
      for (int64_t uu = sq; uu < M; uu += 4) {
        const float2 pu = *reinterpret_cast<const float2*>(pr + uu * 2);
        merge_ms(m, z, pu.x * kLog2e, pu.y);
      }
    }
    merge_ms(m, z, __shfl_xor(m, 1, 64), __shfl_xor(z, 1, 64));
    merge_ms(m, z, __shfl_xor(m, 2, 64), __shfl_xor(z, 2, 64));
    if (sq == 0) { s_m[sr] = m; s_iz[sr] = z > 0.0f ? 1.0f / z : 0.0f; }
    __syncthreads();
  }
  float acc = 0.0f;
  if (u < M) {
    for (int64_t r = r0 + rl; r < r1; r += kAggRowLanes) {
      const int64_t row = gi * rows_per_g + r;
      const float2 pu = *reinterpret_cast<const float2*>(part + (row * M + u) * 2);
      if constexpr (DERIVE)
        acc += pu.y * exp2f(pu.x * kLog2e - s_m[r - r0]) * s_iz[r - r0];
      else
        acc += pu.y * exp2f((pu.x - row_max[row]) * kLog2e) / row_sum[row];
    }
  }
  red[rl][ul] = acc;
  __syncthreads();
  if (rl == 0 && u < M) {
    float t = red[0][ul];
#pragma unroll
    for (int i = 1; i < kAggRowLanes; ++i) t += red[i][ul];
    float* o = dst + (gi * n_rc + rc) * M + u;
    *o = accumulate ? *o + t : t;
  }
}

// Chunk path, stage 2: out[g][u] = sum over row chunks, in order (added to
// out[g][u] with `accumulate`).
__global__ void __launch_bounds__(kThreads)
agg_chunk_sum_kernel(const float* __restrict__ ws, int64_t G, int64_t M, int64_t n_rc,
                     int accumulate, float* __restrict__ out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= G * M) return;
  const int64_t gi = i / M, u = i % M;
  float t = 0.0f;
  for (int64_t rc = 0; rc < n_rc; ++rc) t += ws[(gi * n_rc + rc) * M + u];
  out[i] = accumulate ? out[i] + t : t;
}

constexpr int kQRows = 64;
constexpr int kPad = 4;

// per_token[b][t] = sum_h sum_j alpha[b,h,j,t] (* ||v[b,t,kv(h)]||)
template <typename T, int D, int TPR, bool VNORM>
__global__ void __launch_bounds__(kThreads)
agg_token_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                 int64_t N, int H, int64_t stride_b, int64_t stride_n, int T_, int Hq,
                 float scale2, const float* __restrict__ row_max,
                 const float* __restrict__ row_sum, int64_t tiles,
                 float* __restrict__ per_token) {
  constexpr int TPB = kThreads / TPR;  // cached rows per block
  constexpr int DPT = D / TPR;
  __shared__ __align__(16) float qs[kQRows][D + kPad];
  __shared__ float mz[kQRows][2];

  const int64_t b = blockIdx.x / static_cast<uint32_t>(tiles);   // 32-bit: the grid is below 2^32 workgroups
  const int64_t t = static_cast<int64_t>(blockIdx.x % static_cast<uint32_t>(tiles)) * TPB + threadIdx.x / TPR;
  const int p = threadIdx.x % TPR;
  const bool t_ok = t < N;
  const int G = Hq / H;
  const int R = G * T_;
  float acc = 0.0f;
  for (int g = 0; g < H; ++g) {
    float kf[DPT];
    float vn = 1.0f;
    {
      const int64_t off = b * stride_b + (t_ok ? t : 0) * stride_n + static_cast<int64_t>(g) * D + p * DPT;
      load_f32<T, DPT>(k + off, kf);
      if constexpr (VNORM) {
        float vf[DPT];
        load_f32<T, DPT>(v + off, vf);
        float ss = 0.0f;
#pragma unroll
        for (int d = 0; d < DPT; ++d) ss += vf[d] * vf[d];
        vn = sqrtf(group_sum<TPR>(ss));
      }
    }
    float accg = 0.0f;
    for (int r0 = 0; r0 < R; r0 += kQRows) {
      const int nr = min(kQRows, R - r0);
      __syncthreads();
      for (int e = threadIdx.x; e < nr * D; e += kThreads) {
        const int rr = e / D, d = e % D;
        const int r = r0 + rr;
        const int h = g * G + r / T_, j = r % T_;
        qs[rr][d] = Elem<T>::to_f32(q[((b * T_ + j) * Hq + h) * D + d]);
      }
      for (int rr = threadIdx.x; rr < nr; rr += kThreads) {
        const int r = r0 + rr;
        const int h = g * G + r / T_, j = r % T_;
        const int64_t row = (b * Hq + h) * T_ + j;
        mz[rr][0] = row_max[row] * kLog2e;
        mz[rr][1] = 1.0f / row_sum[row];
      }
      __syncthreads();
      for (int rr = 0; rr < nr; ++rr) {
        float dot = 0.0f;
        if constexpr (DPT >= 4) {
          const float4* qr = reinterpret_cast<const float4*>(&qs[rr][p * DPT]);
#pragma unroll
          for (int d4 = 0; d4 < DPT / 4; ++d4) {
            const float4 qq = qr[d4];
            dot += qq.x * kf[4 * d4] + qq.y * kf[4 * d4 + 1] + qq.z * kf[4 * d4 + 2] +
                   qq.w * kf[4 * d4 + 3];
          }
        } else {
#pragma unroll
          for (int d = 0; d < DPT; ++d) dot += qs[rr][p * DPT + d] * kf[d];
        }
        dot = group_sum<TPR>(dot);
        accg += exp2f(dot * scale2 - mz[rr][0]) * mz[rr][1];
      }
    }
    acc += accg * vn;
  }
  if (t_ok && p == 0) per_token[b * N + t] = acc;
}

// unit_score[g][u] = sum_{b in g} sum_{t in u} per_token[b][t], fixed order
// (added to unit_score[g][u] with `accumulate`).
__global__ void __launch_bounds__(kThreads)
unit_sum_kernel(const float* __restrict__ per_token, int64_t parts, int64_t part_stride,
                int64_t N, int64_t unit_len, int64_t M, int64_t group, int64_t mblocks,
                int accumulate, float* __restrict__ out) {
  const int64_t gi = blockIdx.x / static_cast<uint32_t>(mblocks);   // 32-bit: the grid is below 2^32 workgroups
  const int64_t u = static_cast<int64_t>(blockIdx.x % static_cast<uint32_t>(mblocks)) * kThreads + threadIdx.x;
  if (u >= M) return;
  float acc = 0.0f;
  for (int64_t p = 0; p < parts; ++p) {
    for (int64_t bi = 0; bi < group; ++bi) {
      const float* pt = per_token + p * part_stride + (gi * group + bi) * N + u * unit_len;
      for (int64_t t = 0; t < unit_len; ++t) acc += pt[t];
    }
  }
  out[gi * M + u] = accumulate ? out[gi * M + u] + acc : acc;
}

template <typename T, int D, int TPR>
void launch_tok(const void* q, int64_t T_, int64_t Hq, const void* k, const void* v,
                const kvsel_cache& kc, float scale2, const float* rm, const float* rs, int vnorm,
                float* per_token, hipStream_t s) {
  constexpr int TPB = kThreads / TPR;
  const int64_t tiles = (kc.N + TPB - 1) / TPB;
  const dim3 grid(static_cast<unsigned>(kc.B * tiles));
  if (vnorm)
    hipLaunchKernelGGL((agg_token_kernel<T, D, TPR, true>), grid, dim3(kThreads), 0, s,
                       static_cast<const T*>(q), static_cast<const T*>(k),
                       static_cast<const T*>(v), kc.N, static_cast<int>(kc.H), kc.stride_b,
                       kc.stride_n, static_cast<int>(T_), static_cast<int>(Hq), scale2, rm, rs,
                       tiles, per_token);
  else
    hipLaunchKernelGGL((agg_token_kernel<T, D, TPR, false>), grid, dim3(kThreads), 0, s,
                       static_cast<const T*>(q), static_cast<const T*>(k),
                       static_cast<const T*>(v), kc.N, static_cast<int>(kc.H), kc.stride_b,
                       kc.stride_n, static_cast<int>(T_), static_cast<int>(Hq), scale2, rm, rs,
                       tiles, per_token);
}

}  // namespace

int launch_aggregate_chunks(const float* part, const float* row_max, const float* row_sum,
                            int64_t B, int64_t Hq, int64_t T, int64_t M, int64_t group,
                            float* unit_score, int accumulate, float* ws, hipStream_t s) {
  const int64_t G = B / group;
  const int64_t rows_per_g = group * Hq * T;
  const int64_t n_rc = (rows_per_g + kAggChunkRows - 1) / kAggChunkRows;
  const int64_t n_uc = (M + kAggUnits - 1) / kAggUnits;
  float* dst = n_rc == 1 ? unit_score : ws;
  if (row_max == nullptr)
    hipLaunchKernelGGL(agg_chunk_kernel<true>, dim3(static_cast<unsigned>(G * n_rc * n_uc)),
                       dim3(kThreads), 0, s, part, row_max, row_sum, rows_per_g, M, n_rc, n_uc,
                       n_rc == 1 ? accumulate : 0, dst);
  else
    hipLaunchKernelGGL(agg_chunk_kernel<false>, dim3(static_cast<unsigned>(G * n_rc * n_uc)),
                       dim3(kThreads), 0, s, part, row_max, row_sum, rows_per_g, M, n_rc, n_uc,
                       n_rc == 1 ? accumulate : 0, dst);
  if (n_rc > 1) {
    const int rc = check_launch("kvsel_aggregate");
    if (rc != KVSEL_OK) return rc;
    hipLaunchKernelGGL(agg_chunk_sum_kernel, dim3(static_cast<unsigned>((G * M + kThreads - 1) / kThreads)),
                       dim3(kThreads), 0, s, ws, G, M, n_rc, accumulate, unit_score);
  }
  return check_launch("kvsel_aggregate");
}

bool aggregate_chunks_derive(int64_t M) {
  // each unit chunk's workgroups derive the statistics again: at most two
  return (M + kAggUnits - 1) / kAggUnits <= 2;
}

size_t aggregate_chunk_ws_floats(int64_t B, int64_t Hq, int64_t T, int64_t M) {
  // any group: (B / group) * ceil(group * Hq * T / 64) <= ceil(B * Hq * T / 64) + B
  return static_cast<size_t>(((B * Hq * T + kAggChunkRows - 1) / kAggChunkRows + B) * M);
}

int launch_aggregate_tokens(const void* q, int64_t T, int64_t Hq, const void* k, const void* v,
                            const kvsel_cache& kc, float scale, const float* row_max,
                            const float* row_sum, int vnorm, float* per_token, hipStream_t s) {
  const float scale2 = scale * kLog2e;
  if (aggregate_mfma_ok(kc.dtype, (Hq / kc.H) * T)) {
    launch_aggregate_mfma(q, T, Hq, k, v, kc, scale2, row_max, row_sum, vnorm, per_token, s);
    return check_launch("kvsel_aggregate (token path)");
  }
  if (kc.dtype == KVSEL_BF16) {
    if (kc.D == 128) launch_tok<bf16_t, 128, 4>(q, T, Hq, k, v, kc, scale2, row_max, row_sum, vnorm, per_token, s);
    else launch_tok<bf16_t, 64, 4>(q, T, Hq, k, v, kc, scale2, row_max, row_sum, vnorm, per_token, s);
  } else {
    if (kc.D == 128) launch_tok<float, 128, 4>(q, T, Hq, k, v, kc, scale2, row_max, row_sum, vnorm, per_token, s);
    else launch_tok<float, 64, 4>(q, T, Hq, k, v, kc, scale2, row_max, row_sum, vnorm, per_token, s);
  }
  return check_launch("kvsel_aggregate (token path)");
}

int64_t aggregate_token_parts(const kvsel_cache& kc, int64_t Hq, int64_t T) {
  const int64_t rows = (Hq / kc.H) * T;
  return aggregate_mfma_ok(kc.dtype, rows) ? aggregate_mfma_parts(kc, rows) : 1;
}

int launch_unit_sums(const float* per_token, int64_t parts, int64_t B, int64_t N,
                     int64_t unit_len, int64_t group, float* unit_score, int accumulate,
                     hipStream_t s) {
  const int64_t M = N / unit_len;
  const int64_t mblocks = (M + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(unit_sum_kernel, dim3(static_cast<unsigned>((B / group) * mblocks)),
                     dim3(kThreads), 0, s, per_token, parts, B * N, N, unit_len, M, group, mblocks,
                     accumulate, unit_score);
  return check_launch("kvsel_aggregate (unit sums)");
}

}  // namespace kvsel
