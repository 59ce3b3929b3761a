// Query block -> cached keys: softmax partials per segment of cached rows
// (ACRE §2.4, A = softmax(Q_q K^T / sqrt(d)); ACRE §2.1 Eq. 4).
//
// For every row (query head h, query token j) and every segment of cached
// rows, the kernels produce (m, s): the largest logit of the segment and the
// sum of exp(l - m) over it.  Segments are the scoring units (chunk mode) or
// fixed tiles whose partials merge into the row statistics.
//
// Two paths:
//  * stream: bf16 caches whose rows per kv head (query heads per kv head x
//    query tokens) are few, e.g. one decode token.  The key stream is the
//    whole cost (a few flop per byte), so each lane owns 32 contiguous bytes
//    of a cached row; a wave covers whole rows with fully used 16-byte loads,
//    products use the packed bf16 dot instruction with fp32 accumulation, and
//    the per-head reduction is a 3-step DPP butterfly inside 8 lanes.
//  * tile: any shape.  Keys are staged through LDS in fp32 tiles; each row is
//    owned by TPR lanes that split the head dim.
#include "common.h"
#include "internal.h"

namespace kvsel {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

// ---------------------------------------------------------------------------
// stream path
// ---------------------------------------------------------------------------
// Lane layout: LPH = D/16 = 8 lanes per kv head (16 dims = 32 bytes each),
// LPT = H*LPH lanes per cached row, TPW = 64/LPT rows per wave step.  A wave
// step covers U rows per slot (U*TPW*waves rows per workgroup step).
//
// After the packed-bf16 dot products each lane holds partial sums of V = U*R
// (key, query row) pairs.  A reduce-scatter over the 8 lanes of the head (see
// reduce_scatter8) leaves every lane with V/8 complete logits of ONE query row,
// so the softmax update runs once per logit instead of once per lane.
//
// Lane c of a head group (bits b0 b1 b2) owns index block j = 4*b2 + 2*b0 + b1,
// i.e. the V/8 pairs idx = r*U + u in [j*V/8, (j+1)*V/8): query row
// r = j*V/(8U), keys u = (j*V/8) % U + 0 .. V/8-1.

// Reduce-scatter of V values over the 8 lanes of a head group: three butterfly
// levels (partners: lane i <-> 7-i, then xor 1, then xor 2).  At each level a
// lane keeps the half of its current values picked by one lane-id bit (b2, b0,
// b1 in turn), adds the partner's copy of that half and drops the other half.
template <int V>
__device__ __forceinline__ void reduce_scatter8(float (&x)[V], int c) {
  static_assert(V % 8 == 0, "8 lanes need at least 8 values");
  const bool h2 = (c & 4) != 0, h0 = (c & 1) != 0, h1 = (c & 2) != 0;
#pragma unroll
  for (int i = 0; i < V / 2; ++i) {
    const float keep = h2 ? x[i + V / 2] : x[i];
    const float send = h2 ? x[i] : x[i + V / 2];
    x[i] = keep + dpp_half_mirror(send);
  }
#pragma unroll
  for (int i = 0; i < V / 4; ++i) {
    const float keep = h0 ? x[i + V / 4] : x[i];
    const float send = h0 ? x[i] : x[i + V / 4];
    x[i] = keep + dpp_xor1(send);
  }
#pragma unroll
  for (int i = 0; i < V / 8; ++i) {
    const float keep = h1 ? x[i + V / 8] : x[i];
    const float send = h1 ? x[i] : x[i + V / 8];
    x[i] = keep + dpp_xor2(send);
  }
}

// Merge of softmax partials (log2 domain) with the lane holding the same query
// row: PARTNER 0 = xor 2, 1 = xor 1, 2 = half mirror.
template <int PARTNER>
__device__ __forceinline__ void merge_lane(float& m, float& s) {
  float m2, s2;
  if constexpr (PARTNER == 0) { m2 = dpp_xor2(m); s2 = dpp_xor2(s); }
  else if constexpr (PARTNER == 1) { m2 = dpp_xor1(m); s2 = dpp_xor1(s); }
  else { m2 = dpp_half_mirror(m); s2 = dpp_half_mirror(s); }
  merge_ms(m, s, m2, s2);
}

template <int D, int H, int R, int U, int NTH>
__global__ void __launch_bounds__(NTH)
score_stream_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, int64_t N,
                    int64_t stride_b, int64_t stride_n, int T, int Hq, float scale2,
                    int64_t seg_len, int64_t nseg, int64_t spb, float* __restrict__ ms,
                    int natural) {
  constexpr int LPH = D / 16;
  constexpr int LPT = H * LPH;
  constexpr int TPW = 64 / LPT;
  constexpr int V = U * R;        // (key, row) pairs per lane and step
  constexpr int VL = V / 8;       // complete logits per lane after the scatter
  static_assert(LPH == 8, "head dim 128: 8 lanes per head");
  static_assert(LPT <= 64 && 64 % LPT == 0, "row must tile a wave");
  static_assert(V % 8 == 0 && VL <= U, "need 8 <= U*R <= 8*U");
  constexpr int NWV = NTH / 64;
  __shared__ float red[NWV][H * R][2];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int slot = lane / LPT;
  const int g = (lane % LPT) / LPH;
  const int c = lane % LPH;
  // a workgroup scores spb consecutive segments (one partial each): the
  // query slices are loaded once and the per-segment fixed cost is shared
  const int64_t groups = (nseg + spb - 1) / spb;
  const int64_t b = blockIdx.x / static_cast<uint32_t>(groups);   // 32-bit: the grid is below 2^32 workgroups
  const int64_t seg0 = static_cast<int64_t>(blockIdx.x % static_cast<uint32_t>(groups)) * spb;
  const int64_t seg1 = min(nseg, seg0 + spb);
  const int G = Hq / H;
  // the block of (row, key) pairs this lane owns after the scatter
  const int j = ((c >> 2) & 1) * 4 + (c & 1) * 2 + ((c >> 1) & 1);
  const int own_r = (j * VL) / U;
  const int own_u = (j * VL) % U;

  // query slices of this lane's kv head: R rows x 16 dims (8 packed pairs)
  uint32_t qv[R][8];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int h = g * G + r / T, jj = r % T;
    const uint4* qp = reinterpret_cast<const uint4*>(q + ((b * T + jj) * Hq + h) * D + c * 16);
    const uint4 q0 = qp[0], q1 = qp[1];
    qv[r][0] = q0.x; qv[r][1] = q0.y; qv[r][2] = q0.z; qv[r][3] = q0.w;
    qv[r][4] = q1.x; qv[r][5] = q1.y; qv[r][6] = q1.z; qv[r][7] = q1.w;
  }

  const bf16_t* kb = k + b * stride_b + g * D + c * 16;
  constexpr int STEP = NWV * TPW;
  for (int64_t seg = seg0; seg < seg1; ++seg) {
  float m = -INFINITY, s = 0.0f;  // softmax partial of row own_r over this lane's keys
  const int64_t t_begin = seg * seg_len;
  const int64_t t_end = min(N, t_begin + seg_len);

  // logits of U rows (t0 + u*STEP) from their loaded slices; rows with
  // u >= n_valid are masked out
  auto consume = [&](const uint4 (&kr)[U][2], int n_valid) {
    float x[V];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t kw[8] = {kr[u][0].x, kr[u][0].y, kr[u][0].z, kr[u][0].w,
                              kr[u][1].x, kr[u][1].y, kr[u][1].z, kr[u][1].w};
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float acc = 0.0f;
#pragma unroll
        for (int p = 0; p < 8; ++p) acc = dot2(qv[r][p], kw[p], acc);
        x[r * U + u] = acc;
      }
    }
    reduce_scatter8<V>(x, c);
    float l[VL];
    float bm = -INFINITY;
#pragma unroll
    for (int e = 0; e < VL; ++e) {
      l[e] = (own_u + e < n_valid) ? x[e] * scale2 : -INFINITY;
      bm = fmaxf(bm, l[e]);
    }
    const float mn = fmaxf(m, bm);
    if (mn != -INFINITY) {
      float acc = s * __builtin_amdgcn_exp2f(m - mn);
#pragma unroll
      for (int e = 0; e < VL; ++e) acc += __builtin_amdgcn_exp2f(l[e] - mn);
      s = acc;
      m = mn;
    }
  };
  auto load = [&](uint4 (&kr)[U][2], int64_t t0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint4* kp = reinterpret_cast<const uint4*>(kb + (t0 + static_cast<int64_t>(u) * STEP) * stride_n);
      kr[u][0] = kp[0];
      kr[u][1] = kp[1];
    }
  };

  int64_t t0 = t_begin + wave * TPW + slot;
  const int64_t full_end = t_end - static_cast<int64_t>(U - 1) * STEP;  // t0 < full_end: U rows valid
  for (; t0 < full_end; t0 += static_cast<int64_t>(STEP) * U) {
    uint4 cur[U][2];
    load(cur, t0);
    consume(cur, U);
  }
  if (t0 < t_end) {  // ragged tail: fewer than U rows left for this slot
    const int n_valid = static_cast<int>((t_end - t0 + STEP - 1) / STEP);
    uint4 cur[U][2];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (u < n_valid) {
        const uint4* kp = reinterpret_cast<const uint4*>(kb + (t0 + static_cast<int64_t>(u) * STEP) * stride_n);
        cur[u][0] = kp[0];
        cur[u][1] = kp[1];
      } else {
        cur[u][0] = cur[u][1] = make_uint4(0, 0, 0, 0);
      }
    }
    consume(cur, n_valid);
  }

  // lanes of the head group that own the same query row
  if constexpr (R <= 4) merge_lane<0>(m, s);
  if constexpr (R <= 2) merge_lane<1>(m, s);
  if constexpr (R <= 1) merge_lane<2>(m, s);
  // the TPW row slots of the wave (lanes LPT apart)
#pragma unroll
  for (int off = LPT; off < 64; off <<= 1) {
    const float m2 = __shfl_xor(m, off, 64);
    const float s2 = __shfl_xor(s, off, 64);
    merge_ms(m, s, m2, s2);
  }
  // one lane per (head, row) publishes: the owner of the row's first keys
  if (seg > seg0) __syncthreads();   // the previous segment's partials fully read
  if (slot == 0 && own_u == 0) {
    red[wave][g * R + own_r][0] = m;
    red[wave][g * R + own_r][1] = s;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < H * R; i += NTH) {
    float mm = red[0][i][0], ss = red[0][i][1];
#pragma unroll
    for (int w = 1; w < NWV; ++w) merge_ms(mm, ss, red[w][i][0], red[w][i][1]);
    const int gg = i / R, r = i % R;
    const int h = gg * G + r / T, jj = r % T;
    float* o = ms + (((b * Hq + h) * T + jj) * nseg + seg) * 2;
    o[0] = natural ? mm * kLn2 : mm;
    o[1] = ss;
  }
  }
}

// ---------------------------------------------------------------------------
// tile path
// ---------------------------------------------------------------------------
constexpr int kTileKeys = 64;
constexpr int kPad = 4;

template <typename T, int D, int TPR>
__global__ void __launch_bounds__(kThreads)
score_tile_kernel(const T* __restrict__ q, const T* __restrict__ k, int64_t N, int H,
                  int64_t stride_b, int64_t stride_n, int T_, int Hq, float scale2,
                  int64_t seg_len, int64_t nseg, float* __restrict__ ms, int natural) {
  constexpr int RB = kThreads / TPR;  // rows per pass
  constexpr int DPT = D / TPR;        // dims per lane
  constexpr int V = Elem<T>::kPerVec;
  __shared__ __align__(16) float ks[kTileKeys][D + kPad];

  const int64_t seg = blockIdx.x % static_cast<uint32_t>(nseg);   // 32-bit: the grid is below 2^32 workgroups
  const uint32_t bg = blockIdx.x / static_cast<uint32_t>(nseg);
  const int g = static_cast<int>(bg % static_cast<uint32_t>(H));
  const int64_t b = bg / static_cast<uint32_t>(H);
  const int G = Hq / H;
  const int R = G * T_;
  const int rl = threadIdx.x / TPR;
  const int p = threadIdx.x % TPR;
  const int64_t t_begin = seg * seg_len;
  const int64_t t_end = min(N, t_begin + seg_len);
  const T* kb = k + b * stride_b + static_cast<int64_t>(g) * D;

  for (int row0 = 0; row0 < R; row0 += RB) {
    const int r = row0 + rl;
    const bool row_ok = r < R;
    float qf[DPT];
    if (row_ok) {
      const int h = g * G + r / T_, j = r % T_;
      if constexpr ((DPT * sizeof(T)) % 16 == 0) {
        load_f32<T, DPT>(q + ((b * T_ + j) * Hq + h) * D + p * DPT, qf);
      } else {
        const T* qp = q + ((b * T_ + j) * Hq + h) * D + p * DPT;
#pragma unroll
        for (int d = 0; d < DPT; ++d) qf[d] = Elem<T>::to_f32(qp[d]);
      }
    } else {
#pragma unroll
      for (int d = 0; d < DPT; ++d) qf[d] = 0.0f;
    }
    float m = -INFINITY, s = 0.0f;
    for (int64_t t0 = t_begin; t0 < t_end; t0 += kTileKeys) {
      const int nt = static_cast<int>(min<int64_t>(kTileKeys, t_end - t0));
      __syncthreads();
      for (int e = threadIdx.x; e < nt * (D / V); e += kThreads) {
        const int tt = e / (D / V), cc = e % (D / V);
        float tmp[V];
        unpack16<T>(*reinterpret_cast<const uint4*>(kb + (t0 + tt) * stride_n + cc * V), tmp);
#pragma unroll
        for (int x = 0; x < V; ++x) ks[tt][cc * V + x] = tmp[x];
      }
      __syncthreads();
      for (int tt = 0; tt < nt; ++tt) {
        const float4* kr = reinterpret_cast<const float4*>(&ks[tt][p * DPT]);
        float acc = 0.0f;
        if constexpr (DPT >= 4) {
#pragma unroll
          for (int d4 = 0; d4 < DPT / 4; ++d4) {
            const float4 kk = kr[d4];
            acc += qf[4 * d4] * kk.x + qf[4 * d4 + 1] * kk.y + qf[4 * d4 + 2] * kk.z +
                   qf[4 * d4 + 3] * kk.w;
          }
        } else {
#pragma unroll
          for (int d = 0; d < DPT; ++d) acc += qf[d] * ks[tt][p * DPT + d];
        }
        const float l2 = group_sum<TPR>(acc) * scale2;
        if (l2 > m) {
          s = s * exp2f(m - l2) + 1.0f;
          m = l2;
        } else {
          s += exp2f(l2 - m);
        }
      }
    }
    if (row_ok && p == 0) {
      const int h = g * G + r / T_, j = r % T_;
      float* o = ms + (((b * Hq + h) * T_ + j) * nseg + seg) * 2;
      o[0] = natural ? m * kLn2 : m;
      o[1] = s;
    }
  }
}

// ---------------------------------------------------------------------------
// row statistics: merge the segment partials of each row (one wave per row)
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kThreads)
rowstat_kernel(const float* __restrict__ ms, int64_t rows, int64_t nseg, int natural,
               float* __restrict__ row_max, float* __restrict__ row_sum) {
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const float to2 = natural ? kLog2e : 1.0f;
  float m = -INFINITY, s = 0.0f;
  for (int64_t i = lane; i < nseg; i += 64) {
    const float* p = ms + (row * nseg + i) * 2;
    merge_ms(m, s, p[0] * to2, p[1]);
  }
  const float mw = group_max<64>(m);
  s = (m == -INFINITY) ? 0.0f : s * exp2f(m - mw);
  s = group_sum<64>(s);
  if (lane == 0) {
    row_max[row] = mw * kLn2;
    row_sum[row] = s;
  }
}

// ---------------------------------------------------------------------------
// dispatch
// ---------------------------------------------------------------------------
// rows per slot and step: at least 8 (key, row) pairs per lane.  With
// 1,024-thread workgroups the serving shape (4 query rows per kv head) runs
// fastest at the minimum, 2 rows per step: 5.23-5.33 ms per scoring pass
// against 5.47-5.50 with 4 rows and 5.66-5.68 with 8 (same box).  (Double
// buffering the loads in registers measured the same: the stream runs at the
// memory system's rate.)
template <int R> constexpr int stream_unroll() { return R == 4 ? 2 : R >= 2 ? 4 : 8; }
constexpr int64_t kStreamSegsPerBlock = 2;
// Threads of a streaming-scorer workgroup.  Measured on the serving step (two
// 256-row units of 8 kv heads per workgroup, 1 MiB of keys): 256 threads
// 5.64-5.74 ms, 512 5.56, 1,024 5.41-5.42; 1,024 threads with one unit per
// workgroup 5.52, with four 5.38-5.50 (same box).
constexpr int kStreamThreads = 1024;

template <int D, int H, int R>
void launch_stream(const void* q, int64_t T, int64_t Hq, const void* k, const kvsel_cache& kc,
                   float scale2, int64_t seg_len, int64_t nseg, float* ms, int natural,
                   hipStream_t s) {
  // segments per workgroup: up to kStreamSegsPerBlock while the grid keeps
  // at least 8192 workgroups
  int64_t spb = kStreamSegsPerBlock;
  while (spb > 1 && kc.B * ((nseg + spb - 1) / spb) < 8192) spb /= 2;
  const int64_t groups = (nseg + spb - 1) / spb;
  hipLaunchKernelGGL((score_stream_kernel<D, H, R, stream_unroll<R>(), kStreamThreads>),
                     dim3(static_cast<unsigned>(kc.B * groups)),
                     dim3(kStreamThreads), 0, s, static_cast<const bf16_t*>(q),
                     static_cast<const bf16_t*>(k), kc.N, kc.stride_b, kc.stride_n,
                     static_cast<int>(T), static_cast<int>(Hq), scale2, seg_len, nseg, spb, ms,
                     natural);
}

template <typename T, int D, int TPR>
void launch_tile(const void* q, int64_t T_, int64_t Hq, const void* k, const kvsel_cache& kc,
                 float scale2, int64_t seg_len, int64_t nseg, float* ms, int natural,
                 hipStream_t s) {
  hipLaunchKernelGGL((score_tile_kernel<T, D, TPR>),
                     dim3(static_cast<unsigned>(kc.B * kc.H * nseg)), dim3(kThreads), 0, s,
                     static_cast<const T*>(q), static_cast<const T*>(k), kc.N,
                     static_cast<int>(kc.H), kc.stride_b, kc.stride_n, static_cast<int>(T_),
                     static_cast<int>(Hq), scale2, seg_len, nseg, ms, natural);
}

template <typename T, int D>
void dispatch_tile(const void* q, int64_t T_, int64_t Hq, const void* k, const kvsel_cache& kc,
                   float scale2, int64_t seg_len, int64_t nseg, float* ms, int natural,
                   hipStream_t s) {
  const int64_t R = (Hq / kc.H) * T_;
  // lanes per row: enough rows per pass to fill 256 lanes, at least 4 lanes
  if (R >= 64) launch_tile<T, D, 4>(q, T_, Hq, k, kc, scale2, seg_len, nseg, ms, natural, s);
  else if (R >= 32) launch_tile<T, D, 8>(q, T_, Hq, k, kc, scale2, seg_len, nseg, ms, natural, s);
  else if (R >= 16) launch_tile<T, D, 16>(q, T_, Hq, k, kc, scale2, seg_len, nseg, ms, natural, s);
  else launch_tile<T, D, 32>(q, T_, Hq, k, kc, scale2, seg_len, nseg, ms, natural, s);
}

}  // namespace

bool stream_path_ok(int dtype, int64_t H, int64_t D, int64_t rows_per_kv) {
  if (dtype != KVSEL_BF16 || D != 128) return false;
  if (rows_per_kv != 1 && rows_per_kv != 2 && rows_per_kv != 4 && rows_per_kv != 8) return false;
  return H == 1 || H == 2 || H == 4 || H == 8;
}

int launch_score_partials(const void* q, int64_t T, int64_t Hq, const void* k,
                          const kvsel_cache& kc, float scale, int64_t seg_len, float* ms,
                          int natural, hipStream_t s) {
  const int64_t nseg = (kc.N + seg_len - 1) / seg_len;
  const float scale2 = scale * kLog2e;
  const int64_t R = (Hq / kc.H) * T;
  if (stream_path_ok(kc.dtype, kc.H, kc.D, R)) {
#define KVSEL_SS(H_, R_) \
  if (kc.H == H_ && R == R_) { launch_stream<128, H_, R_>(q, T, Hq, k, kc, scale2, seg_len, nseg, ms, natural, s); return check_launch("kvsel_score"); }
    KVSEL_SS(8, 1) KVSEL_SS(8, 2) KVSEL_SS(8, 4) KVSEL_SS(8, 8)
    KVSEL_SS(4, 1) KVSEL_SS(4, 2) KVSEL_SS(4, 4) KVSEL_SS(4, 8)
    KVSEL_SS(2, 1) KVSEL_SS(2, 2) KVSEL_SS(2, 4) KVSEL_SS(2, 8)
    KVSEL_SS(1, 1) KVSEL_SS(1, 2) KVSEL_SS(1, 4) KVSEL_SS(1, 8)
#undef KVSEL_SS
  }
  if (score_mfma_ok(kc.dtype, R, seg_len)) {
    launch_score_mfma(q, T, Hq, k, kc, scale2, seg_len, nseg, ms, natural, s);
    return check_launch("kvsel_score");
  }
  if (kc.dtype == KVSEL_BF16) {
    if (kc.D == 128) dispatch_tile<bf16_t, 128>(q, T, Hq, k, kc, scale2, seg_len, nseg, ms, natural, s);
    else dispatch_tile<bf16_t, 64>(q, T, Hq, k, kc, scale2, seg_len, nseg, ms, natural, s);
  } else {
    if (kc.D == 128) dispatch_tile<float, 128>(q, T, Hq, k, kc, scale2, seg_len, nseg, ms, natural, s);
    else dispatch_tile<float, 64>(q, T, Hq, k, kc, scale2, seg_len, nseg, ms, natural, s);
  }
  return check_launch("kvsel_score");
}

int launch_rowstats(const float* ms, int64_t rows, int64_t nseg, int natural, float* row_max,
                    float* row_sum, hipStream_t s) {
  const unsigned blocks = static_cast<unsigned>((rows + kWaves - 1) / kWaves);
  hipLaunchKernelGGL(rowstat_kernel, dim3(blocks), dim3(kThreads), 0, s, ms, rows, nseg, natural,
                     row_max, row_sum);
  return check_launch("kvsel_score (row statistics)");
}

}  // namespace kvsel
