// Index-based causal attention of selected tokens (InfoFlow §4.2: a selected
// token is recomputed at its global position, attending to every context row
// up to its own; InfoFlow §8: the pattern is neither dense nor strictly causal).
//
// Row r of kv head g is query head h = g*G + r % G of selected token j = r / G;
// it attends to keys 0 .. lim, lim = min(pos[b][j], N - 1) (none when pos < 0).
// A workgroup's rows are consecutive selected tokens (all G heads of each), so
// with positions listed in ascending order its rows' limits are close; passes
// run from the last rows to the first, so the longest workgroups start first.
//
// Matrix cores, bf16 (lane layout in mfma.h), as the MFMA decode:
//   S^T = K Q^T  (A = 16 keys x 32 dims from the LDS K tile, B = 32 dims x 16
//                 query rows in registers): lane l holds query row l % 16 and
//                 keys 4 * (l / 16) + v of the 16-key block;
//   O^T += V^T P^T (A = 16 dims x 32 keys of V, transposed in LDS as packed
//                 runs of 4 keys; B = the bf16 probabilities of the lane's row).
// A workgroup owns NW * RBW row blocks of 16 rows and walks the key tiles from
// 0 to the largest limit among its rows, all in one pass (no split: the rows
// are many, so partial results would cost more than they save).  Tiles below
// every row's limit of a wave take no mask; past a wave's largest limit the
// wave only helps stage the tiles.  The output is normalised in the kernel.
#include "common.h"
#include "internal.h"
#include "mfma.h"

namespace kvsel {
namespace {

template <int D, int RBW, int NW>
__global__ void __launch_bounds__(64 * NW)
index_attn_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                  const bf16_t* __restrict__ v, int64_t N, int H, int64_t stride_b,
                  int64_t stride_n, const int32_t* __restrict__ pos, int S, int Hq,
                  float scale2, int passes, float* __restrict__ out, float* __restrict__ lse) {
  constexpr int TK = kMfmaTileKeys;
  constexpr int KS = D / 32;
  constexpr int KROW = D + kMfmaPad;
  constexpr int VROW = TK + kMfmaPad;   // transposed V: dims x keys (+32 bytes)
  constexpr int CB = D / 16;            // output column blocks
  constexpr int KG = TK / 4;            // groups of 4 keys
  constexpr int NT = 64 * NW;
  constexpr int NL = NT / 2;               // lead threads: they load and stage the tiles
  constexpr int KV = TK * (D / 8) / NL;    // K vectors per lead thread and tile
  constexpr int VITEMS = KG * (D / 8);     // V items (4 keys x 8 dims) per tile
  constexpr int VI = (VITEMS + NT - 1) / NT;
  static_assert(KV >= 1, "tile too small for the workgroup");
  static_assert(VI == 1, "one V item per thread at most");
  static_assert(VITEMS <= NL, "V is staged by the lead threads");
  __shared__ __align__(16) bf16_t kt[TK * KROW];
  // V of tiles t (t / TK even, odd): with head dim 128 row-major like K and
  // read back transposed (ds_read_b64_tr_b16), else transposed when staged
  constexpr bool VROWMAJ = D == 128;
  __shared__ __align__(16) bf16_t vt2[2][VROWMAJ ? TK * KROW : D * VROW];
  __shared__ int wave_lim[NW];

  int64_t x = blockIdx.x;
  const int pass = passes - 1 - static_cast<int>(x % passes); x /= passes;
  const int g = static_cast<int>(x % H);
  const int64_t b = x / H;
  const int G = Hq / H;
  const int R = G * S;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15, quad = lane >> 4;
  const bf16_t* kb = k + b * stride_b + static_cast<int64_t>(g) * D;
  const bf16_t* vb = v + b * stride_b + static_cast<int64_t>(g) * D;

  // query fragments and the key limit of each of this lane's rows
  uint4 qb[RBW][KS];
  int rb[RBW], lim[RBW];
  int wmax = -1, wmin = 0x7fffffff;
#pragma unroll
  for (int i = 0; i < RBW; ++i) {
    rb[i] = (pass * NW + wave) * RBW + i;
    const int r = rb[i] * 16 + col;
    lim[i] = -1;
    if (r < R) {
      const int h = g * G + r % G, j = r / G;
      const uint4* qp = reinterpret_cast<const uint4*>(q + ((b * S + j) * Hq + h) * D + quad * 8);
#pragma unroll
      for (int s2 = 0; s2 < KS; ++s2) qb[i][s2] = qp[s2 * 4];
      const int64_t p = pos[b * S + j];
      lim[i] = p < 0 ? -1 : static_cast<int>(min<int64_t>(p, N - 1));
    } else {
#pragma unroll
      for (int s2 = 0; s2 < KS; ++s2) qb[i][s2] = make_uint4(0, 0, 0, 0);
    }
    wmax = max(wmax, lim[i]);
    wmin = min(wmin, lim[i]);
  }
  // wave extremes (every quad of a lane column holds the same rows)
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) {
    wmax = max(wmax, __shfl_xor(wmax, off, 64));
    wmin = min(wmin, __shfl_xor(wmin, off, 64));
  }
  if (lane == 0) wave_lim[wave] = wmax;
  __syncthreads();
  int64_t t_end = 0;  // the workgroup's keys: 0 .. largest limit
#pragma unroll
  for (int w = 0; w < NW; ++w) t_end = max<int64_t>(t_end, wave_lim[w] + 1);

  float m[RBW], s[RBW];
  f32x4_t o[RBW][CB];
#pragma unroll
  for (int i = 0; i < RBW; ++i) {
    m[i] = -INFINITY;
    s[i] = 0.0f;
#pragma unroll
    for (int c = 0; c < CB; ++c) o[i][c] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }

  // the next tile's K and V rows are in flight while this tile computes.  Keys
  // from t_end on lie beyond every row's limit and get zero weight from the
  // mask, so a tile is loaded whole; only rows past the cache's end are
  // clamped to its last row.
  uint4 kn[KV], vn4[VI][4];
  // a lead thread's rows within a tile: K rows key0 + i * (NL / (D / 8)), V rows
  // 4 * (thread % KG) + j
  const int64_t koff = (threadIdx.x / (D / 8)) * stride_n + (threadIdx.x % (D / 8)) * 8;
  const int64_t voff = (threadIdx.x % KG) * 4 * stride_n + (threadIdx.x / KG) * 8;
  const int64_t kstep = (NL / (D / 8)) * stride_n;
  auto fetch = [&](int64_t t0) {
    if (t0 + TK <= N) {   // uniform
      const bf16_t* kt0 = kb + t0 * stride_n;
      const bf16_t* vt0 = vb + t0 * stride_n;
#pragma unroll
      for (int i = 0; i < KV; ++i) {
        const uint4 x = *reinterpret_cast<const uint4*>(kt0 + koff + i * kstep);
        kn[i] = x;
      }
      if constexpr (VROWMAJ) {      // V rows as the K rows
#pragma unroll
        for (int i = 0; i < KV; ++i) {
          const uint4 y = *reinterpret_cast<const uint4*>(vt0 + koff + i * kstep);
          vn4[0][i] = y;
        }
      } else if (threadIdx.x < VITEMS) {   // the other threads stage no V
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint4 y = *reinterpret_cast<const uint4*>(vt0 + voff + j * stride_n);
          vn4[0][j] = y;
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < KV; ++i) {
        const int e = threadIdx.x + i * NL;
        const int64_t t = min<int64_t>(t0 + e / (D / 8), N - 1);
        const uint4 x = *reinterpret_cast<const uint4*>(kb + t * stride_n + (e % (D / 8)) * 8);
        kn[i] = x;
      }
      if constexpr (VROWMAJ) {
#pragma unroll
        for (int i = 0; i < KV; ++i) {
          const int e = threadIdx.x + i * NL;
          const int64_t t = min<int64_t>(t0 + e / (D / 8), N - 1);
          const uint4 y = *reinterpret_cast<const uint4*>(vb + t * stride_n + (e % (D / 8)) * 8);
          vn4[0][i] = y;
        }
      } else if (threadIdx.x < VITEMS) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t t = min<int64_t>(t0 + (threadIdx.x % KG) * 4 + j, N - 1);
          const uint4 y = *reinterpret_cast<const uint4*>(vb + t * stride_n + (threadIdx.x / KG) * 8);
          vn4[0][j] = y;
        }
      }
    }
  };
  // S^T blocks of the staged K tile: key block outer, so one K fragment
  // serves every row block
  auto scores = [&](f32x4_t (&sv)[RBW][4]) {
#pragma unroll
    for (int kb4 = 0; kb4 < 4; ++kb4) {
      uint4 ka[KS];
#pragma unroll
      for (int s2 = 0; s2 < KS; ++s2)
        ka[s2] = *reinterpret_cast<const uint4*>(&kt[(kb4 * 16 + col) * KROW + s2 * 32 + quad * 8]);
#pragma unroll
      for (int i = 0; i < RBW; ++i) {
        f32x4_t a = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s2 = 0; s2 < KS; ++s2) a = mfma16x16x32(ka[s2], qb[i][s2], a);
        sv[i][kb4] = a;
      }
    }
  };
  // the causal limit, softmax and value products of the tile at tt (its V
  // staged in vtt)
  auto apply = [&](f32x4_t (&sv)[RBW][4], int64_t tt, const bf16_t* vtt) {
    // the causal limit, only in tiles that reach past some row's limit
    if (tt + TK - 1 > wmin) {
#pragma unroll
      for (int i = 0; i < RBW; ++i)
#pragma unroll
        for (int kb4 = 0; kb4 < 4; ++kb4)
#pragma unroll
          for (int vv = 0; vv < 4; ++vv)
            if (tt + kb4 * 16 + quad * 4 + vv > lim[i]) sv[i][kb4][vv] = -INFINITY;
    }
    // online softmax per row (the lane's column); probabilities as bf16 pairs
    uint32_t pk[RBW][4][2];
#pragma unroll
    for (int i = 0; i < RBW; ++i) attn_softmax<CB>(sv[i], scale2, m[i], s[i], o[i], pk[i]);
    // O^T += V^T P^T: one V^T fragment serves every row block
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) {
#pragma unroll
      for (int c = 0; c < CB; ++c) {
        uint4 va;
        if constexpr (VROWMAJ) va = load_vt_tr<KROW>(vtt, c, pr, lane);
        else va = load_vt<VROW>(vtt, c, pr, col, quad);
#pragma unroll
        for (int i = 0; i < RBW; ++i) {
          const uint4 pb = make_uint4(pk[i][2 * pr][0], pk[i][2 * pr][1], pk[i][2 * pr + 1][0],
                                      pk[i][2 * pr + 1][1]);
          o[i][c] = mfma16x16x32(va, pb, o[i][c]);
        }
      }
    }
  };
  // Waves NW/2 .. NW-1 (one per SIMD beside a lead wave) run one tile behind
  // the lead waves, so that on each SIMD one wave's products overlap the
  // other's softmax; V is staged in two buffers for them.  The lead waves load
  // and stage every tile.  Both loops meet the same two barriers per tile.
  if (wave < NW / 2) {
    if (t_end > 0) fetch(0);
    for (int64_t t0 = 0; t0 < t_end; t0 += TK) {
      __syncthreads();               // every wave is done with the buffers restaged here
#pragma unroll
      for (int i = 0; i < KV; ++i) {
        const int e = threadIdx.x + i * NL;
        const int key = e / (D / 8), ch = e % (D / 8);
        *reinterpret_cast<uint4*>(&kt[key * KROW + ch * 8]) = kn[i];
      }
      bf16_t* vt = vt2[(t0 / TK) & 1];
      if constexpr (VROWMAJ) {
#pragma unroll
        for (int i = 0; i < KV; ++i) {
          const int e = threadIdx.x + i * NL;
          *reinterpret_cast<uint4*>(&vt[(e / (D / 8)) * KROW + (e % (D / 8)) * 8]) = vn4[0][i];
        }
      } else if (threadIdx.x < VITEMS) {
        stage_vt<VROW>(vt, vn4[0], threadIdx.x % KG, threadIdx.x / KG);
      }
      __syncthreads();
      if (t0 + TK < t_end) fetch(t0 + TK);
      if (t0 > wmax) continue;       // this wave's rows are complete (uniform)
      f32x4_t sv[RBW][4];
      scores(sv);
      apply(sv, t0, vt);
    }
  } else {
    // the previous tile's softmax and value products (its V is still staged)
    // first, then this tile's scores: vector work while the lead wave on this
    // SIMD runs its score products
    f32x4_t svp[RBW][4];
    bool have_prev = false;
    for (int64_t t0 = 0; t0 < t_end; t0 += TK) {
      __syncthreads();
      __syncthreads();               // the tile at t0 is staged
      if (have_prev) apply(svp, t0 - TK, vt2[((t0 - TK) / TK) & 1]);
      have_prev = t0 <= wmax;
      if (have_prev) scores(svp);
    }
    if (have_prev) {
      const int64_t last = (t_end - 1) / TK * TK;
      apply(svp, last, vt2[(last / TK) & 1]);
    }
  }

  // normalised output: lane l holds row rb*16 + l%16, dims c*16 + 4*quad .. +3
#pragma unroll
  for (int i = 0; i < RBW; ++i) {
    float tot = s[i];
    tot += __shfl_xor(tot, 16, 64);
    tot += __shfl_xor(tot, 32, 64);
    const int r = rb[i] * 16 + col;
    if (r >= R) continue;
    const int h = g * G + r % G, j = r / G;
    const float inv = tot > 0.0f ? 1.0f / tot : 0.0f;
    float* wo = out + ((b * S + j) * Hq + h) * D;
#pragma unroll
    for (int c = 0; c < CB; ++c)
      *reinterpret_cast<float4*>(wo + c * 16 + quad * 4) =
          make_float4(o[i][c][0] * inv, o[i][c][1] * inv, o[i][c][2] * inv, o[i][c][3] * inv);
    if (lse != nullptr && quad == 0)
      lse[(b * Hq + h) * S + j] = tot > 0.0f ? (m[i] + log2f(tot)) * kLn2 : -INFINITY;
  }
}

template <int D, int RBW, int NW>
void launch(const void* q, int64_t S, int64_t Hq, float scale2, const void* k, const void* v,
            const kvsel_cache& kc, const int32_t* pos, float* out, float* lse, hipStream_t s) {
  const int64_t R = (Hq / kc.H) * S;
  const int64_t rows_per_wg = 16 * RBW * NW;
  const int passes = static_cast<int>((R + rows_per_wg - 1) / rows_per_wg);
  hipLaunchKernelGGL((index_attn_kernel<D, RBW, NW>),
                     dim3(static_cast<unsigned>(kc.B * kc.H * passes)), dim3(64 * NW), 0, s,
                     static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k),
                     static_cast<const bf16_t*>(v), kc.N, static_cast<int>(kc.H), kc.stride_b,
                     kc.stride_n, pos, static_cast<int>(S), static_cast<int>(Hq), scale2, passes,
                     out, lse);
}

}  // namespace

int64_t index_attn_blocks(const kvsel_cache& kc, int64_t S, int64_t Hq) {
  const int64_t R = (Hq / kc.H) * S;
  const int64_t rows_per_wg = R > 4096 ? 256 : 128;
  return kc.B * kc.H * ((R + rows_per_wg - 1) / rows_per_wg);
}

int launch_index_attn(const void* q, int64_t S, int64_t Hq, float scale, const void* k,
                      const void* v, const kvsel_cache& kc, const int32_t* pos, float* out,
                      float* lse, hipStream_t s) {
  const float scale2 = scale * kLog2e;
  const int64_t R = (Hq / kc.H) * S;
  // many rows per kv head: two row blocks per wave (each staged tile serves
  // twice as many rows); few: one
  if (kc.D == 128) {
    if (R > 4096) launch<128, 2, 8>(q, S, Hq, scale2, k, v, kc, pos, out, lse, s);
    else launch<128, 1, 8>(q, S, Hq, scale2, k, v, kc, pos, out, lse, s);
  } else {
    if (R > 4096) launch<64, 2, 8>(q, S, Hq, scale2, k, v, kc, pos, out, lse, s);
    else launch<64, 1, 8>(q, S, Hq, scale2, k, v, kc, pos, out, lse, s);
  }
  return check_launch("kvsel_index_attn");
}

}  // namespace kvsel
