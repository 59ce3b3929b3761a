// Query block -> cached keys on the matrix cores, for bf16 caches whose kv
// heads carry >= 16 query rows (query heads per kv head x query tokens).
// Same outputs as the streaming and tile paths of score.hip: per row and
// segment of cached rows, (m, s) = (max logit, sum of exp(l - m)) in the log2
// domain (ACRE §2.4, A = softmax(Q_q K^T / sqrt(d)); ACRE §2.1 Eq. 4).
//
// S = Q K^T with v_mfma_f32_16x16x32_bf16: A = 16 query rows x 32 dims held in
// registers for the whole block, B = 32 dims x 16 keys read from a 64-key tile
// of K staged in LDS (rows padded by 16 bytes, so the 16 keys a read spans hit
// distinct banks).  Lane l of a 16x16 result holds key l%16 of the block and
// rows 4*(l/16) .. +3.
//
// The four waves split the tile's (row block, key block) pairs: NWR waves
// across row blocks, 4/NWR across key blocks.  Every lane keeps a softmax
// partial per row it holds, over the keys of its column; per tile it first
// takes the max over those keys, then adds one exp per logit.  At the end of a
// segment the partials merge across the 16 key lanes (DPP) and across the waves
// that shared the rows (LDS), in a fixed order.
#include "common.h"
#include "internal.h"
#include "mfma.h"

namespace kvsel {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kTileKeys = kMfmaTileKeys;
constexpr int kPad = kMfmaPad;

// (m, s) merge with the lane holding the same rows in another key column
__device__ __forceinline__ void merge_cols(float& m, float& s) {
  merge_ms(m, s, dpp_xor1(m), dpp_xor1(s));
  merge_ms(m, s, dpp_xor2(m), dpp_xor2(s));
  merge_ms(m, s, dpp_half_mirror(m), dpp_half_mirror(s));
  merge_ms(m, s, dpp_mirror(m), dpp_mirror(s));
}

// Re-positioning fused into the staging of K (kvsel_score_reposition): every
// unit of rot_len cached rows (a multiple of the tile) is rotated by delta[u]
// positions with the same fp64 arithmetic and single rounding as
// kvsel_reposition, so the scored keys are bit-identical to that call's
// output; with WRITE the re-positioned keys are also stored to kout.
struct ScoreRot {
  const int64_t* delta;      // [M] or [B][M] (delta_stride_b = M)
  int64_t delta_stride_b;
  int64_t rot_len;
  double base;
  bf16_t* kout;              // same layout as k, or NULL
};

// D: head dim; RBW: row blocks per wave; NWR: waves across row blocks;
// ROT: 0 none, 1 half-split pairs, 2 interleaved pairs; WRITE: store K'.
template <int D, int RBW, int NWR, int ROT, bool WRITE>
__global__ void __launch_bounds__(kThreads)
score_mfma_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, int64_t N, int H,
                  int64_t stride_b, int64_t stride_n, int T, int Hq, float scale2,
                  int64_t seg_len, int64_t nseg, int64_t segs_per_block, int64_t groups,
                  int passes, float* __restrict__ ms, int natural, ScoreRot rot) {
  constexpr int KS = D / 32;                 // MFMA k-steps
  constexpr int KROW = D + kPad;             // staged row stride (elements)
  constexpr int NWK = kWaves / NWR;          // waves across key blocks
  constexpr int KBW = (kTileKeys / 16) / NWK;  // key blocks per wave and tile
  constexpr int VPT = kTileKeys * D / 8 / kThreads;  // 16-byte vectors per thread and tile
  constexpr int ROWS_PASS = NWR * RBW * 16;
  __shared__ __align__(16) bf16_t kt[kTileKeys * KROW];
  __shared__ float red[NWK][ROWS_PASS][2];
  __shared__ double2 cs[ROT ? D / 2 : 1];

  int64_t x = blockIdx.x;
  const int64_t grp = x % groups; x /= groups;
  const int pass = static_cast<int>(x % passes); x /= passes;
  const int g = static_cast<int>(x % H);
  const int64_t b = x / H;
  const int G = Hq / H;
  const int R = G * T;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wr = wave % NWR, wk = wave / NWR;
  const int col = lane & 15, quad = lane >> 4;

  // query fragments of this wave's row blocks (rows past R are zero)
  uint4 qa[RBW][KS];
#pragma unroll
  for (int i = 0; i < RBW; ++i) {
    const int r = (pass * NWR * RBW + wr + i * NWR) * 16 + col;
    if (r < R) {
      const int h = g * G + r / T, j = r % T;
      const uint4* qp = reinterpret_cast<const uint4*>(q + ((b * T + j) * Hq + h) * D + quad * 8);
#pragma unroll
      for (int s = 0; s < KS; ++s) qa[i][s] = qp[s * 4];
    } else {
#pragma unroll
      for (int s = 0; s < KS; ++s) qa[i][s] = make_uint4(0, 0, 0, 0);
    }
  }

  const int64_t seg0 = grp * segs_per_block;
  const int64_t seg1 = min(nseg, seg0 + segs_per_block);
  const int64_t t_begin = seg0 * seg_len;
  const int64_t t_end = min(N, seg1 * seg_len);
  const bf16_t* kb = k + b * stride_b + static_cast<int64_t>(g) * D;

  // staging of one tile.  Vector i of a thread is (key, chunk) of item
  // e = tid + (i / P) * 256 (P = 2 with half-split rotation: chunk c and its
  // partner c + D/16 travel together; else P = 1 and item e is chunk e).
  constexpr int P = ROT == 1 ? 2 : 1;
  constexpr int CPK = D / 8 / P;  // items per key
  auto item = [&](int i, int& key, int& ch) {
    const int e = threadIdx.x + (i / P) * kThreads;
    key = e / CPK;
    ch = e % CPK + (i % P) * (D / 16);
  };
  auto fetch = [&](uint4 (&v)[VPT], int64_t t0) {
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      int key, ch;
      item(i, key, ch);
      v[i] = (t0 + key < t_end)
                 ? *reinterpret_cast<const uint4*>(kb + (t0 + key) * stride_n + ch * 8)
                 : make_uint4(0, 0, 0, 0);
    }
  };
  const bool write_out = WRITE && pass == 0;
  auto stash = [&](uint4 (&v)[VPT], int64_t t0) {
    if constexpr (ROT == 1) {
#pragma unroll
      for (int i = 0; i < VPT; i += 2) {
        int key, ch;
        item(i, key, ch);
        rope_rotate16<bf16_t, KVSEL_ROPE_HALF>(v[i], v[i + 1], ch * 8, cs);
      }
    } else if constexpr (ROT == 2) {
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        int key, ch;
        item(i, key, ch);
        uint4 unused;
        rope_rotate16<bf16_t, KVSEL_ROPE_INTERLEAVED>(v[i], unused, ch * 8, cs);
      }
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      int key, ch;
      item(i, key, ch);
      *reinterpret_cast<uint4*>(&kt[key * KROW + ch * 8]) = v[i];
      if (write_out && t0 + key < t_end)
        *reinterpret_cast<uint4*>(rot.kout + b * stride_b + (t0 + key) * stride_n +
                                  static_cast<int64_t>(g) * D + ch * 8) = v[i];
    }
  };
  int64_t cs_unit = -1;

  float m[RBW][4], s[RBW][4];
#pragma unroll
  for (int i = 0; i < RBW; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) { m[i][v] = -INFINITY; s[i][v] = 0.0f; }

  uint4 nxt[VPT];
  if (t_begin < t_end) fetch(nxt, t_begin);
  for (int64_t t0 = t_begin; t0 < t_end; t0 += kTileKeys) {
    __syncthreads();               // previous tile fully read
    if constexpr (ROT != 0) {
      const int64_t u = t0 / rot.rot_len;  // a tile lies inside one unit
      if (u != cs_unit) {
        const int64_t delta = rot.delta[b * rot.delta_stride_b + u];
        for (int i = threadIdx.x; i < D / 2; i += kThreads) cs[i] = rope_cs(delta, i, D, rot.base);
        cs_unit = u;
        __syncthreads();
      }
    }
    stash(nxt, t0);
    __syncthreads();
    if (t0 + kTileKeys < t_end) fetch(nxt, t0 + kTileKeys);  // in flight during the math

    f32x4_t acc[RBW][KBW];
#pragma unroll
    for (int jb = 0; jb < KBW; ++jb) {
      const int key = (wk + jb * NWK) * 16 + col;
      uint4 bk[KS];
#pragma unroll
      for (int st = 0; st < KS; ++st)
        bk[st] = *reinterpret_cast<const uint4*>(&kt[key * KROW + st * 32 + quad * 8]);
#pragma unroll
      for (int i = 0; i < RBW; ++i) {
        f32x4_t a = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int st = 0; st < KS; ++st)
          a = mfma16x16x32(qa[i][st], bk[st], a);
        acc[i][jb] = a;
      }
    }
    // keys past the end of the cache take no part
#pragma unroll
    for (int jb = 0; jb < KBW; ++jb) {
      if (t0 + (wk + jb * NWK) * 16 + col >= t_end) {
#pragma unroll
        for (int i = 0; i < RBW; ++i) acc[i][jb] = f32x4_t{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      }
    }
#pragma unroll
    for (int i = 0; i < RBW; ++i) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float tmax = acc[i][0][v];
#pragma unroll
        for (int jb = 1; jb < KBW; ++jb) tmax = fmaxf(tmax, acc[i][jb][v]);
        const float mn = fmaxf(m[i][v], tmax * scale2);
        if (mn == -INFINITY) continue;
        float acc_s = s[i][v] * __builtin_amdgcn_exp2f(m[i][v] - mn);
#pragma unroll
        for (int jb = 0; jb < KBW; ++jb)
          acc_s += __builtin_amdgcn_exp2f(fmaf(acc[i][jb][v], scale2, -mn));
        s[i][v] = acc_s;
        m[i][v] = mn;
      }
    }

    // end of a segment: merge and publish its partials
    const int64_t t_next = t0 + kTileKeys;
    if (t_next % seg_len == 0 || t_next >= t_end) {
      const int64_t seg = (t0 + kTileKeys - 1) / seg_len;
#pragma unroll
      for (int i = 0; i < RBW; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) merge_cols(m[i][v], s[i][v]);
      if (col == 0) {
#pragma unroll
        for (int i = 0; i < RBW; ++i)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int rl = (wr + i * NWR) * 16 + quad * 4 + v;  // row within the pass
            red[wk][rl][0] = m[i][v];
            red[wk][rl][1] = s[i][v];
          }
      }
      __syncthreads();
      for (int rl = threadIdx.x; rl < ROWS_PASS; rl += kThreads) {
        const int r = pass * ROWS_PASS + rl;
        if (r >= R) continue;
        float mm = red[0][rl][0], ss = red[0][rl][1];
#pragma unroll
        for (int w = 1; w < NWK; ++w) merge_ms(mm, ss, red[w][rl][0], red[w][rl][1]);
        const int h = g * G + r / T, j = r % T;
        float* o = ms + (((b * Hq + h) * T + j) * nseg + seg) * 2;
        o[0] = natural ? mm * kLn2 : mm;
        o[1] = ss;
      }
#pragma unroll
      for (int i = 0; i < RBW; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) { m[i][v] = -INFINITY; s[i][v] = 0.0f; }
    }
  }
}

template <int D, int RBW, int NWR, int ROT, bool WRITE>
void launch(const void* q, int64_t T, int64_t Hq, const void* k, const kvsel_cache& kc,
            float scale2, int64_t seg_len, int64_t nseg, int64_t spb, int passes, float* ms,
            int natural, const ScoreRot& rot, hipStream_t s) {
  const int64_t groups = (nseg + spb - 1) / spb;
  const int64_t blocks = kc.B * kc.H * passes * groups;
  hipLaunchKernelGGL((score_mfma_kernel<D, RBW, NWR, ROT, WRITE>),
                     dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, s,
                     static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k), kc.N,
                     static_cast<int>(kc.H), kc.stride_b, kc.stride_n, static_cast<int>(T),
                     static_cast<int>(Hq), scale2, seg_len, nseg, spb, groups, passes, ms, natural,
                     rot);
}

template <int D, int ROT, bool WRITE>
void dispatch(const void* q, int64_t T, int64_t Hq, const void* k, const kvsel_cache& kc,
              float scale2, int64_t seg_len, int64_t nseg, float* ms, int natural,
              const ScoreRot& rot, hipStream_t s) {
  const MfmaRowPlan p = mfma_row_plan((Hq / kc.H) * T);
  // up to 1024 keys per workgroup (segments of 256 go four to a block), fewer
  // when that leaves under ~2048 workgroups for the 256 CUs
  int64_t spb = seg_len >= 1024 ? 1 : 1024 / seg_len;
  while (spb > 1 && kc.B * kc.H * p.passes * ((nseg + spb - 1) / spb) < 2048) spb /= 2;
#define KVSEL_SM(RBW, NWR)                                                                 \
  if (p.rbw == RBW && p.nwr == NWR)                                                        \
    return launch<D, RBW, NWR, ROT, WRITE>(q, T, Hq, k, kc, scale2, seg_len, nseg, spb,    \
                                           p.passes, ms, natural, rot, s);
  KVSEL_SM(1, 1) KVSEL_SM(1, 2) KVSEL_SM(1, 4) KVSEL_SM(2, 4) KVSEL_SM(4, 4)
#undef KVSEL_SM
}

}  // namespace

bool score_mfma_ok(int dtype, int64_t rows_per_kv, int64_t seg_len) {
  return dtype == KVSEL_BF16 && rows_per_kv >= 16 && seg_len % kTileKeys == 0;
}

bool score_mfma_rot_ok(int dtype, int64_t rows_per_kv, int64_t seg_len, int64_t rot_len) {
  return score_mfma_ok(dtype, rows_per_kv, seg_len) && rot_len % kTileKeys == 0;
}

void launch_score_mfma(const void* q, int64_t T, int64_t Hq, const void* k,
                       const kvsel_cache& kc, float scale2, int64_t seg_len, int64_t nseg,
                       float* ms, int natural, hipStream_t s) {
  const ScoreRot none{nullptr, 0, 1, 0.0, nullptr};
  if (kc.D == 128)
    dispatch<128, 0, false>(q, T, Hq, k, kc, scale2, seg_len, nseg, ms, natural, none, s);
  else
    dispatch<64, 0, false>(q, T, Hq, k, kc, scale2, seg_len, nseg, ms, natural, none, s);
}

void launch_score_mfma_rot(const void* q, int64_t T, int64_t Hq, const void* k, void* k_out,
                           const kvsel_cache& kc, float scale, int64_t seg_len, int64_t nseg,
                           float* ms, int natural, int64_t rot_len, const int64_t* delta,
                           int per_instance, double base, int style, hipStream_t s) {
  const float scale2 = scale * kLog2e;
  const ScoreRot rot{delta, per_instance ? kc.N / rot_len : 0, rot_len, base,
                     static_cast<bf16_t*>(k_out)};
  const bool w = k_out != nullptr;
#define KVSEL_SR(D_, ST)                                                                   \
  if (w) dispatch<D_, ST, true>(q, T, Hq, k, kc, scale2, seg_len, nseg, ms, natural, rot, s); \
  else dispatch<D_, ST, false>(q, T, Hq, k, kc, scale2, seg_len, nseg, ms, natural, rot, s);
  if (kc.D == 128) {
    if (style == KVSEL_ROPE_HALF) { KVSEL_SR(128, 1) } else { KVSEL_SR(128, 2) }
  } else {
    if (style == KVSEL_ROPE_HALF) { KVSEL_SR(64, 1) } else { KVSEL_SR(64, 2) }
  }
#undef KVSEL_SR
}

}  // namespace kvsel
