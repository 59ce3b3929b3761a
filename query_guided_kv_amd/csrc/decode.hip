// Final attention pass over the compact cache (ACRE §2.1 Eq. 4; decoding on
// the refilled cache, ACRE §2.4).
//
// Split-K: the keys of every segment are cut into splits (decode_split_len
// rows); one workgroup computes, for its split, each row's reference m, sum s
// and unnormalised output o (online softmax in the log2 domain).  A merge
// kernel combines the splits of a row with the usual rescaling and writes
// o / s and lse = (m + log2 s) * ln 2.
//
// stream variant: bf16, head dim 128, 1 to 4 rows per kv head (up to 8 when it
// gathers the kept rows on the fly).  Lanes own 32 bytes of a key row and the
// matching 32 bytes of the value row; logits use packed bf16 dots and an
// 8-lane DPP reduction; the four waves' partials are merged through LDS one
// wave at a time.
// matrix-core variant: bf16, 5 or more rows per kv head (below).
// tile variant: any other shape; keys and values staged through LDS as fp32.
#include "common.h"
#include "internal.h"
#include "mfma.h"

#include <type_traits>

namespace kvsel {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Word 3 of a raw buffer resource on gfx9-family parts: 32-bit data format,
// so untyped loads return whole dwords and out-of-range ones return zero.
constexpr int kBufferDword3 = 0x00020000;

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

struct SegTable {
  const void* k[kMaxSegments];
  const void* v[kMaxSegments];
  int64_t N[kMaxSegments];
  int64_t stride_b[kMaxSegments];
  int64_t stride_n[kMaxSegments];
  int64_t split_begin[kMaxSegments + 1];
  int64_t split_len;         // keys per split (decode_split_len)
  // At most one segment is gathered on the fly: its row t is source row
  // idx[t / unit_len] * unit_len + t % unit_len of (k, v) above, and the kernel
  // also writes that row to row t of the compact destination (k_dst, v_dst).
  int gather_seg;            // -1 when no segment is gathered
  const int32_t* idx;        // [B / idx_group][n_kept], kept unit ids
  int64_t unit_len, n_kept, idx_group, n_units;
  void* k_dst;
  void* v_dst;
};

// Which segment and key range a split covers.
__device__ __forceinline__ int find_seg(const SegTable& st, int n_seg, int64_t sp) {
  int sg = 0;
  while (sg + 1 < n_seg && sp >= st.split_begin[sg + 1]) ++sg;
  return sg;
}

// ---------------------------------------------------------------------------
// stream variant
// ---------------------------------------------------------------------------
// R: query rows per kv head rounded up to 1, 2, 4 or 8; rows past `rows`
// (the real count) carry zero queries and are not written.
template <int D, int H, int R, int UNROLL>
__global__ void __launch_bounds__(kThreads)
decode_stream_kernel(const bf16_t* __restrict__ q, SegTable st, int n_seg, int64_t n_split,
                     int T, int Hq, int rows, float scale2, float* __restrict__ ws_ms,
                     float* __restrict__ ws_o) {
  constexpr int LPH = D / 16;
  constexpr int LPT = H * LPH;
  constexpr int TPW = 64 / LPT;
  static_assert(LPT <= 64 && 64 % LPT == 0, "row must tile a wave");
  constexpr int ROWS = H * R;
  __shared__ float red_o[ROWS][D];
  __shared__ float red_ms[ROWS][2];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int slot = lane / LPT;
  const int g = (lane % LPT) / LPH;
  const int c = lane % LPH;
  const int64_t b = blockIdx.x / static_cast<uint32_t>(n_split);   // 32-bit: the grid is below 2^32 workgroups
  const int64_t sp = blockIdx.x % static_cast<uint32_t>(n_split);
  const int sg = find_seg(st, n_seg, sp);
  const int64_t t_begin = (sp - st.split_begin[sg]) * st.split_len;
  const int64_t t_end = min(st.N[sg], t_begin + st.split_len);
  const int G = Hq / H;

  // gathered segment: the kept unit ids that this split's rows come from
  __shared__ int32_t s_unit[kDecodeSplit];
  const bool gathered = sg == st.gather_seg;
  int64_t u_first = 0;
  if (gathered) {
    u_first = t_begin / st.unit_len;
    const int64_t nu = (t_end - 1) / st.unit_len - u_first + 1;
    const int32_t* ib = st.idx + (b / st.idx_group) * st.n_kept + u_first;
    for (int64_t i = threadIdx.x; i < nu; i += kThreads) {
      const int32_t u = ib[i];
      s_unit[i] = (u >= 0 && u < st.n_units) ? u : -1;
    }
  }
  __syncthreads();

  uint32_t qv[R][8];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int h = g * G + r / T, j = r % T;
    uint4 q0 = make_uint4(0, 0, 0, 0), q1 = q0;
    if (r < rows) {
      const uint4* qp = reinterpret_cast<const uint4*>(q + ((b * T + j) * Hq + h) * D + c * 16);
      q0 = qp[0];
      q1 = qp[1];
    }
    qv[r][0] = q0.x; qv[r][1] = q0.y; qv[r][2] = q0.z; qv[r][3] = q0.w;
    qv[r][4] = q1.x; qv[r][5] = q1.y; qv[r][6] = q1.z; qv[r][7] = q1.w;
  }
  float m[R], s[R], o[R][16];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    m[r] = -INFINITY;
    s[r] = 0.0f;
#pragma unroll
    for (int d = 0; d < 16; ++d) o[r][d] = 0.0f;
  }

  const int64_t off0 = g * D + c * 16;
  const bf16_t* kb = static_cast<const bf16_t*>(st.k[sg]) + b * st.stride_b[sg] + off0;
  const bf16_t* vb = static_cast<const bf16_t*>(st.v[sg]) + b * st.stride_b[sg] + off0;
  const int64_t sn = st.stride_n[sg];
  constexpr int64_t ROW = static_cast<int64_t>(H) * D;  // elements of a compact row
  bf16_t* kd = gathered ? static_cast<bf16_t*>(st.k_dst) + b * st.N[sg] * ROW + off0 : nullptr;
  bf16_t* vd = gathered ? static_cast<bf16_t*>(st.v_dst) + b * st.N[sg] * ROW + off0 : nullptr;
  constexpr int STEP = kWaves * TPW;
  for (int64_t t0 = t_begin + wave * TPW + slot; t0 < t_end; t0 += STEP * UNROLL) {
    uint4 kr[UNROLL][2], vr[UNROLL][2];
    bool ok[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int64_t t = t0 + static_cast<int64_t>(u) * STEP;
      ok[u] = t < t_end;
      int64_t src = t;
      if (gathered && ok[u]) {
        const int64_t r = t / st.unit_len;
        const int32_t unit = s_unit[r - u_first];
        ok[u] = unit >= 0;
        src = static_cast<int64_t>(unit) * st.unit_len + (t - r * st.unit_len);
      }
      if (ok[u]) {
        const uint4* kp = reinterpret_cast<const uint4*>(kb + src * sn);
        const uint4* vp = reinterpret_cast<const uint4*>(vb + src * sn);
        kr[u][0] = kp[0]; kr[u][1] = kp[1];
        vr[u][0] = vp[0]; vr[u][1] = vp[1];
      } else {
        kr[u][0] = kr[u][1] = vr[u][0] = vr[u][1] = make_uint4(0, 0, 0, 0);
      }
    }
    if (gathered) {
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        if (!ok[u]) continue;
        const int64_t t = t0 + static_cast<int64_t>(u) * STEP;
        uint4* kq = reinterpret_cast<uint4*>(kd + t * ROW);
        uint4* vq = reinterpret_cast<uint4*>(vd + t * ROW);
        kq[0] = kr[u][0]; kq[1] = kr[u][1];
        vq[0] = vr[u][0]; vq[1] = vr[u][1];
      }
    }
    float l2[UNROLL][R];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const uint32_t kw[8] = {kr[u][0].x, kr[u][0].y, kr[u][0].z, kr[u][0].w,
                              kr[u][1].x, kr[u][1].y, kr[u][1].z, kr[u][1].w};
      const bool valid = ok[u];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float acc = 0.0f;
#pragma unroll
        for (int p = 0; p < 8; ++p) acc = dot2(qv[r][p], kw[p], acc);
        acc = group_sum<LPH>(acc);
        l2[u][r] = valid ? acc * scale2 : -INFINITY;
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float bm = l2[0][r];
#pragma unroll
      for (int u = 1; u < UNROLL; ++u) bm = fmaxf(bm, l2[u][r]);
      const float mn = fmaxf(m[r], bm);
      if (mn == -INFINITY) continue;
      const float alpha = exp2f(m[r] - mn);
      float pu[UNROLL];
      float ps = 0.0f;
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) { pu[u] = exp2f(l2[u][r] - mn); ps += pu[u]; }
      s[r] = s[r] * alpha + ps;
      m[r] = mn;
#pragma unroll
      for (int d = 0; d < 16; ++d) o[r][d] *= alpha;
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const uint32_t vw[8] = {vr[u][0].x, vr[u][0].y, vr[u][0].z, vr[u][0].w,
                                vr[u][1].x, vr[u][1].y, vr[u][1].z, vr[u][1].w};
#pragma unroll
        for (int p = 0; p < 8; ++p) {
          o[r][2 * p] += pu[u] * bf16_lo(vw[p]);
          o[r][2 * p + 1] += pu[u] * bf16_hi(vw[p]);
        }
      }
    }
  }

  // merge the TPW row slots of the wave
#pragma unroll
  for (int off = LPT; off < 64; off <<= 1) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float m2 = __shfl_xor(m[r], off, 64);
      const float s2 = __shfl_xor(s[r], off, 64);
      const float mn = fmaxf(m[r], m2);
      const float a1 = (m[r] == -INFINITY) ? 0.0f : exp2f(m[r] - mn);
      const float a2 = (m2 == -INFINITY) ? 0.0f : exp2f(m2 - mn);
#pragma unroll
      for (int d = 0; d < 16; ++d) o[r][d] = o[r][d] * a1 + __shfl_xor(o[r][d], off, 64) * a2;
      s[r] = s[r] * a1 + s2 * a2;
      m[r] = mn;
    }
  }
  // merge the waves through LDS, one wave after the other
  for (int w = 0; w < kWaves; ++w) {
    if (wave == w && slot == 0) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int row = g * R + r;
        if (w == 0) {
#pragma unroll
          for (int d = 0; d < 16; ++d) red_o[row][c * 16 + d] = o[r][d];
          if (c == 0) { red_ms[row][0] = m[r]; red_ms[row][1] = s[r]; }
        } else {
          const float m1 = red_ms[row][0], s1 = red_ms[row][1];
          const float mn = fmaxf(m1, m[r]);
          const float a1 = (m1 == -INFINITY) ? 0.0f : exp2f(m1 - mn);
          const float a2 = (m[r] == -INFINITY) ? 0.0f : exp2f(m[r] - mn);
#pragma unroll
          for (int d = 0; d < 16; ++d)
            red_o[row][c * 16 + d] = red_o[row][c * 16 + d] * a1 + o[r][d] * a2;
          // every lane of the head has read red_ms before lane c == 0 updates it
          __builtin_amdgcn_wave_barrier();
          if (c == 0) { red_ms[row][0] = mn; red_ms[row][1] = s1 * a1 + s[r] * a2; }
        }
      }
    }
    __syncthreads();
  }
  for (int i = threadIdx.x; i < ROWS * (D + 2); i += kThreads) {
    const int row = i / (D + 2), e = i % (D + 2);
    const int gg = row / R, r = row % R;
    if (r >= rows) continue;
    const int h = gg * G + r / T, j = r % T;
    const int64_t orow = (b * Hq + h) * T + j;
    if (e < D) ws_o[(orow * n_split + sp) * D + e] = red_o[row][e];
    else ws_ms[(orow * n_split + sp) * 2 + (e - D)] = red_ms[row][e - D];
  }
}

// ---------------------------------------------------------------------------
// tile variant
// ---------------------------------------------------------------------------
constexpr int kTileKeys = 32;
constexpr int kPad = 4;

template <typename T, int D, int TPR>
__global__ void __launch_bounds__(kThreads)
decode_tile_kernel(const T* __restrict__ q, SegTable st, int n_seg, int64_t n_split, int H,
                   int T_, int Hq, float scale2, int64_t passes, float* __restrict__ ws_ms,
                   float* __restrict__ ws_o) {
  constexpr int RB = kThreads / TPR;
  constexpr int DPT = D / TPR;
  constexpr int V = Elem<T>::kPerVec;
  __shared__ __align__(16) float ks[kTileKeys][D + kPad];
  __shared__ __align__(16) float vs[kTileKeys][D + kPad];

  uint32_t x = blockIdx.x;   // 32-bit: the grid is below 2^32 workgroups
  const int64_t sp = x % static_cast<uint32_t>(n_split); x /= static_cast<uint32_t>(n_split);
  const int64_t pass = x % static_cast<uint32_t>(passes); x /= static_cast<uint32_t>(passes);
  const int g = static_cast<int>(x % static_cast<uint32_t>(H));
  const int64_t b = x / static_cast<uint32_t>(H);
  const int sg = find_seg(st, n_seg, sp);
  const int64_t t_begin = (sp - st.split_begin[sg]) * st.split_len;
  const int64_t t_end = min(st.N[sg], t_begin + st.split_len);
  const int G = Hq / H;
  const int R = G * T_;
  const int r = static_cast<int>(pass) * RB + threadIdx.x / TPR;
  const int p = threadIdx.x % TPR;
  const bool row_ok = r < R;
  const int h = g * G + (row_ok ? r : 0) / T_, j = (row_ok ? r : 0) % T_;

  float qf[DPT], o[DPT];
  if (row_ok) {
    const T* qp = q + ((b * T_ + j) * Hq + h) * D + p * DPT;
#pragma unroll
    for (int d = 0; d < DPT; ++d) qf[d] = Elem<T>::to_f32(qp[d]);
  } else {
#pragma unroll
    for (int d = 0; d < DPT; ++d) qf[d] = 0.0f;
  }
#pragma unroll
  for (int d = 0; d < DPT; ++d) o[d] = 0.0f;
  float m = -INFINITY, s = 0.0f;

  const T* kb = static_cast<const T*>(st.k[sg]) + b * st.stride_b[sg] + static_cast<int64_t>(g) * D;
  const T* vb = static_cast<const T*>(st.v[sg]) + b * st.stride_b[sg] + static_cast<int64_t>(g) * D;
  const int64_t sn = st.stride_n[sg];
  for (int64_t t0 = t_begin; t0 < t_end; t0 += kTileKeys) {
    const int nt = static_cast<int>(min<int64_t>(kTileKeys, t_end - t0));
    __syncthreads();
    for (int e = threadIdx.x; e < nt * (D / V); e += kThreads) {
      const int tt = e / (D / V), cc = e % (D / V);
      float tk[V], tv[V];
      unpack16<T>(*reinterpret_cast<const uint4*>(kb + (t0 + tt) * sn + cc * V), tk);
      unpack16<T>(*reinterpret_cast<const uint4*>(vb + (t0 + tt) * sn + cc * V), tv);
#pragma unroll
      for (int y = 0; y < V; ++y) { ks[tt][cc * V + y] = tk[y]; vs[tt][cc * V + y] = tv[y]; }
    }
    __syncthreads();
    for (int tt = 0; tt < nt; ++tt) {
      float acc = 0.0f;
#pragma unroll
      for (int d = 0; d < DPT; ++d) acc += qf[d] * ks[tt][p * DPT + d];
      const float l2 = group_sum<TPR>(acc) * scale2;
      if (l2 > m) {
        const float alpha = exp2f(m - l2);
        s = s * alpha + 1.0f;
#pragma unroll
        for (int d = 0; d < DPT; ++d) o[d] = o[d] * alpha + vs[tt][p * DPT + d];
        m = l2;
      } else {
        const float pe = exp2f(l2 - m);
        s += pe;
#pragma unroll
        for (int d = 0; d < DPT; ++d) o[d] += pe * vs[tt][p * DPT + d];
      }
    }
  }
  if (row_ok) {
    const int64_t orow = (b * Hq + h) * T_ + j;
#pragma unroll
    for (int d = 0; d < DPT; ++d) ws_o[(orow * n_split + sp) * D + p * DPT + d] = o[d];
    if (p == 0) {
      ws_ms[(orow * n_split + sp) * 2] = m;
      ws_ms[(orow * n_split + sp) * 2 + 1] = s;
    }
  }
}

// One online-softmax step of the first NB of a wave's RBW row blocks over a
// 64-key tile: the steps of attn_softmax (mfma.h) for each row block, with a
// single rescale branch for all of them, so that every exponential and the
// value products after it fall in one basic block that the scheduler can
// interleave.  When the branch is taken, each row's reference moves to its new
// maximum (or stays).
template <int CB, int RBW, int NB>
__device__ __forceinline__ void attn_softmax_rows(const f32x4_t (&sv)[NB][4], float scale2,
                                                  float (&m)[RBW], float (&s)[RBW],
                                                  f32x4_t (&o)[RBW][CB], uint32_t (&pk)[NB][4][2]) {
  static_assert(NB <= RBW, "active row blocks");
  float tm[NB];
  bool grow = false;
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    float tmax = sv[i][0][0];
#pragma unroll
    for (int kb4 = 0; kb4 < 4; ++kb4)
#pragma unroll
      for (int vv = 0; vv < 4; ++vv) tmax = fmaxf(tmax, sv[i][kb4][vv]);
    tm[i] = quad_max(tmax) * scale2;
    grow = grow || tm[i] > m[i] + kAttnLazy;
  }
  if (__any(grow)) {   // uniform: rare once the maxima settle
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const float mn = fmaxf(m[i], tm[i]);
      const float alpha = mn == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m[i] - mn);
      m[i] = mn;
      s[i] *= alpha;
#pragma unroll
      for (int c = 0; c < CB; ++c) o[i][c] *= alpha;
    }
  }
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const float ref = m[i] == -INFINITY ? 0.0f : m[i];
    float ps = s[i];
#pragma unroll
    for (int kb4 = 0; kb4 < 4; ++kb4) {
      float p[4];
#pragma unroll
      for (int vv = 0; vv < 4; ++vv)
        p[vv] = __builtin_amdgcn_exp2f(fmaf(sv[i][kb4][vv], scale2, -ref));
      pk[i][kb4][0] = pack2_bf16(p[0], p[1]);
      pk[i][kb4][1] = pack2_bf16(p[2], p[3]);
      ps = dot2_bf16(pk[i][kb4][0], kBf16Ones, ps);
      ps = dot2_bf16(pk[i][kb4][1], kBf16Ones, ps);
    }
    s[i] = ps;
  }
}

// ---------------------------------------------------------------------------
// matrix-core variant: bf16, >= 16 query rows per kv head
// ---------------------------------------------------------------------------
// Flash decoding with v_mfma_f32_16x16x32_bf16 (lane layout in mfma.h):
//   S^T = K Q^T  (A = 16 keys x 32 dims from the LDS K tile, B = 32 dims x 16
//                 query rows held in registers): lane l gets query row l%16
//                 and keys 4*(l/16) .. +3 of the key block;
//   O^T += V^T P^T  (A = 16 dims x 32 keys of V^T: from a V tile transposed
//                 when staged, or, in the eight-wave plan, from a row-major V
//                 tile through transposing LDS reads; B = the lane's own
//                 probabilities, rounded to bf16): the 32 keys of two key
//                 blocks, in the order the lane holds them.
// The running max, sum and output of a query row all live in the lanes with
// l%16 == row, so rescaling is lane-local (and lazy: attn_softmax_rows);
// the max and the final sum are reduced across the four lane quads.  Waves
// split the query rows, RBW row blocks each; taller blocks run in passes.
template <int D, int RBW, int NW>
__global__ void __launch_bounds__(64 * NW)
decode_mfma_kernel(const bf16_t* __restrict__ q, SegTable st, int n_seg, int64_t n_split, int H,
                   int T_, int Hq, float scale2, int passes, float* __restrict__ ws_ms,
                   float* __restrict__ ws_o) {
  constexpr int TK = kMfmaTileKeys;
  constexpr int KS = D / 32;
  constexpr int KROW = D + kMfmaPad;
  constexpr int VROW = TK + kMfmaPad;   // transposed V: dims x keys (+32 bytes)
  constexpr int CB = D / 16;            // output column blocks
  constexpr int KG = TK / 4;            // groups of 4 keys
  constexpr int NT = 64 * NW;
  constexpr int KV = TK * (D / 8) / NT;    // K vectors per thread and tile
  constexpr int VITEMS = KG * (D / 8);     // V items (4 keys x 8 dims) per tile
  constexpr int VI = (VITEMS + NT - 1) / NT;
  static_assert(KV >= 1 && NT % KG == 0, "tile staging");
  // eight waves, head dim 128: V staged row-major like K and read back
  // transposed (ds_read_b64_tr_b16); otherwise V is transposed when staged
  constexpr bool SPLIT = (NW == 8 && D == 128);
  __shared__ __align__(16) bf16_t kt[TK * KROW];
  __shared__ __align__(16) bf16_t vt[SPLIT ? TK * KROW : D * VROW];

  const int nwaves = NW;
  uint32_t x = blockIdx.x;   // 32-bit: the grid is below 2^32 workgroups
  const int64_t sp = x % static_cast<uint32_t>(n_split); x /= static_cast<uint32_t>(n_split);
  const int pass = static_cast<int>(x % static_cast<uint32_t>(passes)); x /= static_cast<uint32_t>(passes);
  const int g = static_cast<int>(x % static_cast<uint32_t>(H));
  const int64_t b = x / static_cast<uint32_t>(H);
  const int sg = find_seg(st, n_seg, sp);
  const int64_t t_begin = (sp - st.split_begin[sg]) * st.split_len;
  const int64_t t_end = min(st.N[sg], t_begin + st.split_len);
  const int G = Hq / H;
  const int R = G * T_;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15, quad = lane >> 4;
  const bf16_t* kb = static_cast<const bf16_t*>(st.k[sg]) + b * st.stride_b[sg] + static_cast<int64_t>(g) * D;
  const bf16_t* vb = static_cast<const bf16_t*>(st.v[sg]) + b * st.stride_b[sg] + static_cast<int64_t>(g) * D;
  const int64_t sn = st.stride_n[sg];

  // Tile staging: the next tile's K and V rows are in flight (in registers)
  // while this tile computes.  With eight waves and head dim 128 the staging is
  // split by wave: the first four waves load and transpose V (one item of 4
  // keys x 8 dims per thread), the last four load K (4 vectors per thread), so
  // every thread issues the same 4 loads, through a buffer resource that covers
  // rows t0 .. min(t0 + TK, t_end) of its role's cache: rows past the split end
  // read as zero (their logits are masked below, their values weigh 0) and the
  // loads carry no clamp or branch.  Otherwise every thread loads K vectors and
  // the first VITEMS threads V items, rows past the end clamped to the last.
  constexpr int KSV = TK * (D / 8) / (NT / 2);   // K vectors per K-staging thread
  static_assert(!SPLIT || (KSV == 4 && VITEMS == NT / 2), "split staging");
  constexpr int NBUF = SPLIT ? 4 : KV + 4 * VI;
  const bool vwave = SPLIT && __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) < NW / 2;
  const int te = SPLIT ? (vwave ? threadIdx.x : threadIdx.x - NT / 2) : threadIdx.x;
  const int tn = SPLIT ? NT / 2 : NT;              // threads of one staging role
  uint4 bf[NBUF];
  // split: byte offsets of the thread's 4 rows within a tile (row strides are
  // below 2^24 elements, so a tile spans less than 2^31 bytes)
  uint32_t boff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = te / (D / 8) + j * (tn / (D / 8));
    const int ch = te % (D / 8);
    boff[j] = static_cast<uint32_t>((row * sn + ch * 8) * static_cast<int64_t>(sizeof(bf16_t)));
  }
  const bf16_t* sbase = vwave ? vb : kb;
  const int64_t koff = (te / (D / 8)) * sn + (te % (D / 8)) * 8;
  const int64_t kstep = (tn / (D / 8)) * sn;
  auto fetch_k = [&](uint4* kn, int64_t t0) {
    if (t0 + TK <= t_end) {   // uniform
      const bf16_t* kt0 = kb + t0 * sn;
#pragma unroll
      for (int i = 0; i < KV; ++i) {
        const uint4 x = *reinterpret_cast<const uint4*>(kt0 + koff + i * kstep);
        kn[i] = x;
      }
    } else {
#pragma unroll
      for (int i = 0; i < KV; ++i) {
        const int e = te + i * tn;
        const int64_t t = min<int64_t>(t0 + e / (D / 8), t_end - 1);
        const uint4 x = *reinterpret_cast<const uint4*>(kb + t * sn + (e % (D / 8)) * 8);
        kn[i] = x;
      }
    }
  };
  auto fetch_v = [&](uint4* vn, int e, int64_t t0) {   // item e: 4 rows
    if (t0 + TK <= t_end) {   // uniform
      const bf16_t* vt0 = vb + t0 * sn + (e % KG) * 4 * sn + (e / KG) * 8;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint4 y = *reinterpret_cast<const uint4*>(vt0 + j * sn);
        vn[j] = y;
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t t = min<int64_t>(t0 + (e % KG) * 4 + j, t_end - 1);
        const uint4 y = *reinterpret_cast<const uint4*>(vb + t * sn + (e / KG) * 8);
        vn[j] = y;
      }
    }
  };
  auto fetch = [&](int64_t t0) {
    if constexpr (SPLIT) {
      const int64_t rows = max<int64_t>(0, min<int64_t>(TK, t_end - t0));
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<bf16_t*>(sbase + t0 * sn), 0,
          static_cast<int>(rows * sn * static_cast<int64_t>(sizeof(bf16_t))), kBufferDword3);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bf[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, boff[j], 0, 0));
    } else {
      fetch_k(bf, t0);
#pragma unroll
      for (int i = 0; i < VI; ++i)
        if (threadIdx.x + i * NT < VITEMS) fetch_v(bf + KV + 4 * i, threadIdx.x + i * NT, t0);
    }
  };
  // a row-major tile (K, and V in the split plan): item (key, 16-byte chunk)
  auto stage_k = [&](bf16_t* tile, const uint4* kn, int nk) {
#pragma unroll
    for (int i = 0; i < nk; ++i) {
      const int e = te + i * tn;
      const int key = e / (D / 8), ch = e % (D / 8);
      *reinterpret_cast<uint4*>(&tile[key * KROW + ch * 8]) = kn[i];
    }
  };
  // query fragments (B operand: query row col of the row block, 8 dims per k-step)
  // Row block of slot i: a pass fills slot 0 of every wave, then slot 1, and
  // so on, so the padding of a pass's last, partial set of blocks lands in
  // the last slots of the last waves; with two slots, at most one such wave
  // per SIMD (waves w and w + NW / 2 share one).  A wave with at most one
  // block of query rows runs the one-block loop below and skips the
  // padding's products and exponentials.
  uint4 qb[RBW][KS];
  int rb[RBW];
  int nb = 0;                      // row blocks of this wave holding query rows
#pragma unroll
  for (int i = 0; i < RBW; ++i) {
    rb[i] = (pass * RBW + i) * nwaves + wave;
    nb += rb[i] * 16 < R ? 1 : 0;
    const int r = rb[i] * 16 + col;
    if (r < R) {
      const int h = g * G + r / T_, j = r % T_;
      const uint4* qp = reinterpret_cast<const uint4*>(q + ((b * T_ + j) * Hq + h) * D + quad * 8);
#pragma unroll
      for (int s2 = 0; s2 < KS; ++s2) qb[i][s2] = qp[s2 * 4];
    } else {
#pragma unroll
      for (int s2 = 0; s2 < KS; ++s2) qb[i][s2] = make_uint4(0, 0, 0, 0);
    }
  }
  float m[RBW], s[RBW];
  f32x4_t o[RBW][CB];
#pragma unroll
  for (int i = 0; i < RBW; ++i) {
    m[i] = -INFINITY;
    s[i] = 0.0f;
#pragma unroll
    for (int c = 0; c < CB; ++c) o[i][c] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }

  if (SPLIT || t_begin < t_end) fetch(t_begin);
  __builtin_amdgcn_sched_barrier(0);
  // full tiles, then the split's last, partial tile (rows past its end masked)
  auto tile = [&](auto nbc, int64_t t0, bool partial) __attribute__((always_inline)) {
    constexpr int NB = decltype(nbc)::value;   // active row blocks (the first NB slots)
    __syncthreads();
    if constexpr (SPLIT) {
      stage_k(vwave ? vt : kt, bf, KSV);
    } else {
      stage_k(kt, bf, KV);
      // V transposed: item (4 consecutive keys, 8-dim chunk)
#pragma unroll
      for (int i = 0; i < VI; ++i) {
        const int e = threadIdx.x + i * NT;
        if (e < VITEMS)
          stage_vt<VROW>(vt, *reinterpret_cast<const uint4(*)[4]>(bf + KV + 4 * i), e % KG, e / KG);
      }
    }
    __syncthreads();
    if (SPLIT || t0 + TK < t_end) fetch(t0 + TK);

    // S^T blocks: key block outer, so one K fragment serves every row block
    f32x4_t sv[NB][4];
#pragma unroll
    for (int kb4 = 0; kb4 < 4; ++kb4) {
      uint4 ka[KS];
#pragma unroll
      for (int s2 = 0; s2 < KS; ++s2)
        ka[s2] = *reinterpret_cast<const uint4*>(&kt[(kb4 * 16 + col) * KROW + s2 * 32 + quad * 8]);
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        f32x4_t a = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s2 = 0; s2 < KS; ++s2) a = mfma16x16x32(ka[s2], qb[i][s2], a);
        sv[i][kb4] = a;
      }
    }
    if (partial) {
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int kb4 = 0; kb4 < 4; ++kb4)
#pragma unroll
          for (int vv = 0; vv < 4; ++vv)
            if (t0 + kb4 * 16 + quad * 4 + vv >= t_end) sv[i][kb4][vv] = -INFINITY;
    }
    uint32_t pk[NB][4][2];
    attn_softmax_rows<CB, RBW, NB>(sv, scale2, m, s, o, pk);
    // O^T += V^T P^T: one V^T fragment serves every row block
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) {
#pragma unroll
      for (int c = 0; c < CB; ++c) {
        uint4 va;
        if constexpr (SPLIT) va = load_vt_tr<KROW>(vt, c, pr, lane);
        else va = load_vt<VROW>(vt, c, pr, col, quad);
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          const uint4 pb = make_uint4(pk[i][2 * pr][0], pk[i][2 * pr][1], pk[i][2 * pr + 1][0],
                                      pk[i][2 * pr + 1][1]);
          o[i][c] = mfma16x16x32(va, pb, o[i][c]);
        }
      }
    }
  };
  const int64_t t_full = t_begin + max<int64_t>(0, t_end - t_begin) / TK * TK;
  auto run = [&](auto nbc) __attribute__((always_inline)) {
    for (int64_t t0 = t_begin; t0 < t_full; t0 += TK) tile(nbc, t0, false);
    if (t_full < t_end) tile(nbc, t_full, true);
  };
  // every wave passes the same barriers in either loop; a wave with no query
  // rows (a short last pass) runs the one-block loop on zero queries
  if constexpr (RBW == 1) run(std::integral_constant<int, 1>{});
  else if (nb > 1) run(std::integral_constant<int, RBW>{});   // padded slots too, if any
  else run(std::integral_constant<int, 1>{});

  // publish: lane l holds query row rb*16 + l%16, dims c*16 + 4*quad .. +3
#pragma unroll
  for (int i = 0; i < RBW; ++i) {
    float st_sum = s[i];
    st_sum += __shfl_xor(st_sum, 16, 64);
    st_sum += __shfl_xor(st_sum, 32, 64);
    const int r = rb[i] * 16 + col;
    if (r >= R) continue;
    const int h = g * G + r / T_, j = r % T_;
    const int64_t orow = (b * Hq + h) * T_ + j;
    float* wo = ws_o + (orow * n_split + sp) * D;
#pragma unroll
    for (int c = 0; c < CB; ++c)
      *reinterpret_cast<float4*>(wo + c * 16 + quad * 4) =
          make_float4(o[i][c][0], o[i][c][1], o[i][c][2], o[i][c][3]);
    if (quad == 0) {
      ws_ms[(orow * n_split + sp) * 2] = m[i];
      ws_ms[(orow * n_split + sp) * 2 + 1] = st_sum;
    }
  }
}

// ---------------------------------------------------------------------------
// merge of the splits: one block of 256 threads per row
// ---------------------------------------------------------------------------
// The splits are dealt round-robin to NG groups of D / 4 threads; a thread
// reads 16 bytes (4 dims) of each of its splits' partial outputs, so a row's
// partials are all in flight at once.  The groups' maxima, sums and outputs
// meet in LDS.  Partial outputs start at a 16-byte boundary of the workspace.
// A thread's first PF splits (every split of up to PF * NG) are loaded whole
// before the row's maximum is known, so the partials take one trip to memory.
template <int D>
__global__ void __launch_bounds__(256)
decode_merge_kernel(const float* __restrict__ ws_ms, const float* __restrict__ ws_o,
                    int64_t n_split, int T_, int Hq, float* __restrict__ out,
                    float* __restrict__ lse) {
  constexpr int LPS = D / 4;       // threads per split (4 dims each)
  constexpr int NG = 256 / LPS;    // split groups
  constexpr int PF = 4;            // splits per thread held in registers
  __shared__ float gmax[NG], gsum[NG];
  __shared__ float4 gacc[NG][LPS];
  const int64_t row = blockIdx.x;  // (b*Hq + h)*T + j
  const int gi = threadIdx.x / LPS, li = threadIdx.x % LPS;
  const float* ms = ws_ms + row * n_split * 2;   // (m_i, s_i) pairs
  const float4* po = reinterpret_cast<const float4*>(ws_o + row * n_split * D) + li;
  float pm[PF], psum[PF];
  float4 pov[PF];
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < PF; ++j) {
    const int64_t i = gi + j * NG;
    pm[j] = -INFINITY;   // past the last split: weight 0
    psum[j] = 0.0f;
    pov[j] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (i < n_split) {
      pm[j] = ms[2 * i];
      psum[j] = ms[2 * i + 1];
      pov[j] = po[i * (D / 4)];
    }
    m = fmaxf(m, pm[j]);
  }
  for (int64_t i = gi + PF * NG; i < n_split; i += NG) m = fmaxf(m, ms[2 * i]);
  if (li == 0) gmax[gi] = m;
  __syncthreads();
  m = gmax[0];
#pragma unroll
  for (int k = 1; k < NG; ++k) m = fmaxf(m, gmax[k]);
  // a split with no keys (m_i = -inf) weighs 0
  const float ref = m == -INFINITY ? 0.0f : m;
  float s = 0.0f;
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
  for (int j = 0; j < PF; ++j) {
    const float a = __builtin_amdgcn_exp2f(pm[j] - ref);
    s = fmaf(psum[j], a, s);
    acc.x = fmaf(pov[j].x, a, acc.x);
    acc.y = fmaf(pov[j].y, a, acc.y);
    acc.z = fmaf(pov[j].z, a, acc.z);
    acc.w = fmaf(pov[j].w, a, acc.w);
  }
#pragma unroll 4
  for (int64_t i = gi + PF * NG; i < n_split; i += NG) {
    const float a = __builtin_amdgcn_exp2f(ms[2 * i] - ref);
    const float4 p = po[i * (D / 4)];
    s = fmaf(ms[2 * i + 1], a, s);
    acc.x = fmaf(p.x, a, acc.x);
    acc.y = fmaf(p.y, a, acc.y);
    acc.z = fmaf(p.z, a, acc.z);
    acc.w = fmaf(p.w, a, acc.w);
  }
  gacc[gi][li] = acc;
  if (li == 0) gsum[gi] = s;
  __syncthreads();
  if (gi != 0) return;
  float4 t = gacc[0][li];
  float st = gsum[0];
#pragma unroll
  for (int k = 1; k < NG; ++k) {
    const float4 u = gacc[k][li];
    t.x += u.x; t.y += u.y; t.z += u.z; t.w += u.w;
    st += gsum[k];
  }
  const int64_t j = row % T_;
  const int64_t h = (row / T_) % Hq;
  const int64_t b = row / (static_cast<int64_t>(T_) * Hq);
  *reinterpret_cast<float4*>(out + ((b * T_ + j) * Hq + h) * D + li * 4) =
      make_float4(t.x / st, t.y / st, t.z / st, t.w / st);
  if (lse != nullptr && li == 0) lse[row] = (m + log2f(st)) * kLn2;
}

template <int D, int H, int R>
void launch_stream(const void* q, const SegTable& st, int n_seg, int64_t n_split, int64_t B,
                   int64_t T, int64_t Hq, float scale2, float* ms, float* o, hipStream_t s) {
  // 8 rows in flight per slot measured ~3.5% faster than 4 on the serving
  // shape (<= 4 query rows per kv head); 8 query rows keep 4
  hipLaunchKernelGGL((decode_stream_kernel<D, H, R, (R >= 8 ? 4 : 8)>), dim3(static_cast<unsigned>(B * n_split)),
                     dim3(kThreads), 0, s, static_cast<const bf16_t*>(q), st, n_seg, n_split,
                     static_cast<int>(T), static_cast<int>(Hq), static_cast<int>((Hq / H) * T),
                     scale2, ms, o);
}

template <typename T, int D, int TPR>
void launch_tile(const void* q, const SegTable& st, int n_seg, int64_t n_split, int64_t B,
                 int64_t H, int64_t T_, int64_t Hq, float scale2, float* ms, float* o,
                 hipStream_t s) {
  constexpr int RB = kThreads / TPR;
  const int64_t R = (Hq / H) * T_;
  const int64_t passes = (R + RB - 1) / RB;
  hipLaunchKernelGGL((decode_tile_kernel<T, D, TPR>),
                     dim3(static_cast<unsigned>(B * H * passes * n_split)), dim3(kThreads), 0, s,
                     static_cast<const T*>(q), st, n_seg, n_split, static_cast<int>(H),
                     static_cast<int>(T_), static_cast<int>(Hq), scale2, passes, ms, o);
}

template <typename T, int D>
void dispatch_tile(const void* q, const SegTable& st, int n_seg, int64_t n_split, int64_t B,
                   int64_t H, int64_t T_, int64_t Hq, float scale2, float* ms, float* o,
                   hipStream_t s) {
  const int64_t R = (Hq / H) * T_;
  if (R >= 64) launch_tile<T, D, 4>(q, st, n_seg, n_split, B, H, T_, Hq, scale2, ms, o, s);
  else if (R >= 32) launch_tile<T, D, 8>(q, st, n_seg, n_split, B, H, T_, Hq, scale2, ms, o, s);
  else if (R >= 16) launch_tile<T, D, 16>(q, st, n_seg, n_split, B, H, T_, Hq, scale2, ms, o, s);
  else launch_tile<T, D, 32>(q, st, n_seg, n_split, B, H, T_, Hq, scale2, ms, o, s);
}

}  // namespace

bool decode_stream_ok(int dtype, int64_t H, int64_t D, int64_t rows_per_kv) {
  return dtype == KVSEL_BF16 && D == 128 && rows_per_kv >= 1 && rows_per_kv <= 8 &&
         (H == 1 || H == 2 || H == 4 || H == 8);
}

bool decode_uses_stream(int dtype, int64_t H, int64_t D, int64_t rows_per_kv, bool gathered) {
  // the streaming kernel is the only one that gathers on the fly (up to 8
  // rows); a plain pass with 5 or more rows runs faster on the matrix cores
  // (one 16-row block, padded), which read K and V through LDS tiles
  return decode_stream_ok(dtype, H, D, rows_per_kv) && (gathered || rows_per_kv < kDecodeMfmaRows);
}

namespace {
// Matrix-core plan for R query rows per kv head.  Tall query blocks (12 row
// blocks or more): eight waves of two row blocks, so every staged K and V
// fragment feeds two products; 256 rows a pass.  Otherwise one row block per
// wave: two waves for up to two row blocks, else four.
struct DecodeMfmaPlan {
  int rbw, nwaves, passes;
};
DecodeMfmaPlan decode_mfma_plan(int64_t R) {
  const int64_t rbs = (R + 15) / 16;
  const int rbw = rbs >= 12 ? 2 : 1;
  const int nwaves = rbs >= 12 ? 8 : rbs <= 2 ? 2 : 4;
  return {rbw, nwaves, static_cast<int>((rbs + rbw * nwaves - 1) / (rbw * nwaves))};
}
// waves a matrix-core decode launch should hold at least (8 per CU)
constexpr int64_t kDecodeFillWaves = 2048;
}  // namespace

int64_t decode_split_len(int dtype, int64_t H, int64_t D, int64_t rows_per_kv, bool gathered,
                         int64_t B, int64_t n_keys) {
  if (decode_uses_stream(dtype, H, D, rows_per_kv, gathered)) return kDecodeSplit;
  if (!(dtype == KVSEL_BF16 && rows_per_kv >= kDecodeMfmaRows)) return kDecodeSplit;
  // the matrix-core variant: splits of 1024 keys leave fewer (m, s, o)
  // partials to write and merge; they are halved, down to 256, while the
  // launch would hold fewer than kDecodeFillWaves waves
  const DecodeMfmaPlan p = decode_mfma_plan(rows_per_kv);
  int64_t len = 1024;
  while (len > 256 && B * H * p.passes * ((n_keys + len - 1) / len) * p.nwaves < kDecodeFillWaves)
    len /= 2;
  return len;
}

int launch_decode(const void* q, int64_t T, int64_t Hq, float scale, const DecodeSeg* segs,
                  int n_seg, int64_t B, int64_t H, int64_t D, int dtype, int64_t n_split,
                  float* out, float* lse, float* ws_ms, float* ws_o, hipStream_t s,
                  const DecodeGather* gather) {
  SegTable st{};
  st.gather_seg = -1;
  int64_t n_keys = 0;
  for (int i = 0; i < n_seg; ++i) n_keys += segs[i].N;
  st.split_len = decode_split_len(dtype, H, D, (Hq / H) * T, gather != nullptr, B, n_keys);
  if (gather != nullptr) {
    // only the streaming variant gathers on the fly
    if (!decode_stream_ok(dtype, H, D, (Hq / H) * T)) {
      set_error("kvsel: fused gather is not available for this shape");
      return KVSEL_ERR_UNSUPPORTED;
    }
    st.gather_seg = gather->seg;
    st.idx = gather->idx;
    st.unit_len = gather->unit_len;
    st.n_kept = gather->n_kept;
    st.idx_group = gather->idx_group;
    st.n_units = gather->n_units;
    st.k_dst = gather->k_dst;
    st.v_dst = gather->v_dst;
  }
  for (int i = 0; i < n_seg; ++i) {
    st.k[i] = segs[i].k;
    st.v[i] = segs[i].v;
    st.N[i] = segs[i].N;
    st.stride_b[i] = segs[i].stride_b;
    st.stride_n[i] = segs[i].stride_n;
    st.split_begin[i] = segs[i].split_begin;
  }
  st.split_begin[n_seg] = n_split;
  const float scale2 = scale * kLog2e;
  const int64_t R = (Hq / H) * T;
  bool done = false;
  if (decode_uses_stream(dtype, H, D, R, gather != nullptr)) {
    // rows per kv head padded to 1, 2, 4 or 8
    const int64_t RP = R <= 1 ? 1 : R <= 2 ? 2 : R <= 4 ? 4 : 8;
#define KVSEL_DS(H_, R_) \
  if (!done && H == H_ && RP == R_) { launch_stream<128, H_, R_>(q, st, n_seg, n_split, B, T, Hq, scale2, ws_ms, ws_o, s); done = true; }
    KVSEL_DS(8, 1) KVSEL_DS(8, 2) KVSEL_DS(8, 4) KVSEL_DS(8, 8)
    KVSEL_DS(4, 1) KVSEL_DS(4, 2) KVSEL_DS(4, 4) KVSEL_DS(4, 8)
    KVSEL_DS(2, 1) KVSEL_DS(2, 2) KVSEL_DS(2, 4) KVSEL_DS(2, 8)
    KVSEL_DS(1, 1) KVSEL_DS(1, 2) KVSEL_DS(1, 4) KVSEL_DS(1, 8)
#undef KVSEL_DS
  }
  if (!done && dtype == KVSEL_BF16 && R >= kDecodeMfmaRows) {
    const DecodeMfmaPlan p = decode_mfma_plan(R);
    const int rbw = p.rbw, nwaves = p.nwaves, passes = p.passes;
    const dim3 grid(static_cast<unsigned>(B * H * passes * n_split)), block(64 * nwaves);
#define KVSEL_DM(D_, RBW_, NW_) \
    hipLaunchKernelGGL((decode_mfma_kernel<D_, RBW_, NW_>), grid, block, 0, s, static_cast<const bf16_t*>(q), st, \
                       n_seg, n_split, static_cast<int>(H), static_cast<int>(T), static_cast<int>(Hq), scale2, \
                       passes, ws_ms, ws_o)
    if (D == 128) {
      if (rbw == 2) KVSEL_DM(128, 2, 8); else if (nwaves == 2) KVSEL_DM(128, 1, 2); else KVSEL_DM(128, 1, 4);
    } else {
      if (rbw == 2) KVSEL_DM(64, 2, 8); else if (nwaves == 2) KVSEL_DM(64, 1, 2); else KVSEL_DM(64, 1, 4);
    }
#undef KVSEL_DM
    done = true;
  }
  if (!done) {
    if (dtype == KVSEL_BF16) {
      if (D == 128) dispatch_tile<bf16_t, 128>(q, st, n_seg, n_split, B, H, T, Hq, scale2, ws_ms, ws_o, s);
      else dispatch_tile<bf16_t, 64>(q, st, n_seg, n_split, B, H, T, Hq, scale2, ws_ms, ws_o, s);
    } else {
      if (D == 128) dispatch_tile<float, 128>(q, st, n_seg, n_split, B, H, T, Hq, scale2, ws_ms, ws_o, s);
      else dispatch_tile<float, 64>(q, st, n_seg, n_split, B, H, T, Hq, scale2, ws_ms, ws_o, s);
    }
  }
  int rc = check_launch("kvsel_decode_attn");
  if (rc != KVSEL_OK) return rc;
  if (D == 128)
    hipLaunchKernelGGL(decode_merge_kernel<128>, dim3(static_cast<unsigned>(B * Hq * T)), dim3(256), 0, s,
                       ws_ms, ws_o, n_split, static_cast<int>(T), static_cast<int>(Hq), out, lse);
  else
    hipLaunchKernelGGL(decode_merge_kernel<64>, dim3(static_cast<unsigned>(B * Hq * T)), dim3(256), 0, s,
                       ws_ms, ws_o, n_split, static_cast<int>(T), static_cast<int>(Hq), out, lse);
  return check_launch("kvsel_decode_attn (merge)");
}

}  // namespace kvsel
