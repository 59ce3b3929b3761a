// Matrix-core helpers shared by the bf16 MFMA kernels (gfx950).
//
// v_mfma_f32_16x16x32_bf16, lane l of a wave (checked on MI355X):
//   A (16 x 32): row l % 16, k = 8 * (l / 16) + e, e = 0..7
//   B (32 x 16): column l % 16, same k
//   D (16 x 16): column l % 16, rows 4 * (l / 16) + v, v = 0..3
#pragma once

#include "common.h"
#include "internal.h"

namespace kvsel {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

__device__ __forceinline__ f32x4_t mfma16x16x32(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// Padding of a staged row of an LDS tile (keys of the K tile, dims of the
// transposed V tile): 32 bytes, so that the row stride is 8 dwords past a
// multiple of 16.  Measured on gfx950 for the 16-byte fragment reads of these
// kernels: strides of 68, 76, 36 or 44 dwords conflict (up to 44% of the LDS
// cycles), 72 and 40 do not.
constexpr int kMfmaPad = 16;

// Row blocks of 16 query rows: how the four waves of a workgroup share them.
// NWR waves split the row blocks (RBW per wave), 4 / NWR split the key blocks.
struct MfmaRowPlan {
  int rbw;      // row blocks per wave: 1, 2 or 4
  int nwr;      // waves across row blocks: 1, 2 or 4
  int passes;   // row passes (rows beyond 4 * 4 * 16 = 256)
};
inline MfmaRowPlan mfma_row_plan(int64_t rows) {
  const int64_t rb = (rows + 15) / 16;
  if (rb == 1) return {1, 1, 1};
  if (rb <= 2) return {1, 2, 1};
  if (rb <= 4) return {1, 4, 1};
  if (rb <= 8) return {2, 4, 1};
  return {4, 4, static_cast<int>((rb + 15) / 16)};
}

// ---------------------------------------------------------------------------
// Pieces of the attention kernels (decode and index-based causal attention):
//   S^T = K Q^T   A = 16 keys x 32 dims of the LDS K tile, B = 32 dims x 16
//                 query rows in registers: lane l gets query row l % 16 and
//                 keys 4 * (l / 16) + v of each 16-key block;
//   O^T += V^T P^T  A = 16 dims x 32 keys of the transposed LDS V tile, B = the
//                 lane's own probabilities as bf16, in the order it holds them.
// ---------------------------------------------------------------------------

// The running maximum, the reference of the probabilities, moves only when a
// row's maximum grows by more than 2^kAttnLazy; until then every p <= 2^8.
// Numerator and denominator share the reference, so the result is unchanged.
constexpr float kAttnLazy = 8.0f;
constexpr uint32_t kBf16Ones = 0x3F803F80u;   // two bf16 ones

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_hw_t, a),
                                         __builtin_bit_cast(bf16x2_hw_t, b), c, false);
}

// Maximum over the four lanes of a row (l, l ^ 16, l ^ 32, l ^ 48).  Each swap
// with itself leaves one lane of every pair in each result, so the max of the
// two results is the pair's max, without the LDS crossbar.
__device__ __forceinline__ float quad_max(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Column of key t (0..63) in the transposed V tile.  Lane quad q of the value
// product reads, for 32-key half pr, the keys 4q..4q+3 of its two 16-key
// blocks; they sit side by side, so one 16-byte read fetches them.
__device__ __forceinline__ int vt_col(int t) {
  return (t >> 5) * 32 + ((t >> 2) & 3) * 8 + ((t >> 4) & 1) * 4 + (t & 3);
}

// Writes keys 4 kg .. 4 kg + 3 (rows[0..3]) x dims 8 ch .. 8 ch + 7 of V into the
// transposed tile vt (D rows of VROW elements): eight runs of four keys.
template <int VROW>
__device__ __forceinline__ void stage_vt(bf16_t* vt, const uint4 (&rows)[4], int kg, int ch) {
  const int vc = vt_col(kg * 4);
  uint32_t w[4][4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    w[j][0] = rows[j].x; w[j][1] = rows[j].y; w[j][2] = rows[j].z; w[j][3] = rows[j].w;
  }
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    // dims 8 ch + 2p (low halves) and 8 ch + 2p + 1 (high halves)
    const uint2 lo = make_uint2((w[0][p] & 0xffffu) | (w[1][p] << 16),
                                (w[2][p] & 0xffffu) | (w[3][p] << 16));
    const uint2 hi = make_uint2((w[0][p] >> 16) | (w[1][p] & 0xffff0000u),
                                (w[2][p] >> 16) | (w[3][p] & 0xffff0000u));
    *reinterpret_cast<uint2*>(&vt[(ch * 8 + 2 * p) * VROW + vc]) = lo;
    *reinterpret_cast<uint2*>(&vt[(ch * 8 + 2 * p + 1) * VROW + vc]) = hi;
  }
}

// A fragment of V^T: dims 16 c + (l % 16), the lane quad's keys of 32-key half pr.
template <int VROW>
__device__ __forceinline__ uint4 load_vt(const bf16_t* vt, int c, int pr, int col, int quad) {
  return *reinterpret_cast<const uint4*>(&vt[(c * 16 + col) * VROW + pr * 32 + quad * 8]);
}

typedef short i16x4_t __attribute__((ext_vector_type(4)));

// A fragment of V^T (dims 16 c + (l % 16), the lane quad's keys of 32-key half
// pr, in the order of the probabilities: keys 32 pr + 4 q + 0..3, then
// 32 pr + 16 + 4 q + 0..3) from a row-major V tile (rows of KROW elements),
// with two transposing LDS reads.  ds_read_b64_tr_b16 (gfx950, checked on
// MI355X): in each group of 16 lanes, lane i receives element i % 4 of the
// 4 elements that lanes i / 4 + 4 k (k = 0..3) point at.  So lane j of the
// group points at 4 dims 4 (j % 4) of key j / 4, and lane i gets dim i of 4
// consecutive keys.
template <int KROW>
__device__ __forceinline__ uint4 load_vt_tr(const bf16_t* vt, int c, int pr, int lane) {
  const int q = lane >> 4, j = lane & 15;
  const bf16_t* p = vt + (32 * pr + 4 * q + (j >> 2)) * KROW + c * 16 + 4 * (j & 3);
  typedef __attribute__((address_space(3))) i16x4_t* lds_v4;
  const i16x4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4)(p));
  const i16x4_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4)(p + 16 * KROW));
  const uint2 ua = __builtin_bit_cast(uint2, a), ub = __builtin_bit_cast(uint2, b);
  return make_uint4(ua.x, ua.y, ub.x, ub.y);
}

// One online-softmax step of a row block over a 64-key tile.  sv holds the
// lane's logits (keys 16 kb4 + 4 (l / 16) + v; -inf where masked); m, s and o
// are the row's reference, sum and output accumulators.  The probabilities come
// back as bf16 pairs for the value product, and the sum adds those same
// rounded values.  A row with nothing seen yet keeps m = -inf and p = 0.
template <int CB>
__device__ __forceinline__ void attn_softmax(const f32x4_t (&sv)[4], float scale2, float& m,
                                             float& s, f32x4_t (&o)[CB], uint32_t (&pk)[4][2]) {
  float tmax = sv[0][0];
#pragma unroll
  for (int kb4 = 0; kb4 < 4; ++kb4)
#pragma unroll
    for (int vv = 0; vv < 4; ++vv) tmax = fmaxf(tmax, sv[kb4][vv]);
  const float tm = quad_max(tmax) * scale2;
  if (__any(tm > m + kAttnLazy)) {   // uniform: rare once the maximum settles
    const float mn = fmaxf(m, tm);
    const float alpha = mn == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m - mn);
    m = mn;
    s *= alpha;
#pragma unroll
    for (int c = 0; c < CB; ++c) o[c] *= alpha;
  }
  const float ref = m == -INFINITY ? 0.0f : m;
  float ps = s;
#pragma unroll
  for (int kb4 = 0; kb4 < 4; ++kb4) {
    float p[4];
#pragma unroll
    for (int vv = 0; vv < 4; ++vv) p[vv] = __builtin_amdgcn_exp2f(fmaf(sv[kb4][vv], scale2, -ref));
    pk[kb4][0] = pack2_bf16(p[0], p[1]);
    pk[kb4][1] = pack2_bf16(p[2], p[3]);
    ps = dot2_bf16(pk[kb4][0], kBf16Ones, ps);
    ps = dot2_bf16(pk[kb4][1], kBf16Ones, ps);
  }
  s = ps;
}

}  // namespace kvsel
