// Token-path aggregation on the matrix cores (bf16 caches with >= 16 query
// rows per kv head):
//   per_token[b][t] = sum_h sum_j alpha[b,h,j,t]            (mass)
//   per_token[b][t] = sum_h sum_j alpha[b,h,j,t] * ||v[b,t,kv(h)]||_2   (vnorm)
// with alpha = exp(l - row_max) / row_sum (ACRE §2.4 Eq. 15 as a sum;
// InfoFlow §4.2, s_j = sum_i A_ij with A_ij read as attention weight times
// value norm).
//
// A workgroup owns a range of cached rows of one instance and loops over the kv
// heads (and row passes for very tall query blocks); for small caches the
// (kv head, row pass) items are split over groups of workgroups, each group
// writing its own per-token partials.  For every 64-key tile of
// K staged in LDS it recomputes the logits with v_mfma_f32_16x16x32_bf16 (the
// same operand layout as score_mfma.hip), forms alpha with one exp per logit,
// sums it over the lane's rows, over the four lane quads (shuffles) and over
// the waves that split the rows (LDS), then scales by the value norm of the
// head.  The per-token totals stay in LDS across heads and are written once:
// a fixed summation order, no atomics.
#include <algorithm>

#include "common.h"
#include "internal.h"
#include "mfma.h"

namespace kvsel {
namespace {

constexpr int kTileKeys = kMfmaTileKeys;
constexpr int kPad = kMfmaPad;
constexpr int kMaxRange = 1024;   // cached rows per workgroup
constexpr int kSmallRange = 256;  // cached rows per workgroup for small caches
constexpr int kTargetBlocks = 512;

template <int D, int RBW, int NWR, int NW, bool VNORM>
__global__ void __launch_bounds__(64 * NW)
agg_mfma_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                const bf16_t* __restrict__ v, int64_t N, int H, int64_t stride_b,
                int64_t stride_n, int T, int Hq, float scale2, const float* __restrict__ row_max,
                const float* __restrict__ row_sum, int64_t range, int64_t ranges, int passes,
                int64_t parts, int hp_per_block, int64_t nb, float* __restrict__ per_token) {
  constexpr int KS = D / 32;
  constexpr int KROW = D + kPad;
  constexpr int NT = 64 * NW;
  static_assert(!VNORM || NW == 4, "the value norms are staged by 4 lanes per key of 256 threads");
  constexpr int NWK = NW / NWR;
  constexpr int KBW = (kTileKeys / 16) / NWK;
  constexpr int VPT = kTileKeys * D / 8 / NT;
  __shared__ __align__(16) bf16_t kt[kTileKeys * KROW];
  __shared__ float vn[kTileKeys];
  __shared__ float part[NW][kTileKeys];
  __shared__ float tot[kMaxRange];

  uint32_t x = blockIdx.x;   // 32-bit: the grid is below 2^32 workgroups
  const int64_t grp = x % static_cast<uint32_t>(parts); x /= static_cast<uint32_t>(parts);
  const int64_t b = x / static_cast<uint32_t>(ranges);
  const int64_t t_begin = static_cast<int64_t>(x % static_cast<uint32_t>(ranges)) * range;
  const int64_t t_end = min(N, t_begin + range);
  const int G = Hq / H;
  const int R = G * T;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wr = wave % NWR, wk = wave / NWR;
  const int col = lane & 15, quad = lane >> 4;
  // this group's (kv head, row pass) items: hp = g * passes + pass
  const int hp0 = static_cast<int>(grp) * hp_per_block;
  const int hp1 = min(H * passes, hp0 + hp_per_block);

  for (int i = threadIdx.x; i < range; i += NT) tot[i] = 0.0f;

  // items (hp, tile) in order; the next item's K slice (and V slice for the
  // norms) is in flight during the math.  The fetch cursor advances by one
  // tile with an add and a compare.
  constexpr int VV = D / 32;  // 16-byte vectors of V per thread (4 lanes per key)
  const int64_t n_tiles = (t_end - t_begin + kTileKeys - 1) / kTileKeys;
  uint4 kn[VPT], vr[VNORM ? VV : 1];
  int f_hp = hp0;
  int64_t f_ti = 0;
  auto fetch = [&]() {
    const int g = f_hp / passes;
    const int64_t t0 = t_begin + f_ti * kTileKeys;
    const bf16_t* kb = k + b * stride_b + static_cast<int64_t>(g) * D;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int e = threadIdx.x + i * NT;
      const int key = e / (D / 8), ch = e % (D / 8);
      kn[i] = (t0 + key < t_end) ? *reinterpret_cast<const uint4*>(kb + (t0 + key) * stride_n + ch * 8)
                                 : make_uint4(0, 0, 0, 0);
    }
    if constexpr (VNORM) {
      const bf16_t* vb = v + b * stride_b + static_cast<int64_t>(g) * D;
      const int key = threadIdx.x >> 2, qd = threadIdx.x & 3;
#pragma unroll
      for (int i = 0; i < VV; ++i)
        vr[i] = (t0 + key < t_end)
                    ? *reinterpret_cast<const uint4*>(vb + (t0 + key) * stride_n + qd * (D / 4) + i * 8)
                    : make_uint4(0, 0, 0, 0);
    }
    if (++f_ti == n_tiles) {
      f_ti = 0;
      ++f_hp;
    }
  };

  uint4 qa[RBW][KS];
  float m2[RBW][4], iz[RBW][4];
  if (hp0 < hp1 && n_tiles > 0) fetch();
  for (int hp = hp0; hp < hp1; ++hp) {
    const int g = hp / passes, pass = hp % passes;
    // query fragments and row statistics of this wave's row blocks; rows past
    // R get zero weight
#pragma unroll
    for (int i = 0; i < RBW; ++i) {
      const int rb = pass * NWR * RBW + wr + i * NWR;
      const int r = rb * 16 + col;
      if (r < R) {
        const int h = g * G + r / T, j = r % T;
        const uint4* qp = reinterpret_cast<const uint4*>(q + ((b * T + j) * Hq + h) * D + quad * 8);
#pragma unroll
        for (int s2 = 0; s2 < KS; ++s2) qa[i][s2] = qp[s2 * 4];
      } else {
#pragma unroll
        for (int s2 = 0; s2 < KS; ++s2) qa[i][s2] = make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int vv = 0; vv < 4; ++vv) {
        const int rr = rb * 16 + quad * 4 + vv;
        if (rr < R) {
          const int h = g * G + rr / T, j = rr % T;
          const int64_t row = (b * Hq + h) * T + j;
          m2[i][vv] = row_max[row] * kLog2e;
          iz[i][vv] = 1.0f / row_sum[row];
        } else {
          m2[i][vv] = 0.0f;
          iz[i][vv] = 0.0f;
        }
      }
    }
    for (int64_t ti = 0; ti < n_tiles; ++ti) {
      const int64_t t0 = t_begin + ti * kTileKeys;
      __syncthreads();  // previous tile's kt / vn / part fully used
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        const int e = threadIdx.x + i * NT;
        const int key = e / (D / 8), ch = e % (D / 8);
        *reinterpret_cast<uint4*>(&kt[key * KROW + ch * 8]) = kn[i];
      }
      if constexpr (VNORM) {
        // squares summed with the packed bf16 dot, two elements an
        // instruction with no unpacking (a bf16 square is exact in fp32)
        float ss = 0.0f, st = 0.0f;
#pragma unroll
        for (int i = 0; i < VV; ++i) {
          ss = dot2_bf16(vr[i].x, vr[i].x, ss);
          st = dot2_bf16(vr[i].y, vr[i].y, st);
          ss = dot2_bf16(vr[i].z, vr[i].z, ss);
          st = dot2_bf16(vr[i].w, vr[i].w, st);
        }
        ss = group_sum<4>(ss + st);
        if ((threadIdx.x & 3) == 0) vn[threadIdx.x >> 2] = sqrtf(ss);
      }
      __syncthreads();
      if (f_hp < hp1) fetch();

      float c[KBW];
#pragma unroll
      for (int jb = 0; jb < KBW; ++jb) {
        const int key = (wk + jb * NWK) * 16 + col;
        uint4 bk[KS];
#pragma unroll
        for (int st = 0; st < KS; ++st)
          bk[st] = *reinterpret_cast<const uint4*>(&kt[key * KROW + st * 32 + quad * 8]);
        float sum = 0.0f;
#pragma unroll
        for (int i = 0; i < RBW; ++i) {
          f32x4_t a = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int st = 0; st < KS; ++st) a = mfma16x16x32(qa[i][st], bk[st], a);
#pragma unroll
          for (int vv = 0; vv < 4; ++vv)
            sum = fmaf(__builtin_amdgcn_exp2f(fmaf(a[vv], scale2, -m2[i][vv])), iz[i][vv], sum);
        }
        sum += __shfl_xor(sum, 16, 64);
        sum += __shfl_xor(sum, 32, 64);
        c[jb] = sum;
      }
      if (quad == 0) {
#pragma unroll
        for (int jb = 0; jb < KBW; ++jb) part[wave][(wk + jb * NWK) * 16 + col] = c[jb];
      }
      __syncthreads();
      if (threadIdx.x < kTileKeys) {
        const int key = threadIdx.x;
        const int owner = (key / 16) % NWK;  // the waves (wr, owner) computed this key
        float s2 = 0.0f;
#pragma unroll
        for (int w = 0; w < NWR; ++w) s2 += part[w + owner * NWR][key];
        if (VNORM) s2 *= vn[key];
        if (t0 + key < t_end) tot[t0 - t_begin + key] += s2;
      }
    }
  }
  __syncthreads();
  float* out = per_token + (grp * nb + b) * N;   // this group's partials
  for (int i = threadIdx.x; i < t_end - t_begin; i += NT) out[t_begin + i] = tot[i];
}

// Workgroup plan: cached rows per workgroup, and how the (kv head, row pass)
// items split over groups.  Large caches: one group, ranges sized to fill the
// chip.  Small caches (B * N < kAggSplitRows): ranges of kSmallRange rows and
// up to kAggMaxParts groups, so each workgroup keeps its query fragments for
// several tiles instead of reloading them for every tile; about two
// workgroups per CU, which the eight-wave plan's registers allow.
struct AggPlan {
  int64_t range, ranges, parts;
  int hp_per_block, passes, rbw, nwr, nw;
};

AggPlan agg_plan(const kvsel_cache& kc, int64_t rows_per_kv, bool vnorm) {
  const MfmaRowPlan p = mfma_row_plan(rows_per_kv);
  AggPlan a{};
  a.passes = p.passes;
  a.rbw = p.rbw;
  a.nwr = p.nwr;
  a.nw = 4;
  if (!vnorm && kc.D == 128 && p.rbw == 4) {
    // tall query blocks: eight waves of two row blocks (half the registers
    // per wave, two waves per SIMD), 16 row blocks a pass as with four waves
    // of four, so the passes and the partials are the same
    a.rbw = 2;
    a.nwr = 8;
    a.nw = 8;
  }
  const int64_t hp_total = kc.H * p.passes;
  if (kc.B * kc.N < kAggSplitRows) {
    a.range = std::min<int64_t>(kSmallRange, (kc.N + kTileKeys - 1) / kTileKeys * kTileKeys);
    a.ranges = (kc.N + a.range - 1) / a.range;
    int64_t want = (kTargetBlocks + kc.B * a.ranges - 1) / (kc.B * a.ranges);
    want = std::max<int64_t>(1, std::min<int64_t>(want, std::min<int64_t>(kAggMaxParts, hp_total)));
    a.hp_per_block = static_cast<int>((hp_total + want - 1) / want);
    a.parts = (hp_total + a.hp_per_block - 1) / a.hp_per_block;
  } else {
    int64_t range = (kc.B * kc.N / 1024) / kTileKeys * kTileKeys;
    a.range = range < kTileKeys ? kTileKeys : (range > kMaxRange ? kMaxRange : range);
    a.ranges = (kc.N + a.range - 1) / a.range;
    a.hp_per_block = static_cast<int>(hp_total);
    a.parts = 1;
  }
  return a;
}

template <int D, int RBW, int NWR, int NW>
void launch(const void* q, int64_t T, int64_t Hq, const void* k, const void* v,
            const kvsel_cache& kc, float scale2, const float* rm, const float* rs, int vnorm,
            const AggPlan& a, float* per_token, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(kc.B * a.ranges * a.parts));
#define KVSEL_AM(VN)                                                                         \
  hipLaunchKernelGGL((agg_mfma_kernel<D, RBW, NWR, NW, VN>), grid, dim3(64 * NW), 0, s,       \
                     static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k),            \
                     static_cast<const bf16_t*>(v), kc.N, static_cast<int>(kc.H), kc.stride_b, \
                     kc.stride_n, static_cast<int>(T), static_cast<int>(Hq), scale2, rm, rs,   \
                     a.range, a.ranges, a.passes, a.parts, a.hp_per_block, kc.B, per_token)
  if constexpr (NW == 4) {
    if (vnorm) KVSEL_AM(true); else KVSEL_AM(false);
  } else {
    KVSEL_AM(false);
  }
#undef KVSEL_AM
}

template <int D>
void dispatch(const void* q, int64_t T, int64_t Hq, const void* k, const void* v,
              const kvsel_cache& kc, float scale2, const float* rm, const float* rs, int vnorm,
              float* per_token, hipStream_t s) {
  const AggPlan a = agg_plan(kc, (Hq / kc.H) * T, vnorm != 0);
#define KVSEL_AD(RBW, NWR, NW) \
  if (a.rbw == RBW && a.nwr == NWR && a.nw == NW) \
    return launch<D, RBW, NWR, NW>(q, T, Hq, k, v, kc, scale2, rm, rs, vnorm, a, per_token, s);
  KVSEL_AD(1, 1, 4) KVSEL_AD(1, 2, 4) KVSEL_AD(1, 4, 4) KVSEL_AD(2, 4, 4) KVSEL_AD(4, 4, 4)
  if constexpr (D == 128) { KVSEL_AD(2, 8, 8) }
#undef KVSEL_AD
}

}  // namespace

int64_t aggregate_mfma_parts(const kvsel_cache& kc, int64_t rows_per_kv) {
  // the same for either signal: both plans cover 16 row blocks a pass
  return agg_plan(kc, rows_per_kv, true).parts;
}

bool aggregate_mfma_ok(int dtype, int64_t rows_per_kv) {
  return dtype == KVSEL_BF16 && rows_per_kv >= 16;
}

void launch_aggregate_mfma(const void* q, int64_t T, int64_t Hq, const void* k, const void* v,
                           const kvsel_cache& kc, float scale2, const float* row_max,
                           const float* row_sum, int vnorm, float* per_token, hipStream_t s) {
  if (kc.D == 128)
    dispatch<128>(q, T, Hq, k, v, kc, scale2, row_max, row_sum, vnorm, per_token, s);
  else
    dispatch<64>(q, T, Hq, k, v, kc, scale2, row_max, row_sum, vnorm, per_token, s);
}

}  // namespace kvsel
