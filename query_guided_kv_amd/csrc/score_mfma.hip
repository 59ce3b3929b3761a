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

#include <type_traits>

namespace kvsel {
namespace {

constexpr int kTileKeys = kMfmaTileKeys;
constexpr int kPad = kMfmaPad;

// (m, s) of one row merged over the 16 key-column lanes that hold it: the
// lanes' max, each lane's sum rescaled to it, then the sum over the lanes
// (DPP, a fixed order; one exp per lane instead of one per merge step)
__device__ __forceinline__ void merge_cols(float& m, float& s) {
  const float mx = group_max<16>(m);
  const float ref = mx == -INFINITY ? 0.0f : mx;
  s = group_sum<16>(s * __builtin_amdgcn_exp2f(m - ref));
  m = mx;
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
  bf16_t* kout;              // same layout as k, or NULL
  RopeTheta theta;           // theta_i of the call's base and head dim
};

// D: head dim; RBW: row blocks per wave; NWR: waves across row blocks; NW:
// waves per workgroup (4, or 8 for tall query blocks: fewer rows per wave
// keeps the registers low enough for two waves per SIMD);
// ROT: 0 none, 1 half-split pairs, 2 interleaved pairs; WRITE: store K'.
// N is the number of scored (virtual) rows; with map.units set they are the
// listed units of the source cache, in list order (a unit length that is a
// multiple of the tile, so every tile reads one source unit).
template <int D, int RBW, int NWR, int NW, int ROT, bool WRITE>
__global__ void __launch_bounds__(NW * 64)
score_mfma_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, int64_t N, int H,
                  int64_t stride_b, int64_t stride_n, int T, int Hq, float scale2,
                  int64_t seg_len, int64_t nseg, int64_t segs_per_block, int64_t groups,
                  int passes, float* __restrict__ ms, int natural, ScoreRot rot, UnitMap map) {
  constexpr int KS = D / 32;                 // MFMA k-steps
  constexpr int KROW = D + kPad;             // staged row stride (elements)
  constexpr int kThreads = NW * 64;
  constexpr int NWK = NW / NWR;              // waves across key blocks
  constexpr int KBW = (kTileKeys / 16) / NWK;  // key blocks per wave and tile
  constexpr int VPT = kTileKeys * D / 8 / kThreads;  // 16-byte vectors per thread and tile
  constexpr int ROWS_PASS = NWR * RBW * 16;
  static_assert(VPT >= 1 && KBW >= 1, "tile too small for the workgroup");
  __shared__ __align__(16) bf16_t kt[kTileKeys * KROW];
  __shared__ float red[NWK][ROWS_PASS][2];
  __shared__ double2 cs[ROT ? D / 2 : 1];

  // workgroups are dealt kv head fastest: those running together read the
  // heads of the same cached rows, so their 256-byte pieces of each row are
  // fetched close together (32 kv heads, 8 KiB rows: 43.8 -> 41.5 us; no
  // change with 4 or 8 kv heads)
  // in 32 bits (the grid is below 2^32 workgroups): a 64-bit division by a
  // runtime value is a long scalar sequence that every workgroup would run
  uint32_t x = blockIdx.x;
  const int g = static_cast<int>(x % static_cast<uint32_t>(H)); x /= static_cast<uint32_t>(H);
  const int64_t grp = x % static_cast<uint32_t>(groups); x /= static_cast<uint32_t>(groups);
  const int pass = static_cast<int>(x % static_cast<uint32_t>(passes));
  const int64_t b = x / static_cast<uint32_t>(passes);
  const int G = Hq / H;
  const int R = G * T;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wr = wave % NWR, wk = wave / NWR;
  const int col = lane & 15, quad = lane >> 4;

  // query fragments of this wave's row blocks (rows past R are zero).  A pass
  // fills the first slot of every wave row, then the second, and so on, so a
  // last, partial pass leaves its padding in the last slots of the last wave
  // rows; with eight waves of two slots, one such wave per SIMD.  A wave with
  // at most one block of query rows runs the one-block loop below.
  uint4 qa[RBW][KS];
  int nb = 0;                      // row blocks of this wave holding query rows
#pragma unroll
  for (int i = 0; i < RBW; ++i) {
    const int r = (pass * NWR * RBW + wr + i * NWR) * 16 + col;
    nb += (pass * NWR * RBW + wr + i * NWR) * 16 < R ? 1 : 0;
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
  static_assert(VPT % P == 0, "rotation pairs must stay in one thread");
  auto item = [&](int i, int& key, int& ch) {
    const int e = threadIdx.x + (i / P) * kThreads;
    key = e / CPK;
    ch = e % CPK + (i % P) * (D / 16);
  };
  // Tile cursors.  Every length stepped here (scoring segment, rotation unit,
  // listed unit) is a multiple of the 64-key tile and t_begin starts a
  // segment, so each position advances by one tile with an add and a compare:
  // no integer division inside the loop (64-bit divisions are long scalar
  // sequences that every wave would repeat).
  struct Cursor {
    int64_t u, off, len;
    __device__ void advance() {
      off += kTileKeys;
      if (off >= len) { off = 0; ++u; }
    }
  };
  auto cursor_at = [&](int64_t len) {
    const int64_t u = (t_begin >> 32) == 0 && (len >> 32) == 0
                          ? static_cast<int64_t>(static_cast<uint32_t>(t_begin) / static_cast<uint32_t>(len))
                          : t_begin / len;
    return Cursor{u, t_begin - u * len, len};
  };
  // per-thread offsets of the tile's vectors from the tile's first row
  int64_t voff[VPT];
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    int key, ch;
    item(i, key, ch);
    voff[i] = key * stride_n + ch * 8;
  }
  // load the tile whose first virtual row is t0 (cursor c on its listed unit);
  // returns false when the listed unit is outside the source
  auto fetch = [&](uint4 (&v)[VPT], int64_t t0, const Cursor& c) -> bool {
    int64_t r0 = t0;
    if (map.units != nullptr) {
      const int64_t su = map.units[b * map.n_units + c.u];
      r0 = (su >= 0 && su < map.n_src) ? su * map.unit_len + c.off : -1;
    }
    const int rem = static_cast<int>(min<int64_t>(t_end - t0, kTileKeys));
    const bf16_t* base = kb + r0 * stride_n;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      int key, ch;
      item(i, key, ch);
      v[i] = (key < rem && r0 >= 0) ? *reinterpret_cast<const uint4*>(base + voff[i])
                                     : make_uint4(0, 0, 0, 0);
    }
    return r0 >= 0;
  };
  const bool write_out = WRITE && pass == 0;
  // A thread stages the same chunks of every tile, so it always needs the
  // cos/sin of the same pairs: where these are at most 8 (eight waves), they
  // are copied to registers once per rotation unit instead of read from LDS
  // for every tile.
  constexpr int NCS = ROT == 1 ? (VPT / 2) * 8 : VPT * 4;
  constexpr bool CS_REG = ROT != 0 && NCS <= 8;
  double2 creg[CS_REG ? NCS : 1];
  auto load_cs = [&]() {
    if constexpr (CS_REG) {
#pragma unroll
      for (int i = 0; i < VPT; i += P) {
        int key, ch;
        item(i, key, ch);
        if constexpr (ROT == 1) {
#pragma unroll
          for (int e = 0; e < 8; ++e) creg[(i / 2) * 8 + e] = cs[ch * 8 + e];
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) creg[i * 4 + e] = cs[ch * 4 + e];
        }
      }
    }
  };
  // rotation of a staged tile in registers (cs / creg hold its unit)
  auto rotate_tile = [&](uint4 (&v)[VPT]) {
    if constexpr (ROT == 1) {
#pragma unroll
      for (int i = 0; i < VPT; i += 2) {
        int key, ch;
        item(i, key, ch);
        if constexpr (CS_REG)
          rope_rotate16_with<bf16_t, KVSEL_ROPE_HALF>(
              v[i], v[i + 1], [&](int e) { return creg[(i / 2) * 8 + e]; });
        else
          rope_rotate16<bf16_t, KVSEL_ROPE_HALF>(v[i], v[i + 1], ch * 8, cs);
      }
    } else if constexpr (ROT == 2) {
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        int key, ch;
        item(i, key, ch);
        uint4 unused;
        if constexpr (CS_REG)
          rope_rotate16_with<bf16_t, KVSEL_ROPE_INTERLEAVED>(
              v[i], unused, [&](int e) { return creg[i * 4 + (e >> 1)]; });
        else
          rope_rotate16<bf16_t, KVSEL_ROPE_INTERLEAVED>(v[i], unused, ch * 8, cs);
      }
    }
  };
  auto store = [&](uint4 (&v)[VPT], int64_t t0) {
    const int rem = static_cast<int>(min<int64_t>(t_end - t0, kTileKeys));
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      int key, ch;
      item(i, key, ch);
      *reinterpret_cast<uint4*>(&kt[key * KROW + ch * 8]) = v[i];
      if (write_out && key < rem)
        *reinterpret_cast<uint4*>(rot.kout + b * stride_b + t0 * stride_n +
                                  static_cast<int64_t>(g) * D + voff[i]) = v[i];
    }
  };
  int64_t cs_unit = -1;

  float m[RBW][4], s[RBW][4];
#pragma unroll
  for (int i = 0; i < RBW; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) { m[i][v] = -INFINITY; s[i][v] = 0.0f; }

  Cursor fc = map.units != nullptr ? cursor_at(map.unit_len) : Cursor{0, 0, kTileKeys};
  Cursor rc = ROT != 0 ? cursor_at(rot.rot_len) : Cursor{0, 0, kTileKeys};
  int64_t seg = seg0, seg_off = 0;
  // cos/sin of the rotation unit rc.u (a uniform test; the table is rebuilt
  // only at a unit change, between barriers that every rotation lies outside)
  auto unit_cs = [&]() {
    if constexpr (ROT != 0) {
      if (rc.u != cs_unit) {
        const int64_t delta = rot.delta[b * rot.delta_stride_b + rc.u];
        for (int i = threadIdx.x; i < D / 2; i += kThreads) cs[i] = rope_cs(delta, rot.theta.t[i]);
        cs_unit = rc.u;
        __syncthreads();
        load_cs();
      }
    }
  };
  // Staging pipeline.  A tile's loads are issued one tile ahead into the
  // buffer just stored, and a rotated tile is rotated right before it is
  // stored.  With eight waves (registers to spare) the rotation is pipelined:
  // loads run two tiles ahead and tile t + 1 is rotated in registers while
  // tile t's products run on the matrix cores; tiles alternate between two
  // buffers (a tile's buffer is free once stored, and takes tile t + 2).
  constexpr bool PIPE = ROT != 0 && NW == 8;
  uint4 bufA[VPT], bufB[VPT];
  bool okA = true, okB = true;
  if (t_begin < t_end) {
    okA = fetch(bufA, t_begin, fc);
    fc.advance();
    if constexpr (PIPE) {
      unit_cs();
      rotate_tile(bufA);
      rc.advance();
      if (t_begin + kTileKeys < t_end) {
        okB = fetch(bufB, t_begin + kTileKeys, fc);
        fc.advance();
      }
    }
  }
  // one tile: sb holds it (rotated), rb the next tile's raw rows
  auto body = [&](auto nbc, uint4 (&sb)[VPT], bool& sb_ok, uint4 (&rb)[VPT], int64_t t0)
      __attribute__((always_inline)) {
    constexpr int NB = decltype(nbc)::value;   // active row blocks (the first NB slots)
    __syncthreads();               // previous tile fully read
    if constexpr (ROT != 0 && !PIPE) {
      unit_cs();
      rotate_tile(sb);
      rc.advance();
    }
    store(sb, t0);
    const bool tile_ok = sb_ok;
    __syncthreads();
    constexpr int64_t ahead = PIPE ? 2 * kTileKeys : kTileKeys;
    if (t0 + ahead < t_end) {      // in flight during the math
      sb_ok = fetch(sb, t0 + ahead, fc);
      fc.advance();
    }

    f32x4_t acc[NB][KBW];
#pragma unroll
    for (int jb = 0; jb < KBW; ++jb) {
      const int key = (wk + jb * NWK) * 16 + col;
      uint4 bk[KS];
#pragma unroll
      for (int st = 0; st < KS; ++st)
        bk[st] = *reinterpret_cast<const uint4*>(&kt[key * KROW + st * 32 + quad * 8]);
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        f32x4_t a = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int st = 0; st < KS; ++st)
          a = mfma16x16x32(qa[i][st], bk[st], a);
        acc[i][jb] = a;
      }
    }
    if constexpr (PIPE) {
      if (t0 + kTileKeys < t_end) {   // tile t + 1, while the products run
        unit_cs();
        rotate_tile(rb);
        rc.advance();
      }
    }
    // keys past the end of the cache, or of a unit outside the source, take
    // no part (a uniform test: only a range's last tile or an invalid unit
    // pays for the masking)
    const int rem = static_cast<int>(min<int64_t>(t_end - t0, kTileKeys));
    if (!tile_ok || rem < kTileKeys) {
#pragma unroll
      for (int jb = 0; jb < KBW; ++jb) {
        if (!tile_ok || (wk + jb * NWK) * 16 + col >= rem) {
#pragma unroll
          for (int i = 0; i < NB; ++i)
            acc[i][jb] = f32x4_t{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
        }
      }
    }
    // online softmax, branch-free: while a row has seen only masked keys its
    // max stays -inf and the reference 0 keeps every exp at exp2(-inf) = 0
#pragma unroll
    for (int i = 0; i < NB; ++i) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float tmax = acc[i][0][v];
#pragma unroll
        for (int jb = 1; jb < KBW; ++jb) tmax = fmaxf(tmax, acc[i][jb][v]);
        const float mn = fmaxf(m[i][v], tmax * scale2);
        const float ref = mn == -INFINITY ? 0.0f : mn;
        float acc_s = s[i][v] * __builtin_amdgcn_exp2f(m[i][v] - ref);
#pragma unroll
        for (int jb = 0; jb < KBW; ++jb)
          acc_s += __builtin_amdgcn_exp2f(fmaf(acc[i][jb][v], scale2, -ref));
        s[i][v] = acc_s;
        m[i][v] = mn;
      }
    }

    // end of a segment: merge and publish its partials
    seg_off += kTileKeys;
    if (seg_off == seg_len || t0 + kTileKeys >= t_end) {
      // a skipped slot holds only padded rows, which are not published
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) merge_cols(m[i][v], s[i][v]);
      if (col == 0) {
#pragma unroll
        for (int i = 0; i < NB; ++i)
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
      ++seg;
      seg_off = 0;
    }
  };
  auto run = [&](auto nbc) __attribute__((always_inline)) {
    if constexpr (PIPE) {
      for (int64_t t0 = t_begin; t0 < t_end; t0 += 2 * kTileKeys) {
        body(nbc, bufA, okA, bufB, t0);
        if (t0 + kTileKeys < t_end) body(nbc, bufB, okB, bufA, t0 + kTileKeys);
      }
    } else {
      for (int64_t t0 = t_begin; t0 < t_end; t0 += kTileKeys) body(nbc, bufA, okA, bufA, t0);
    }
  };
  // every wave passes the same barriers in either loop; a wave with no query
  // rows (a short last pass) runs the one-block loop on zero queries
  if constexpr (RBW == 1) run(std::integral_constant<int, 1>{});
  else if (nb > 1) run(std::integral_constant<int, RBW>{});   // padded slots too, if any
  else run(std::integral_constant<int, 1>{});
}

template <int D, int RBW, int NWR, int NW, int ROT, bool WRITE>
void launch(const void* q, int64_t T, int64_t Hq, const void* k, const kvsel_cache& kc,
            float scale2, int64_t seg_len, int64_t nseg, int64_t spb, int passes, float* ms,
            int natural, const ScoreRot& rot, const UnitMap& map, hipStream_t s) {
  const int64_t groups = (nseg + spb - 1) / spb;
  const int64_t blocks = kc.B * kc.H * passes * groups;
  hipLaunchKernelGGL((score_mfma_kernel<D, RBW, NWR, NW, ROT, WRITE>),
                     dim3(static_cast<unsigned>(blocks)), dim3(NW * 64), 0, s,
                     static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k), kc.N,
                     static_cast<int>(kc.H), kc.stride_b, kc.stride_n, static_cast<int>(T),
                     static_cast<int>(Hq), scale2, seg_len, nseg, spb, groups, passes, ms, natural,
                     rot, map);
}

template <int D, int ROT, bool WRITE>
void dispatch(const void* q, int64_t T, int64_t Hq, const void* k, const kvsel_cache& kc,
              float scale2, int64_t seg_len, int64_t nseg, float* ms, int natural,
              const ScoreRot& rot, const UnitMap& map, hipStream_t s) {
  const int64_t rows = (Hq / kc.H) * T;
  const int64_t rb = (rows + 15) / 16;
  // up to 8 row blocks: four waves (mfma_row_plan; a wave's row blocks share
  // each key fragment it reads from LDS).  Taller blocks, head dim 128: eight
  // waves of two row blocks, which halves the registers per wave (two waves
  // per SIMD instead of one).  Measured on MI355X: 224 and 448 rows per kv
  // head run faster with eight waves, 128 rows slower.
  MfmaRowPlan p = mfma_row_plan(rows);
  int nw = 4;
  if (D == 128 && rb > 8) {
    nw = 8;
    p = MfmaRowPlan{2, 8, static_cast<int>((rb + 15) / 16)};
  }
  // up to 1024 keys per workgroup (segments of 256 go four to a block), fewer
  // when that leaves under ~2048 workgroups for the 256 CUs, but not fewer
  // than 256: a workgroup loads its query fragments once for at least 4
  // tiles.  448 rows per kv head over 16,384 keys: 512 workgroups of 256 keys,
  // two to a CU (122 VGPRs), 22.3 -> 20.0 us against 256 of 512 keys
  int64_t spb = seg_len >= 1024 ? 1 : 1024 / seg_len;
  while (spb > 1 && spb * seg_len > 256 && kc.B * kc.H * p.passes * ((nseg + spb - 1) / spb) < 2048)
    spb /= 2;
#define KVSEL_SM(RBW, NWR, NW)                                                             \
  if (p.rbw == RBW && p.nwr == NWR && nw == NW)                                            \
    return launch<D, RBW, NWR, NW, ROT, WRITE>(q, T, Hq, k, kc, scale2, seg_len, nseg, spb, \
                                               p.passes, ms, natural, rot, map, s);
  KVSEL_SM(1, 1, 4) KVSEL_SM(1, 2, 4) KVSEL_SM(1, 4, 4) KVSEL_SM(2, 4, 4) KVSEL_SM(4, 4, 4)
  if constexpr (D == 128) { KVSEL_SM(2, 8, 8) }
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
  const ScoreRot none{nullptr, 0, 1, nullptr, RopeTheta{}};
  const UnitMap all{nullptr, 0, 1, 0};
  if (kc.D == 128)
    dispatch<128, 0, false>(q, T, Hq, k, kc, scale2, seg_len, nseg, ms, natural, none, all, s);
  else
    dispatch<64, 0, false>(q, T, Hq, k, kc, scale2, seg_len, nseg, ms, natural, none, all, s);
}

void launch_score_mfma_rot(const void* q, int64_t T, int64_t Hq, const void* k, void* k_out,
                           const kvsel_cache& kc, float scale, int64_t seg_len, int64_t nseg,
                           float* ms, int natural, int64_t rot_len, const int64_t* delta,
                           int per_instance, double base, int style, hipStream_t s) {
  const float scale2 = scale * kLog2e;
  const ScoreRot rot{delta, per_instance ? kc.N / rot_len : 0, rot_len,
                     static_cast<bf16_t*>(k_out), rope_theta(base, kc.D)};
  const bool w = k_out != nullptr;
  const UnitMap all{nullptr, 0, 1, 0};
#define KVSEL_SR(D_, ST)                                                                   \
  if (w) dispatch<D_, ST, true>(q, T, Hq, k, kc, scale2, seg_len, nseg, ms, natural, rot, all, s); \
  else dispatch<D_, ST, false>(q, T, Hq, k, kc, scale2, seg_len, nseg, ms, natural, rot, all, s);
  if (kc.D == 128) {
    if (style == KVSEL_ROPE_HALF) { KVSEL_SR(128, 1) } else { KVSEL_SR(128, 2) }
  } else {
    if (style == KVSEL_ROPE_HALF) { KVSEL_SR(64, 1) } else { KVSEL_SR(64, 2) }
  }
#undef KVSEL_SR
}

void launch_score_mfma_units(const void* q, int64_t T, int64_t Hq, const void* k,
                             const kvsel_cache& kc, const UnitMap& map, float scale,
                             int64_t seg_len, int64_t nseg, float* ms, int natural,
                             const int64_t* delta, int per_instance, double base, int style,
                             hipStream_t s) {
  const float scale2 = scale * kLog2e;
  kvsel_cache kv = kc;  // N = scored rows; strides stay the source's
  kv.N = map.n_units * map.unit_len;
  const ScoreRot rot{delta, per_instance ? map.n_units : 0, map.unit_len, nullptr,
                     delta != nullptr ? rope_theta(base, kc.D) : RopeTheta{}};
#define KVSEL_SU(D_, ST) \
  dispatch<D_, ST, false>(q, T, Hq, k, kv, scale2, seg_len, nseg, ms, natural, rot, map, s);
  if (kc.D == 128) {
    if (delta == nullptr) { KVSEL_SU(128, 0) }
    else if (style == KVSEL_ROPE_HALF) { KVSEL_SU(128, 1) } else { KVSEL_SU(128, 2) }
  } else {
    if (delta == nullptr) { KVSEL_SU(64, 0) }
    else if (style == KVSEL_ROPE_HALF) { KVSEL_SU(64, 1) } else { KVSEL_SU(64, 2) }
  }
#undef KVSEL_SU
}

}  // namespace kvsel
