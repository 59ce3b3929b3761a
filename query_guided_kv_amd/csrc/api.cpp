// C ABI of libkvsel: argument validation, workspace sizing and dispatch.
// Every check runs on the host before anything is enqueued; no call allocates
// device memory.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "internal.h"
#include "kvsel.h"

namespace kvsel {

namespace {
thread_local char g_err[512] = "";
}

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

RopeTheta rope_theta(double base, int64_t D) {
  RopeTheta th{};
  for (int64_t i = 0; i < D / 2 && i < 64; ++i)
    th.t[i] = std::pow(base, -2.0 * static_cast<double>(i) / static_cast<double>(D));
  return th;
}

int check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e == hipSuccess) return KVSEL_OK;
  set_error("%s: %s", what, hipGetErrorString(e));
  return KVSEL_ERR_HIP;
}

namespace {

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Where the rows of a gather source live.  Device (and managed) memory is read
// directly; pinned host memory through the device address the runtime maps it
// to, over the host link; anything else, pageable host memory in particular,
// is refused here, before a kernel could touch it.
int resolve_rows(const void* p, const void** out, const char* name) {
  hipPointerAttribute_t a{};
  const hipError_t e = hipPointerGetAttributes(&a, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();  // leave no sticky error for the next launch check
    return fail(KVSEL_ERR_UNSUPPORTED,
                "%s: neither device memory nor pinned host memory (%s)", name, hipGetErrorString(e));
  }
  switch (a.type) {
    case hipMemoryTypeDevice:
    case hipMemoryTypeManaged:
    case hipMemoryTypeUnified:
      *out = p;
      return KVSEL_OK;
    case hipMemoryTypeHost:
      if (a.devicePointer == nullptr)
        return fail(KVSEL_ERR_UNSUPPORTED, "%s: pinned host memory without a device mapping", name);
      if ((reinterpret_cast<uintptr_t>(a.devicePointer) & 15u) != 0)
        return fail(KVSEL_ERR_UNSUPPORTED, "%s: mapped host address is not 16-byte aligned", name);
      *out = a.devicePointer;
      return KVSEL_OK;
    default:
      return fail(KVSEL_ERR_UNSUPPORTED,
                  "%s: pageable host memory; allocate it pinned (hipHostMalloc)", name);
  }
}

// do the byte ranges [a, a + na) and [b, b + nb) share a byte?
bool overlap(const void* a, int64_t na, const void* b, int64_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return na > 0 && nb > 0 && x < y + static_cast<uintptr_t>(nb) && y < x + static_cast<uintptr_t>(na);
}

int check_cache(const kvsel_cache& kc, const char* what) {
  if (kc.dtype != KVSEL_BF16 && kc.dtype != KVSEL_FP32)
    return fail(KVSEL_ERR_DTYPE, "%s: dtype %d is neither bf16 nor fp32", what, kc.dtype);
  if (kc.B < 1 || kc.N < 1 || kc.H < 1)
    return fail(KVSEL_ERR_SHAPE, "%s: B, N, H must be >= 1 (B=%lld N=%lld H=%lld)", what,
                (long long)kc.B, (long long)kc.N, (long long)kc.H);
  if (kc.D != 64 && kc.D != 128)
    return fail(KVSEL_ERR_UNSUPPORTED, "%s: head dim %lld not in {64, 128}", what, (long long)kc.D);
  if (kc.stride_n < kc.H * kc.D || kc.stride_b < kc.N * kc.stride_n)
    return fail(KVSEL_ERR_SHAPE, "%s: strides too small for [N][H][D]", what);
  if (kc.stride_n % 8 != 0 || kc.stride_b % 8 != 0)
    return fail(KVSEL_ERR_UNSUPPORTED, "%s: strides must be multiples of 8 elements", what);
  if (kc.B > (int64_t{1} << 24) || kc.N >= (int64_t{1} << 31))
    return fail(KVSEL_ERR_SHAPE, "%s: B or N out of range", what);
  if (kc.stride_n >= (int64_t{1} << 24))
    return fail(KVSEL_ERR_UNSUPPORTED, "%s: row stride %lld is not below 2^24 elements", what,
                (long long)kc.stride_n);
  return KVSEL_OK;
}

int check_ptr(const void* p, const char* name) {
  if (p == nullptr) return fail(KVSEL_ERR_NULL, "%s is NULL", name);
  if (!aligned16(p)) return fail(KVSEL_ERR_UNSUPPORTED, "%s is not 16-byte aligned", name);
  return KVSEL_OK;
}

int check_heads(int64_t T, int64_t Hq, const kvsel_cache& kc, const char* what) {
  if (T < 1 || Hq < 1 || Hq % kc.H != 0)
    return fail(KVSEL_ERR_SHAPE, "%s: need T >= 1 and Hq a multiple of H (T=%lld Hq=%lld H=%lld)",
                what, (long long)T, (long long)Hq, (long long)kc.H);
  if (Hq > 4096 || T > 65536 || (Hq / kc.H) * T > (int64_t{1} << 20))
    return fail(KVSEL_ERR_SHAPE, "%s: query block too large", what);
  return KVSEL_OK;
}

// The matrix-core kernels take the maximum of the raw dot products and scale
// it afterwards, which is the maximum scaled logit only for a positive scale;
// a scale that is not finite would turn every logit into inf or NaN.
int check_scale(float scale, const char* what) {
  if (!(scale > 0.0f) || !std::isfinite(scale))
    return fail(KVSEL_ERR_SHAPE, "%s: scale %g must be finite and > 0", what, static_cast<double>(scale));
  return KVSEL_OK;
}

int check_units(const kvsel_cache& kc, int64_t unit_len, const char* what) {
  if (unit_len < 1 || kc.N % unit_len != 0)
    return fail(KVSEL_ERR_SHAPE, "%s: unit_len %lld must be >= 1 and divide N=%lld", what,
                (long long)unit_len, (long long)kc.N);
  return KVSEL_OK;
}

#define KVSEL_TRY(x)            \
  do {                          \
    const int rc_ = (x);        \
    if (rc_ != KVSEL_OK) return rc_; \
  } while (0)

size_t score_ws(int64_t B, int64_t N, int64_t Hq, int64_t T, int64_t unit_len, bool stats,
                bool part) {
  if (!stats || (part && unit_len > 1)) return 0;
  const int64_t nseg = (N + kTokenTile - 1) / kTokenTile;
  return static_cast<size_t>(B * Hq * T * nseg * 2) * sizeof(float);
}

// chunk path: [derived row stats: 2 * B*Hq*T] [row-chunk sums]; token path:
// per-token sums B*N
size_t aggregate_ws(int64_t B, int64_t N, int64_t Hq, int64_t T, int64_t unit_len, bool chunk,
                    bool have_stats) {
  if (chunk)
    return (static_cast<size_t>(have_stats ? 0 : 2 * B * Hq * T) +
            aggregate_chunk_ws_floats(B, Hq, T, N / unit_len)) * sizeof(float);
  // token path: per-token sums, in up to kAggMaxParts partial arrays for small caches
  return static_cast<size_t>(B * N * (B * N < kAggSplitRows ? kAggMaxParts : 1)) * sizeof(float);
}

int64_t decode_splits(const kvsel_segment* segs, int n_seg, int64_t split_len) {
  int64_t n = 0;
  for (int i = 0; i < n_seg; ++i) n += (segs[i].kc.N + split_len - 1) / split_len;
  return n;
}

int64_t total_keys(const kvsel_segment* segs, int n_seg) {
  int64_t n = 0;
  for (int i = 0; i < n_seg; ++i) n += segs[i].kc.N;
  return n;
}

int64_t split_len_of(int64_t T, int64_t Hq, const kvsel_cache& c, bool gathered, int64_t n_keys) {
  return decode_split_len(c.dtype, c.H, c.D, c.H > 0 ? (Hq / c.H) * T : 1, gathered, c.B, n_keys);
}

// (m, s, o) partials of every split of the segments; `gathered` when the last
// segment is gathered on the fly (the split length depends on the kernel)
// Decode workspace: the (m, s) pairs of every row and split, then, from a
// 16-byte boundary, the rows' partial outputs (D floats per row and split).
int64_t decode_ms_floats(int64_t rows, int64_t n_split) { return (rows * n_split * 2 + 3) / 4 * 4; }

size_t decode_ws(int64_t T, int64_t Hq, const kvsel_segment* segs, int n_seg, bool gathered) {
  if (segs == nullptr || n_seg < 1 || n_seg > kMaxSegments || T < 1 || Hq < 1) return 0;
  for (int i = 0; i < n_seg; ++i)
    if (segs[i].kc.N < 1 || segs[i].kc.B < 1 || segs[i].kc.D < 1) return 0;
  const int64_t n_split =
      decode_splits(segs, n_seg, split_len_of(T, Hq, segs[0].kc, gathered, total_keys(segs, n_seg)));
  const int64_t rows = segs[0].kc.B * Hq * T;
  return static_cast<size_t>(decode_ms_floats(rows, n_split) + rows * n_split * segs[0].kc.D) *
         sizeof(float);
}

}  // namespace
}  // namespace kvsel

using namespace kvsel;

extern "C" {

int kvsel_version(void) { return 100; }

const char* kvsel_last_error(void) { return kvsel::g_err; }

const char* kvsel_status_str(int status) {
  switch (status) {
    case KVSEL_OK: return "ok";
    case KVSEL_ERR_NULL: return "null pointer";
    case KVSEL_ERR_SHAPE: return "inconsistent or out-of-range sizes";
    case KVSEL_ERR_DTYPE: return "unsupported dtype";
    case KVSEL_ERR_UNSUPPORTED: return "unsupported head dim, alignment or stride";
    case KVSEL_ERR_WORKSPACE: return "workspace too small";
    case KVSEL_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int kvsel_reposition(const void* k_in, void* k_out, kvsel_cache kc, int64_t unit_len,
                     const int64_t* delta, int32_t delta_per_instance, double rope_base,
                     int32_t rope_style, hipStream_t stream) {
  KVSEL_TRY(check_ptr(k_in, "k_in"));
  KVSEL_TRY(check_ptr(k_out, "k_out"));
  if (delta == nullptr) return fail(KVSEL_ERR_NULL, "delta is NULL");
  KVSEL_TRY(check_cache(kc, "kvsel_reposition"));
  KVSEL_TRY(check_units(kc, unit_len, "kvsel_reposition"));
  if (rope_style != KVSEL_ROPE_HALF && rope_style != KVSEL_ROPE_INTERLEAVED)
    return fail(KVSEL_ERR_SHAPE, "kvsel_reposition: unknown rope_style %d", rope_style);
  if (!(rope_base > 1.0))
    return fail(KVSEL_ERR_SHAPE, "kvsel_reposition: rope_base must be > 1");
  return launch_reposition(k_in, k_out, kc, unit_len, delta, delta_per_instance != 0, rope_base,
                           rope_style, stream);
}

size_t kvsel_score_workspace(int64_t B, int64_t N, int64_t Hq, int64_t T, int64_t unit_len,
                             int32_t want_row_stats, int32_t want_part) {
  if (B < 1 || N < 1 || Hq < 1 || T < 1 || unit_len < 1) return 0;
  return score_ws(B, N, Hq, T, unit_len, want_row_stats != 0, want_part != 0);
}

}  // extern "C"

namespace {

// Re-positioning that a scoring call applies on the fly.
struct ScoreRotArgs {
  void* k_out;
  int64_t unit_len;
  const int64_t* delta;
  int per_instance;
  double base;
  int style;
};

size_t round256(size_t n) { return (n + 255) / 256 * 256; }

// Workspace of kvsel_score_reposition: the scoring workspace, plus room for
// the re-positioned keys when they cannot be formed on the fly and the caller
// keeps none.
size_t score_rot_ws(int64_t T, int64_t Hq, const kvsel_cache& kc, int64_t unit_len,
                    int64_t rot_unit_len, bool stats, bool part, bool have_k_out) {
  const size_t base = score_ws(kc.B, kc.N, Hq, T, unit_len, stats, part);
  const int64_t seg_len = part ? unit_len : kTokenTile;
  const bool fused = score_mfma_rot_ok(kc.dtype, (Hq / kc.H) * T, seg_len, rot_unit_len);
  if (fused || have_k_out) return base;
  const size_t esz = kc.dtype == KVSEL_BF16 ? 2 : 4;
  return round256(base) + static_cast<size_t>(kc.B * kc.stride_b) * esz;
}

// kvsel_score_units takes the matrix-core scorer, which reads the listed
// units in place, when a unit is a whole number of 64-key tiles; otherwise the
// units are copied to the workspace first.
bool score_units_mfma(int dtype, int64_t rows_per_kv, int64_t seg_len, int64_t unit_len) {
  return score_mfma_ok(dtype, rows_per_kv, seg_len) && unit_len % kMfmaTileKeys == 0;
}

size_t score_units_ws(int64_t T, int64_t Hq, const kvsel_cache& kc, int64_t unit_len,
                      int64_t n_units, bool stats, bool part) {
  const int64_t nv = n_units * unit_len;
  const size_t base = score_ws(kc.B, nv, Hq, T, unit_len, stats, part);
  const int64_t seg_len = part ? unit_len : kTokenTile;
  if (kc.H < 1 || score_units_mfma(kc.dtype, (Hq / kc.H) * T, seg_len, unit_len)) return base;
  const size_t esz = kc.dtype == KVSEL_BF16 ? 2 : 4;
  return round256(base) + static_cast<size_t>(kc.B * nv * kc.H * kc.D) * esz;
}

int score_impl(const void* q, int64_t T, int64_t Hq, const void* k, const kvsel_cache& kc,
               float scale, int64_t unit_len, float* row_max, float* row_sum, float* part,
               void* ws, size_t ws_bytes, hipStream_t stream, const ScoreRotArgs* rot,
               const char* what) {
  KVSEL_TRY(check_ptr(q, "q"));
  KVSEL_TRY(check_ptr(k, "k"));
  KVSEL_TRY(check_cache(kc, what));
  KVSEL_TRY(check_heads(T, Hq, kc, what));
  KVSEL_TRY(check_units(kc, unit_len, what));
  KVSEL_TRY(check_scale(scale, what));
  if ((row_max == nullptr) != (row_sum == nullptr))
    return fail(KVSEL_ERR_NULL, "%s: row_max and row_sum must both be set or both NULL", what);
  const bool stats = row_max != nullptr;
  if (!stats && part == nullptr) return fail(KVSEL_ERR_NULL, "%s: no output requested", what);
  if (part != nullptr && unit_len < 2)
    return fail(KVSEL_ERR_SHAPE, "%s: per-unit partials need unit_len > 1", what);
  const size_t need = rot == nullptr
                          ? score_ws(kc.B, kc.N, Hq, T, unit_len, stats, part != nullptr)
                          : score_rot_ws(T, Hq, kc, unit_len, rot->unit_len, stats,
                                         part != nullptr, rot->k_out != nullptr);
  if (need > 0 && (ws == nullptr || ws_bytes < need))
    return fail(KVSEL_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", what, ws_bytes, need);
  const int64_t rows = kc.B * Hq * T;
  const int64_t seg_len = part != nullptr ? unit_len : kTokenTile;
  const int64_t nseg = (kc.N + seg_len - 1) / seg_len;
  float* ms = part != nullptr ? part : static_cast<float*>(ws);
  const int natural = part != nullptr ? 1 : 0;
  if (rot != nullptr) {
    if (score_mfma_rot_ok(kc.dtype, (Hq / kc.H) * T, seg_len, rot->unit_len)) {
      launch_score_mfma_rot(q, T, Hq, k, rot->k_out, kc, scale, seg_len, nseg, ms,
                            natural, rot->unit_len, rot->delta, rot->per_instance, rot->base,
                            rot->style, stream);
      KVSEL_TRY(check_launch(what));
    } else {
      // separate passes; without k_out the keys go to the workspace tail
      void* kp = rot->k_out;
      if (kp == nullptr)
        kp = static_cast<char*>(ws) +
             round256(score_ws(kc.B, kc.N, Hq, T, unit_len, stats, part != nullptr));
      KVSEL_TRY(launch_reposition(k, kp, kc, rot->unit_len, rot->delta, rot->per_instance,
                                  rot->base, rot->style, stream));
      KVSEL_TRY(launch_score_partials(q, T, Hq, kp, kc, scale, seg_len, ms, natural, stream));
    }
  } else {
    KVSEL_TRY(launch_score_partials(q, T, Hq, k, kc, scale, seg_len, ms, natural, stream));
  }
  if (stats) return launch_rowstats(ms, rows, nseg, natural, row_max, row_sum, stream);
  return KVSEL_OK;
}

}  // namespace

extern "C" {

int kvsel_score(const void* q, int64_t T, int64_t Hq, const void* k, kvsel_cache kc, float scale,
                int64_t unit_len, float* row_max, float* row_sum, float* part, void* ws,
                size_t ws_bytes, hipStream_t stream) {
  return score_impl(q, T, Hq, k, kc, scale, unit_len, row_max, row_sum, part, ws, ws_bytes,
                    stream, nullptr, "kvsel_score");
}

size_t kvsel_score_reposition_workspace(int64_t T, int64_t Hq, kvsel_cache kc, int64_t unit_len,
                                        int64_t rot_unit_len, int32_t want_row_stats,
                                        int32_t want_part, int32_t have_k_out) {
  if (T < 1 || Hq < 1 || kc.B < 1 || kc.N < 1 || kc.H < 1 || unit_len < 1 || rot_unit_len < 1)
    return 0;
  return score_rot_ws(T, Hq, kc, unit_len, rot_unit_len, want_row_stats != 0, want_part != 0,
                      have_k_out != 0);
}

int kvsel_score_reposition(const void* q, int64_t T, int64_t Hq, const void* k, void* k_out,
                           kvsel_cache kc, float scale, int64_t unit_len, int64_t rot_unit_len,
                           const int64_t* delta, int32_t delta_per_instance, double rope_base,
                           int32_t rope_style, float* row_max, float* row_sum, float* part,
                           void* ws, size_t ws_bytes, hipStream_t stream) {
  const char* what = "kvsel_score_reposition";
  if (delta == nullptr) return fail(KVSEL_ERR_NULL, "delta is NULL");
  if (k_out != nullptr) {
    KVSEL_TRY(check_ptr(k_out, "k_out"));
    if (k_out == k) return fail(KVSEL_ERR_SHAPE, "%s: k_out must not overlap k", what);
  }
  KVSEL_TRY(check_cache(kc, what));
  KVSEL_TRY(check_units(kc, rot_unit_len, what));
  if (rope_style != KVSEL_ROPE_HALF && rope_style != KVSEL_ROPE_INTERLEAVED)
    return fail(KVSEL_ERR_SHAPE, "%s: unknown rope_style %d", what, rope_style);
  if (!(rope_base > 1.0)) return fail(KVSEL_ERR_SHAPE, "%s: rope_base must be > 1", what);
  const ScoreRotArgs rot{k_out, rot_unit_len, delta, delta_per_instance != 0, rope_base,
                         rope_style};
  return score_impl(q, T, Hq, k, kc, scale, unit_len, row_max, row_sum, part, ws, ws_bytes,
                    stream, &rot, what);
}

size_t kvsel_score_units_workspace(int64_t T, int64_t Hq, kvsel_cache kc, int64_t unit_len,
                                   int64_t n_units, int32_t want_row_stats, int32_t want_part) {
  if (T < 1 || Hq < 1 || kc.B < 1 || kc.H < 1 || unit_len < 1 || n_units < 1) return 0;
  return score_units_ws(T, Hq, kc, unit_len, n_units, want_row_stats != 0, want_part != 0);
}

int kvsel_score_units(const void* q, int64_t T, int64_t Hq, const void* k, kvsel_cache kc,
                      float scale, int64_t unit_len, const int32_t* units, int64_t n_units,
                      const int64_t* delta, int32_t delta_per_instance, double rope_base,
                      int32_t rope_style, float* row_max, float* row_sum, float* part, void* ws,
                      size_t ws_bytes, hipStream_t stream) {
  const char* what = "kvsel_score_units";
  KVSEL_TRY(check_ptr(q, "q"));
  KVSEL_TRY(check_ptr(k, "k"));
  if (units == nullptr) return fail(KVSEL_ERR_NULL, "units is NULL");
  KVSEL_TRY(check_cache(kc, what));
  KVSEL_TRY(check_heads(T, Hq, kc, what));
  KVSEL_TRY(check_units(kc, unit_len, what));
  KVSEL_TRY(check_scale(scale, what));
  if (n_units < 1 || n_units * unit_len >= (int64_t{1} << 31))
    return fail(KVSEL_ERR_SHAPE, "%s: n_units=%lld out of range", what, (long long)n_units);
  if (delta != nullptr) {
    if (rope_style != KVSEL_ROPE_HALF && rope_style != KVSEL_ROPE_INTERLEAVED)
      return fail(KVSEL_ERR_SHAPE, "%s: unknown rope_style %d", what, rope_style);
    if (!(rope_base > 1.0)) return fail(KVSEL_ERR_SHAPE, "%s: rope_base must be > 1", what);
  }
  if ((row_max == nullptr) != (row_sum == nullptr))
    return fail(KVSEL_ERR_NULL, "%s: row_max and row_sum must both be set or both NULL", what);
  const bool stats = row_max != nullptr;
  if (!stats && part == nullptr) return fail(KVSEL_ERR_NULL, "%s: no output requested", what);
  if (part != nullptr && unit_len < 2)
    return fail(KVSEL_ERR_SHAPE, "%s: per-unit partials need unit_len > 1", what);
  const size_t need = score_units_ws(T, Hq, kc, unit_len, n_units, stats, part != nullptr);
  if (need > 0 && (ws == nullptr || ws_bytes < need))
    return fail(KVSEL_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", what, ws_bytes, need);
  const int64_t nv = n_units * unit_len;  // scored rows per instance
  const int64_t rows = kc.B * Hq * T;
  const int64_t seg_len = part != nullptr ? unit_len : kTokenTile;
  const int64_t nseg = (nv + seg_len - 1) / seg_len;
  float* ms = part != nullptr ? part : static_cast<float*>(ws);
  const int natural = part != nullptr ? 1 : 0;
  const int per_instance = delta_per_instance != 0;
  if (score_units_mfma(kc.dtype, (Hq / kc.H) * T, seg_len, unit_len)) {
    const UnitMap map{units, n_units, unit_len, kc.N / unit_len};
    launch_score_mfma_units(q, T, Hq, k, kc, map, scale, seg_len, nseg, ms, natural, delta,
                            per_instance, rope_base, rope_style, stream);
    KVSEL_TRY(check_launch(what));
  } else {
    // copy the listed units to the workspace tail, re-position them there,
    // then score the copy
    const kvsel_cache kv{kc.B, nv, kc.H, kc.D, nv * kc.H * kc.D, kc.H * kc.D, kc.dtype};
    void* kp = static_cast<char*>(ws) +
               round256(score_ws(kc.B, nv, Hq, T, unit_len, stats, part != nullptr));
    KVSEL_TRY(launch_gather(k, nullptr, kc, unit_len, units, n_units, 1, nullptr, -1, 0.0,
                            KVSEL_ROPE_HALF, 0, nv, kp, nullptr, stream));
    if (delta != nullptr)
      KVSEL_TRY(launch_reposition(kp, kp, kv, unit_len, delta, per_instance, rope_base,
                                  rope_style, stream));
    KVSEL_TRY(launch_score_partials(q, T, Hq, kp, kv, scale, seg_len, ms, natural, stream));
  }
  if (stats) return launch_rowstats(ms, rows, nseg, natural, row_max, row_sum, stream);
  return KVSEL_OK;
}

size_t kvsel_aggregate_workspace(int64_t B, int64_t N, int64_t Hq, int64_t T, int64_t unit_len,
                                 int32_t chunk_path, int32_t have_row_stats) {
  if (B < 1 || N < 1 || Hq < 1 || T < 1 || unit_len < 1) return 0;
  return aggregate_ws(B, N, Hq, T, unit_len, chunk_path != 0, have_row_stats != 0);
}

int kvsel_aggregate(const void* q, int64_t T, int64_t Hq, const void* k, const void* v,
                    kvsel_cache kc, float scale, const float* row_max, const float* row_sum,
                    const float* part, int32_t signal, int64_t unit_len, int64_t group,
                    float* unit_score, int32_t accumulate, void* ws, size_t ws_bytes,
                    hipStream_t stream) {
  KVSEL_TRY(check_cache(kc, "kvsel_aggregate"));
  KVSEL_TRY(check_heads(T, Hq, kc, "kvsel_aggregate"));
  KVSEL_TRY(check_units(kc, unit_len, "kvsel_aggregate"));
  KVSEL_TRY(check_scale(scale, "kvsel_aggregate"));
  if (signal != KVSEL_SIG_MASS && signal != KVSEL_SIG_VNORM)
    return fail(KVSEL_ERR_SHAPE, "kvsel_aggregate: unknown signal %d", signal);
  if (group < 1 || kc.B % group != 0)
    return fail(KVSEL_ERR_SHAPE, "kvsel_aggregate: group %lld must divide B=%lld",
                (long long)group, (long long)kc.B);
  if (unit_score == nullptr) return fail(KVSEL_ERR_NULL, "unit_score is NULL");
  if ((row_max == nullptr) != (row_sum == nullptr))
    return fail(KVSEL_ERR_NULL, "kvsel_aggregate: row_max and row_sum must both be set or both NULL");
  const bool chunk = signal == KVSEL_SIG_MASS && part != nullptr;
  const bool stats = row_max != nullptr;
  const int64_t M = kc.N / unit_len;
  const int64_t rows = kc.B * Hq * T;
  const size_t need = aggregate_ws(kc.B, kc.N, Hq, T, unit_len, chunk, stats);
  if (need > 0 && (ws == nullptr || ws_bytes < need))
    return fail(KVSEL_ERR_WORKSPACE, "kvsel_aggregate: workspace %zu < %zu bytes", ws_bytes, need);
  if (chunk) {
    if (unit_len < 2) return fail(KVSEL_ERR_SHAPE, "kvsel_aggregate: partials need unit_len > 1");
    const float* rm = row_max;
    const float* rs = row_sum;
    float* w = static_cast<float*>(ws);
    if (!stats && aggregate_chunks_derive(M)) {
      rm = rs = nullptr;             // derived inside the aggregation launch
      w += 2 * rows;
    } else if (!stats) {
      KVSEL_TRY(launch_rowstats(part, rows, M, 1, w, w + rows, stream));
      rm = w;
      rs = w + rows;
      w += 2 * rows;
    }
    return launch_aggregate_chunks(part, rm, rs, kc.B, Hq, T, M, group, unit_score,
                                   accumulate != 0, w, stream);
  }
  KVSEL_TRY(check_ptr(q, "q"));
  KVSEL_TRY(check_ptr(k, "k"));
  if (signal == KVSEL_SIG_VNORM) KVSEL_TRY(check_ptr(v, "v"));
  if (!stats)
    return fail(KVSEL_ERR_NULL, "kvsel_aggregate: the token path needs row_max and row_sum");
  float* per_token = static_cast<float*>(ws);
  const int64_t parts = aggregate_token_parts(kc, Hq, T);
  KVSEL_TRY(launch_aggregate_tokens(q, T, Hq, k, v, kc, scale, row_max, row_sum,
                                    signal == KVSEL_SIG_VNORM, per_token, stream));
  return launch_unit_sums(per_token, parts, kc.B, kc.N, unit_len, group, unit_score,
                          accumulate != 0, stream);
}

int kvsel_topk(const float* score, int64_t G, int64_t M, int64_t k, int32_t* idx, float* val,
               hipStream_t stream) {
  if (score == nullptr) return fail(KVSEL_ERR_NULL, "score is NULL");
  // one 1024-thread workgroup per row: G * 1024 work-items fit in 32 bits
  if (G < 1 || M < 1 || M >= (int64_t{1} << 31) || G >= (int64_t{1} << 21))
    return fail(KVSEL_ERR_SHAPE, "kvsel_topk: G=%lld M=%lld out of range", (long long)G,
                (long long)M);
  if (k < 0 || k > M)
    return fail(KVSEL_ERR_SHAPE, "kvsel_topk: k=%lld not in [0, M=%lld]", (long long)k,
                (long long)M);
  if (k == 0) return KVSEL_OK;
  if (idx == nullptr) return fail(KVSEL_ERR_NULL, "idx is NULL");
  return launch_topk(score, G, M, k, idx, val, stream);
}

int kvsel_take(const int32_t* src, int64_t G, int64_t m, const int32_t* idx, int64_t k,
               int32_t* out, hipStream_t stream) {
  // one work-item per output element: G * k must fit the dispatch's 32-bit size
  if (G < 1 || m < 1 || m >= (int64_t{1} << 31) || k < 0 || k >= (int64_t{1} << 31) ||
      G >= (int64_t{1} << 31) || G * k >= (int64_t{1} << 31))
    return fail(KVSEL_ERR_SHAPE, "kvsel_take: G=%lld m=%lld k=%lld out of range", (long long)G,
                (long long)m, (long long)k);
  if (k == 0) return KVSEL_OK;
  if (src == nullptr || idx == nullptr || out == nullptr)
    return fail(KVSEL_ERR_NULL, "kvsel_take: src, idx and out must be set");
  if (overlap(out, G * k * 4, src, G * m * 4) || overlap(out, G * k * 4, idx, G * k * 4))
    return fail(KVSEL_ERR_SHAPE, "kvsel_take: out must not overlap src or idx");
  return launch_take(src, G, m, idx, k, out, stream);
}

int kvsel_order(const float* score, int64_t G, int64_t M, const int32_t* idx, int64_t k,
                int32_t descending, int32_t* idx_out, float* val_out, hipStream_t stream) {
  if (G < 1 || M < 1 || M >= (int64_t{1} << 31) || k < 0 || k >= (int64_t{1} << 31))
    return fail(KVSEL_ERR_SHAPE, "kvsel_order: G=%lld M=%lld k=%lld out of range", (long long)G,
                (long long)M, (long long)k);
  if (G >= (int64_t{1} << 31) || G * ((k + 255) / 256) >= (int64_t{1} << 23))
    return fail(KVSEL_ERR_SHAPE, "kvsel_order: too many rows");  // 256 work-items per block
  if (k == 0) return KVSEL_OK;
  if (score == nullptr || idx == nullptr || idx_out == nullptr)
    return fail(KVSEL_ERR_NULL, "kvsel_order: score, idx and idx_out must be set");
  if (overlap(idx_out, G * k * 4, idx, G * k * 4))
    return fail(KVSEL_ERR_SHAPE, "kvsel_order: idx_out must not overlap idx");
  return launch_order(score, G, M, idx, k, descending != 0, idx_out, val_out, stream);
}

int kvsel_index_attn(const void* q, int64_t S, int64_t Hq, float scale, const void* k,
                     const void* v, kvsel_cache kc, const int32_t* pos, float* out, float* lse,
                     hipStream_t stream) {
  const char* what = "kvsel_index_attn";
  KVSEL_TRY(check_ptr(q, "q"));
  KVSEL_TRY(check_ptr(k, "k"));
  KVSEL_TRY(check_ptr(v, "v"));
  if (pos == nullptr) return fail(KVSEL_ERR_NULL, "pos is NULL");
  if (out == nullptr) return fail(KVSEL_ERR_NULL, "out is NULL");
  KVSEL_TRY(check_cache(kc, what));
  KVSEL_TRY(check_scale(scale, what));
  if (kc.dtype != KVSEL_BF16)
    return fail(KVSEL_ERR_UNSUPPORTED, "%s: bf16 caches only (matrix cores)", what);
  if (S < 1 || Hq < 1 || Hq % kc.H != 0 || Hq > 4096 || S >= (int64_t{1} << 31) / Hq)
    return fail(KVSEL_ERR_SHAPE, "%s: need S >= 1, Hq a multiple of H, S * Hq < 2^31", what);
  // 512 work-items per workgroup: the dispatch counts work-items in 32 bits
  if (index_attn_blocks(kc, S, Hq) >= (int64_t{1} << 23))
    return fail(KVSEL_ERR_SHAPE, "%s: too many rows for one launch", what);
  return launch_index_attn(q, S, Hq, scale, k, v, kc, pos, out, lse, stream);
}

int kvsel_unit_fractions(const int32_t* sel, int64_t G, int64_t k, int64_t unit_len,
                         int64_t M, float* r, hipStream_t stream) {
  // one work-item per (row, unit): G * M must fit the dispatch's 32-bit size
  if (G < 1 || k < 0 || k >= (int64_t{1} << 31) || unit_len < 1 || M < 1 ||
      M >= (int64_t{1} << 31) || G >= (int64_t{1} << 31) || G * M >= (int64_t{1} << 31) ||
      unit_len * M >= (int64_t{1} << 31))
    return fail(KVSEL_ERR_SHAPE, "kvsel_unit_fractions: G=%lld k=%lld unit_len=%lld M=%lld out of range",
                (long long)G, (long long)k, (long long)unit_len, (long long)M);
  if (r == nullptr) return fail(KVSEL_ERR_NULL, "r is NULL");
  if (k > 0 && sel == nullptr) return fail(KVSEL_ERR_NULL, "sel is NULL");
  if (k > 0 && overlap(r, G * M * 4, sel, G * k * 4))
    return fail(KVSEL_ERR_SHAPE, "kvsel_unit_fractions: r must not overlap sel");
  return launch_unit_fractions(sel, G, k, unit_len, M, r, stream);
}

int kvsel_slot_starts(const int32_t* order, int64_t G, int64_t M, int64_t unit_len, int64_t base,
                      int64_t rep, int64_t* delta, hipStream_t stream) {
  if (G < 1 || M < 1 || M >= (int64_t{1} << 31) || unit_len < 1 || rep < 1 || rep > 65536 ||
      G >= (int64_t{1} << 31) || G * M >= (int64_t{1} << 31) || base < 0 ||
      base + unit_len * M >= (int64_t{1} << 31))
    return fail(KVSEL_ERR_SHAPE, "kvsel_slot_starts: G=%lld M=%lld unit_len=%lld rep=%lld base=%lld out of range",
                (long long)G, (long long)M, (long long)unit_len, (long long)rep, (long long)base);
  if (order == nullptr || delta == nullptr)
    return fail(KVSEL_ERR_NULL, "kvsel_slot_starts: order and delta must be set");
  if (overlap(delta, G * rep * M * 8, order, G * M * 4))
    return fail(KVSEL_ERR_SHAPE, "kvsel_slot_starts: delta must not overlap order");
  return launch_slot_starts(order, G, M, unit_len, base, rep, delta, stream);
}

int kvsel_gather(const void* k_src, const void* v_src, kvsel_cache kc, int64_t unit_len,
                 const int32_t* idx, int64_t k, int64_t idx_group, const int64_t* src_start,
                 int64_t align_base, double rope_base, int32_t rope_style,
                 const void* k_proxy, const void* v_proxy, const kvsel_cache* proxy,
                 void* k_dst, void* v_dst, hipStream_t stream) {
  KVSEL_TRY(check_ptr(k_src, "k_src"));
  KVSEL_TRY(check_ptr(k_dst, "k_dst"));
  if ((v_src == nullptr) != (v_dst == nullptr))
    return fail(KVSEL_ERR_NULL, "kvsel_gather: v_src and v_dst must both be set or both NULL");
  if (v_src != nullptr) {
    KVSEL_TRY(check_ptr(v_src, "v_src"));
    KVSEL_TRY(check_ptr(v_dst, "v_dst"));
  }
  KVSEL_TRY(check_cache(kc, "kvsel_gather"));
  KVSEL_TRY(check_units(kc, unit_len, "kvsel_gather"));
  const int64_t M = kc.N / unit_len;
  if (k < 0 || k > M)
    return fail(KVSEL_ERR_SHAPE, "kvsel_gather: k=%lld not in [0, M=%lld]", (long long)k, (long long)M);
  if (idx_group < 1 || kc.B % idx_group != 0)
    return fail(KVSEL_ERR_SHAPE, "kvsel_gather: idx_group must divide B");
  if (k > 0 && idx == nullptr) return fail(KVSEL_ERR_NULL, "idx is NULL");
  if (align_base >= 0) {
    if (rope_style != KVSEL_ROPE_HALF && rope_style != KVSEL_ROPE_INTERLEAVED)
      return fail(KVSEL_ERR_SHAPE, "kvsel_gather: unknown rope_style %d", rope_style);
    if (!(rope_base > 1.0)) return fail(KVSEL_ERR_SHAPE, "kvsel_gather: rope_base must be > 1");
    if (align_base + (M + 1) * unit_len >= (int64_t{1} << 31))
      return fail(KVSEL_ERR_SHAPE, "kvsel_gather: aligned positions out of range");
  }
  int64_t dst_rows = k * unit_len;
  if (proxy != nullptr) {
    KVSEL_TRY(check_cache(*proxy, "kvsel_gather proxy"));
    KVSEL_TRY(check_ptr(k_proxy, "k_proxy"));
    if ((v_proxy == nullptr) != (v_src == nullptr))
      return fail(KVSEL_ERR_NULL, "kvsel_gather: v_proxy must be set exactly when v_src is");
    if (v_proxy != nullptr) KVSEL_TRY(check_ptr(v_proxy, "v_proxy"));
    if (proxy->B != kc.B || proxy->H != kc.H || proxy->D != kc.D || proxy->dtype != kc.dtype)
      return fail(KVSEL_ERR_SHAPE, "kvsel_gather: proxy cache must share B, H, D and dtype");
    if (proxy->N != M)
      return fail(KVSEL_ERR_SHAPE, "kvsel_gather: proxy has %lld entries, source has %lld units",
                  (long long)proxy->N, (long long)M);
    if (align_base >= 0)
      return fail(KVSEL_ERR_UNSUPPORTED, "kvsel_gather: re-positioning is not available in nested mode");
    dst_rows += proxy->N;
  }
  if (k > 0) {
    // the kept rows may live in pinned host memory (a host-resident cache)
    const void* ks = nullptr;
    const void* vs = nullptr;
    KVSEL_TRY(resolve_rows(k_src, &ks, "k_src"));
    if (v_src != nullptr) KVSEL_TRY(resolve_rows(v_src, &vs, "v_src"));
    KVSEL_TRY(launch_gather(ks, vs, kc, unit_len, idx, k, idx_group, src_start, align_base,
                            rope_base, rope_style, proxy != nullptr, dst_rows, k_dst, v_dst,
                            stream));
  }
  if (proxy != nullptr)
    return launch_proxy_copy(k_proxy, v_proxy, *proxy, unit_len, idx, k, idx_group, dst_rows,
                             k_dst, v_dst, stream);
  return KVSEL_OK;
}

size_t kvsel_decode_workspace(int64_t T, int64_t Hq, const kvsel_segment* segs, int32_t n_seg) {
  return decode_ws(T, Hq, segs, n_seg, false);
}

int kvsel_decode_attn(const void* q, int64_t T, int64_t Hq, float scale, const kvsel_segment* segs,
                      int32_t n_seg, float* out, float* lse, void* ws, size_t ws_bytes,
                      hipStream_t stream) {
  KVSEL_TRY(check_ptr(q, "q"));
  KVSEL_TRY(check_ptr(out, "out"));
  if (segs == nullptr) return fail(KVSEL_ERR_NULL, "segs is NULL");
  if (n_seg < 1 || n_seg > kMaxSegments)
    return fail(KVSEL_ERR_SHAPE, "kvsel_decode_attn: n_seg=%d not in [1, %d]", n_seg, kMaxSegments);
  const kvsel_cache& c0 = segs[0].kc;
  DecodeSeg ds[kMaxSegments];
  int64_t split = 0;
  for (int i = 0; i < n_seg; ++i) {
    const kvsel_cache& c = segs[i].kc;
    KVSEL_TRY(check_cache(c, "kvsel_decode_attn segment"));
    KVSEL_TRY(check_ptr(segs[i].k, "segment k"));
    KVSEL_TRY(check_ptr(segs[i].v, "segment v"));
    if (c.B != c0.B || c.H != c0.H || c.D != c0.D || c.dtype != c0.dtype)
      return fail(KVSEL_ERR_SHAPE, "kvsel_decode_attn: segments must share B, H, D and dtype");
    ds[i] = DecodeSeg{segs[i].k, segs[i].v, c.N, c.stride_b, c.stride_n, 0};
  }
  KVSEL_TRY(check_heads(T, Hq, c0, "kvsel_decode_attn"));
  KVSEL_TRY(check_scale(scale, "kvsel_decode_attn"));
  // splits of every segment, numbered across the segments (sizes validated)
  const int64_t split_len = split_len_of(T, Hq, c0, false, total_keys(segs, n_seg));
  for (int i = 0; i < n_seg; ++i) {
    ds[i].split_begin = split;
    split += (segs[i].kc.N + split_len - 1) / split_len;
  }
  const size_t need = kvsel_decode_workspace(T, Hq, segs, n_seg);
  if (ws == nullptr || ws_bytes < need)
    return fail(KVSEL_ERR_WORKSPACE, "kvsel_decode_attn: workspace %zu < %zu bytes", ws_bytes, need);
  KVSEL_TRY(check_ptr(ws, "ws"));
  float* ws_ms = static_cast<float*>(ws);
  float* ws_o = ws_ms + decode_ms_floats(c0.B * Hq * T, split);
  return launch_decode(q, T, Hq, scale, ds, n_seg, c0.B, c0.H, c0.D, c0.dtype, split, out, lse,
                       ws_ms, ws_o, stream);
}

size_t kvsel_gather_decode_workspace(int64_t T, int64_t Hq, kvsel_cache kc, int64_t unit_len,
                                     int64_t k, const kvsel_segment* extra, int32_t n_extra) {
  if (T < 1 || Hq < 1 || unit_len < 1 || k < 0 || n_extra < 0 || n_extra >= kMaxSegments ||
      (n_extra > 0 && extra == nullptr))
    return 0;
  kvsel_segment segs[kMaxSegments];
  int n = 0;
  for (int i = 0; i < n_extra; ++i) segs[n++] = extra[i];
  if (k > 0) {
    const int64_t rows = k * unit_len;
    segs[n++] = kvsel_segment{nullptr, nullptr,
                              kvsel_cache{kc.B, rows, kc.H, kc.D, rows * kc.H * kc.D,
                                          kc.H * kc.D, kc.dtype}};
  }
  if (n == 0) return 0;
  const bool fused = k > 0 && kc.H > 0 && decode_stream_ok(kc.dtype, kc.H, kc.D, (Hq / kc.H) * T);
  return decode_ws(T, Hq, segs, n, fused);
}

int kvsel_gather_decode(const void* q, int64_t T, int64_t Hq, float scale, const void* k_src,
                        const void* v_src, kvsel_cache kc, int64_t unit_len, const int32_t* idx,
                        int64_t k, int64_t idx_group, void* k_dst, void* v_dst,
                        const kvsel_segment* extra, int32_t n_extra, float* out, float* lse,
                        void* ws, size_t ws_bytes, hipStream_t stream) {
  KVSEL_TRY(check_ptr(q, "q"));
  KVSEL_TRY(check_ptr(k_src, "k_src"));
  KVSEL_TRY(check_ptr(v_src, "v_src"));
  if (k > 0) {  // an empty compact cache may have no storage
    KVSEL_TRY(check_ptr(k_dst, "k_dst"));
    KVSEL_TRY(check_ptr(v_dst, "v_dst"));
  }
  KVSEL_TRY(check_ptr(out, "out"));
  KVSEL_TRY(check_cache(kc, "kvsel_gather_decode"));
  KVSEL_TRY(check_units(kc, unit_len, "kvsel_gather_decode"));
  KVSEL_TRY(check_heads(T, Hq, kc, "kvsel_gather_decode"));
  KVSEL_TRY(check_scale(scale, "kvsel_gather_decode"));
  const int64_t M = kc.N / unit_len;
  if (k < 0 || k > M)
    return fail(KVSEL_ERR_SHAPE, "kvsel_gather_decode: k=%lld not in [0, M=%lld]", (long long)k,
                (long long)M);
  if (idx_group < 1 || kc.B % idx_group != 0)
    return fail(KVSEL_ERR_SHAPE, "kvsel_gather_decode: idx_group must divide B");
  if (k > 0 && idx == nullptr) return fail(KVSEL_ERR_NULL, "idx is NULL");
  if (n_extra < 0 || n_extra >= kMaxSegments)
    return fail(KVSEL_ERR_SHAPE, "kvsel_gather_decode: n_extra=%d not in [0, %d]", n_extra,
                kMaxSegments - 1);
  if (n_extra > 0 && extra == nullptr) return fail(KVSEL_ERR_NULL, "extra is NULL");
  if (k == 0 && n_extra == 0)
    return fail(KVSEL_ERR_SHAPE, "kvsel_gather_decode: nothing to attend (k = 0, no extra segment)");
  const int64_t rows = k * unit_len;
  kvsel_segment segs[kMaxSegments];
  int n = 0;
  for (int i = 0; i < n_extra; ++i) segs[n++] = extra[i];
  if (k > 0)
    segs[n++] = kvsel_segment{k_dst, v_dst,
                              kvsel_cache{kc.B, rows, kc.H, kc.D, rows * kc.H * kc.D,
                                          kc.H * kc.D, kc.dtype}};
  for (int i = 0; i < n_extra; ++i) {
    const kvsel_cache& c = extra[i].kc;
    KVSEL_TRY(check_cache(c, "kvsel_gather_decode extra segment"));
    KVSEL_TRY(check_ptr(extra[i].k, "extra segment k"));
    KVSEL_TRY(check_ptr(extra[i].v, "extra segment v"));
    if (c.B != kc.B || c.H != kc.H || c.D != kc.D || c.dtype != kc.dtype)
      return fail(KVSEL_ERR_SHAPE, "kvsel_gather_decode: segments must share B, H, D and dtype");
  }
  // one pass (each kept row read once, copied to the compact cache and
  // attended) where the streaming kernel applies; else a copy then a decode
  const bool fused = k > 0 && decode_stream_ok(kc.dtype, kc.H, kc.D, (Hq / kc.H) * T);
  const size_t need = decode_ws(T, Hq, segs, n, fused);
  if (ws == nullptr || ws_bytes < need)
    return fail(KVSEL_ERR_WORKSPACE, "kvsel_gather_decode: workspace %zu < %zu bytes", ws_bytes,
                need);
  KVSEL_TRY(check_ptr(ws, "ws"));
  if (k > 0) {  // the kept rows may live in pinned host memory
    KVSEL_TRY(resolve_rows(k_src, &k_src, "k_src"));
    KVSEL_TRY(resolve_rows(v_src, &v_src, "v_src"));
  }
  if (fused) {
    DecodeSeg ds[kMaxSegments];
    int64_t split = 0;
    const int64_t split_len = split_len_of(T, Hq, kc, true, total_keys(segs, n));
    for (int i = 0; i < n; ++i) {
      const bool g = i == n - 1;
      ds[i] = DecodeSeg{g ? k_src : segs[i].k, g ? v_src : segs[i].v, segs[i].kc.N,
                        g ? kc.stride_b : segs[i].kc.stride_b,
                        g ? kc.stride_n : segs[i].kc.stride_n, split};
      split += (segs[i].kc.N + split_len - 1) / split_len;
    }
    const DecodeGather gather{n - 1, idx, unit_len, k, idx_group, M, k_dst, v_dst};
    float* ws_ms = static_cast<float*>(ws);
    float* ws_o = ws_ms + decode_ms_floats(kc.B * Hq * T, split);
    return launch_decode(q, T, Hq, scale, ds, n, kc.B, kc.H, kc.D, kc.dtype, split, out, lse,
                         ws_ms, ws_o, stream, &gather);
  }
  if (k > 0)
    KVSEL_TRY(launch_gather(k_src, v_src, kc, unit_len, idx, k, idx_group, nullptr, -1, 0.0,
                            KVSEL_ROPE_HALF, 0, rows, k_dst, v_dst, stream));
  return kvsel_decode_attn(q, T, Hq, scale, segs, n, out, lse, ws, ws_bytes, stream);
}

}  // extern "C"
