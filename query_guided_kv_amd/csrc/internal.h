// Host-side launchers behind the C ABI.  Arguments are validated by api.cpp
// before any of these is called; each returns KVSEL_OK or KVSEL_ERR_HIP.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kvsel.h"

namespace kvsel {

// Maximum segments of one decode call.
constexpr int kMaxSegments = 4;
// Rows of one score / aggregate tile partial when unit_len == 1.
constexpr int kTokenTile = 256;
// Keys per LDS tile of the MFMA kernels (4 key blocks of 16).
constexpr int kMfmaTileKeys = 64;
// Keys per split of the final attention pass (streaming and tile variants;
// decode_split_len gives the length a call actually uses).
constexpr int kDecodeSplit = 512;

// The RoPE frequencies theta_i = base^(-2i/D), i < D/2, formed once per call
// on the host in fp64 (the C library's pow) and passed to the kernels by value,
// so that no workgroup spends its start on a pow chain.
struct RopeTheta {
  double t[64];
};
RopeTheta rope_theta(double base, int64_t D);

int launch_reposition(const void* k_in, void* k_out, const kvsel_cache& kc, int64_t unit_len,
                      const int64_t* delta, int per_instance, double base, int style,
                      hipStream_t s);

// Segment partials of the query block: for every row (b, h, j) and segment of
// `seg_len` cached rows, (m, s) with m the max logit in log2 units and
// s = sum 2^(l2 - m).  Written to ms[((b*Hq + h)*T + j)*nseg + seg][2].
// When `natural` is set, m is converted to natural-log units on output (the
// layout of kvsel_score's `part`).
int launch_score_partials(const void* q, int64_t T, int64_t Hq, const void* k,
                          const kvsel_cache& kc, float scale, int64_t seg_len, float* ms,
                          int natural, hipStream_t s);

// Matrix-core variant of launch_score_partials (bf16, >= 16 query rows per kv
// head, segments a multiple of 64 cached rows); score_mfma_ok tells whether it
// applies.
bool score_mfma_ok(int dtype, int64_t rows_per_kv, int64_t seg_len);
void launch_score_mfma(const void* q, int64_t T, int64_t Hq, const void* k,
                       const kvsel_cache& kc, float scale2, int64_t seg_len, int64_t nseg,
                       float* ms, int natural, hipStream_t s);
// Same, scoring the keys re-positioned on the fly (units of rot_len rows, a
// multiple of 64, rotated by delta[u]); k_out (or NULL) receives them.
bool score_mfma_rot_ok(int dtype, int64_t rows_per_kv, int64_t seg_len, int64_t rot_len);
void launch_score_mfma_rot(const void* q, int64_t T, int64_t Hq, const void* k, void* k_out,
                           const kvsel_cache& kc, float scale, int64_t seg_len, int64_t nseg,
                           float* ms, int natural, int64_t rot_len, const int64_t* delta,
                           int per_instance, double base, int style, hipStream_t s);

// Scored rows of instance b listed by unit: virtual row t is row
// units[b * n_units + t / unit_len] * unit_len + t % unit_len of the source
// cache (entries outside [0, n_src) take no part in the softmax).
struct UnitMap {
  const int32_t* units;
  int64_t n_units;
  int64_t unit_len;
  int64_t n_src;
};
// MFMA scorer over the listed units of `kc` (kc.N is the source length);
// `delta` (NULL: no rotation) re-positions virtual unit u by delta[u] (or
// delta[b][u] with per_instance).
void launch_score_mfma_units(const void* q, int64_t T, int64_t Hq, const void* k,
                             const kvsel_cache& kc, const UnitMap& map, float scale,
                             int64_t seg_len, int64_t nseg, float* ms, int natural,
                             const int64_t* delta, int per_instance, double base, int style,
                             hipStream_t s);

// Row statistics from segment partials (log2 or natural units as written).
int launch_rowstats(const float* ms, int64_t rows, int64_t nseg, int natural, float* row_max,
                    float* row_sum, hipStream_t s);

// Chunk path: unit_score[g][u] from natural-unit partials and row stats.
// `ws` holds aggregate_chunk_ws_floats(B, Hq, T, M) floats of row-chunk sums.
// True where the chunk path derives the row statistics inside its own
// launch (row_max = row_sum = NULL to launch_aggregate_chunks).
bool aggregate_chunks_derive(int64_t M);
int launch_aggregate_chunks(const float* part, const float* row_max, const float* row_sum,
                            int64_t B, int64_t Hq, int64_t T, int64_t M, int64_t group,
                            float* unit_score, int accumulate, float* ws, hipStream_t s);
size_t aggregate_chunk_ws_floats(int64_t B, int64_t Hq, int64_t T, int64_t M);

// Token path: per_token[b][t] = sum_h sum_j alpha (* ||v||), then per unit/group sums.
// Small caches split the (kv head, row pass) items of the matrix-core variant
// over aggregate_token_parts() workgroup groups; each group writes its own
// per-token partials (parts arrays of B * N floats, summed by the unit sums in
// a fixed order).  Parts stay 1 unless B * N < kAggSplitRows, and never exceed
// kAggMaxParts.
constexpr int64_t kAggSplitRows = int64_t{1} << 19;
constexpr int64_t kAggMaxParts = 16;
int64_t aggregate_token_parts(const kvsel_cache& kc, int64_t Hq, int64_t T);
int launch_aggregate_tokens(const void* q, int64_t T, int64_t Hq, const void* k, const void* v,
                            const kvsel_cache& kc, float scale, const float* row_max,
                            const float* row_sum, int vnorm, float* per_token, hipStream_t s);
// Matrix-core variant of launch_aggregate_tokens (bf16, >= 16 query rows per
// kv head); aggregate_mfma_ok tells whether it applies.
bool aggregate_mfma_ok(int dtype, int64_t rows_per_kv);
int64_t aggregate_mfma_parts(const kvsel_cache& kc, int64_t rows_per_kv);
void launch_aggregate_mfma(const void* q, int64_t T, int64_t Hq, const void* k, const void* v,
                           const kvsel_cache& kc, float scale2, const float* row_max,
                           const float* row_sum, int vnorm, float* per_token, hipStream_t s);
int launch_unit_sums(const float* per_token, int64_t parts, int64_t B, int64_t N,
                     int64_t unit_len, int64_t group, float* unit_score, int accumulate,
                     hipStream_t s);

int launch_topk(const float* score, int64_t G, int64_t M, int64_t k, int32_t* idx, float* val,
                hipStream_t s);
int launch_take(const int32_t* src, int64_t G, int64_t m, const int32_t* idx, int64_t k,
                int32_t* out, hipStream_t s);
int launch_order(const float* score, int64_t G, int64_t M, const int32_t* idx, int64_t k,
                 int descending, int32_t* idx_out, float* val_out, hipStream_t s);
// index-based causal attention (index_attn.hip): workgroups of the launch,
// and the launch
int64_t index_attn_blocks(const kvsel_cache& kc, int64_t S, int64_t Hq);
int launch_index_attn(const void* q, int64_t S, int64_t Hq, float scale, const void* k,
                      const void* v, const kvsel_cache& kc, const int32_t* pos, float* out,
                      float* lse, hipStream_t s);
int launch_unit_fractions(const int32_t* sel, int64_t G, int64_t k, int64_t unit_len, int64_t M,
                          float* r, hipStream_t s);
int launch_slot_starts(const int32_t* order, int64_t G, int64_t M, int64_t unit_len, int64_t base,
                       int64_t rep, int64_t* delta, hipStream_t s);

int launch_gather(const void* k_src, const void* v_src, const kvsel_cache& kc, int64_t unit_len,
                  const int32_t* idx, int64_t k, int64_t idx_group, const int64_t* src_start,
                  int64_t align_base, double base, int style, int nested, int64_t dst_rows,
                  void* k_dst, void* v_dst, hipStream_t s);
int launch_proxy_copy(const void* k_proxy, const void* v_proxy, const kvsel_cache& proxy,
                      int64_t unit_len, const int32_t* idx, int64_t k, int64_t idx_group,
                      int64_t dst_rows, void* k_dst, void* v_dst, hipStream_t s);

struct DecodeSeg {
  const void* k;
  const void* v;
  int64_t N;
  int64_t stride_b;
  int64_t stride_n;
  int64_t split_begin;  // index of this segment's first split
};
// Segment `seg` of a decode call read through a kept-unit index list: its row t
// is source row idx[b / idx_group][t / unit_len] * unit_len + t % unit_len, and
// the kernel also copies it to row t of the compact cache (k_dst, v_dst,
// [B][n_kept * unit_len][H][D]).  Streaming variant only.
struct DecodeGather {
  int seg;
  const int32_t* idx;
  int64_t unit_len;
  int64_t n_kept;
  int64_t idx_group;
  int64_t n_units;
  void* k_dst;
  void* v_dst;
};
// Keys per split of a decode launch over n_keys keys (all segments) of B
// instances; the workspace query and the launch use the same value.
int64_t decode_split_len(int dtype, int64_t H, int64_t D, int64_t rows_per_kv, bool gathered,
                         int64_t B, int64_t n_keys);
int launch_decode(const void* q, int64_t T, int64_t Hq, float scale, const DecodeSeg* segs,
                  int n_seg, int64_t B, int64_t H, int64_t D, int dtype, int64_t n_split,
                  float* out, float* lse, float* ws_ms, float* ws_o, hipStream_t s,
                  const DecodeGather* gather = nullptr);

// Which score / decode path a shape takes (exposed for tests and docs).
bool stream_path_ok(int dtype, int64_t H, int64_t D, int64_t rows_per_kv);
// the streaming decode (and the one-pass refill + decode): bf16, head dim 128,
// <= 8 kv heads (a power of two), 1 .. 8 query rows per kv head
bool decode_stream_ok(int dtype, int64_t H, int64_t D, int64_t rows_per_kv);
// Rows per kv head from which a plain (not gathering) pass runs on the matrix cores.
constexpr int64_t kDecodeMfmaRows = 5;
bool decode_uses_stream(int dtype, int64_t H, int64_t D, int64_t rows_per_kv, bool gathered);

}  // namespace kvsel
