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

// Padding of a staged row of an LDS key tile (kMfmaTileKeys keys): 16 bytes,
// so the 16 keys one B-fragment read spans land on distinct banks.
constexpr int kMfmaPad = 8;

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

}  // namespace kvsel
