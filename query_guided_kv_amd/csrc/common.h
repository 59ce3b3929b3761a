// Device helpers shared by the kvsel kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvsel.h"

namespace kvsel {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

using bf16_t = uint16_t;  // raw bfloat16 bit pattern

// ---------------------------------------------------------------------------
// bf16 <-> fp32
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef __bf16 bf16x2_hw_t __attribute__((ext_vector_type(2)));

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f));
}
// Two fp32 values -> a packed bf16 pair (lo, hi), one instruction.
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
  const bf16x2_hw_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// Element access for the two cache dtypes.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int kPerVec = 4;  // elements per 16-byte vector
  __device__ static __forceinline__ float load(const float* p) { return *p; }
  __device__ static __forceinline__ float to_f32(float x) { return x; }
  __device__ static __forceinline__ float from_f32(float x) { return x; }
};
template <> struct Elem<bf16_t> {
  static constexpr int kPerVec = 8;
  __device__ static __forceinline__ float load(const bf16_t* p) { return bf16_to_f32(*p); }
  __device__ static __forceinline__ float to_f32(bf16_t x) { return bf16_to_f32(x); }
  __device__ static __forceinline__ bf16_t from_f32(float x) { return f32_to_bf16(x); }
};

// 16-byte vector unpacked to fp32 / packed from fp32.
template <typename T>
__device__ __forceinline__ void unpack16(const uint4& raw, float* out) {
  if constexpr (sizeof(T) == 4) {
    out[0] = __uint_as_float(raw.x); out[1] = __uint_as_float(raw.y);
    out[2] = __uint_as_float(raw.z); out[3] = __uint_as_float(raw.w);
  } else {
    out[0] = bf16_lo(raw.x); out[1] = bf16_hi(raw.x);
    out[2] = bf16_lo(raw.y); out[3] = bf16_hi(raw.y);
    out[4] = bf16_lo(raw.z); out[5] = bf16_hi(raw.z);
    out[6] = bf16_lo(raw.w); out[7] = bf16_hi(raw.w);
  }
}
template <typename T>
__device__ __forceinline__ uint4 pack16(const float* in) {
  uint4 r;
  if constexpr (sizeof(T) == 4) {
    r.x = __float_as_uint(in[0]); r.y = __float_as_uint(in[1]);
    r.z = __float_as_uint(in[2]); r.w = __float_as_uint(in[3]);
  } else {
    r.x = pack2_bf16(in[0], in[1]);
    r.y = pack2_bf16(in[2], in[3]);
    r.z = pack2_bf16(in[4], in[5]);
    r.w = pack2_bf16(in[6], in[7]);
  }
  return r;
}

// Load n contiguous elements (n * sizeof(T) a multiple of 16, 16-byte aligned)
// as fp32.
template <typename T, int n>
__device__ __forceinline__ void load_f32(const T* p, float* out) {
  constexpr int V = Elem<T>::kPerVec;
  static_assert(n % V == 0, "slice must be whole 16-byte vectors");
#pragma unroll
  for (int i = 0; i < n / V; ++i) unpack16<T>(reinterpret_cast<const uint4*>(p)[i], out + i * V);
}

// ---------------------------------------------------------------------------
// Cross-lane reductions inside groups of W consecutive lanes (W | 64).
// DPP for W <= 16 (quad permutes and row mirrors), LDS crossbar beyond.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float dpp_xor1(float x) {
  return __builtin_amdgcn_update_dpp(0.0f, x, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
}
__device__ __forceinline__ float dpp_xor2(float x) {
  return __builtin_amdgcn_update_dpp(0.0f, x, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
}
__device__ __forceinline__ float dpp_half_mirror(float x) {
  return __builtin_amdgcn_update_dpp(0.0f, x, 0x141, 0xF, 0xF, false);  // lane i <- lane 7-i (per 8)
}
__device__ __forceinline__ float dpp_mirror(float x) {
  return __builtin_amdgcn_update_dpp(0.0f, x, 0x140, 0xF, 0xF, false);  // lane i <- lane 15-i (per 16)
}

// Sum over groups of W lanes; every lane of a group gets the group's sum.
template <int W>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(W == 1 || W == 2 || W == 4 || W == 8 || W == 16 || W == 32 || W == 64, "W");
  if constexpr (W >= 2) x += dpp_xor1(x);
  if constexpr (W >= 4) x += dpp_xor2(x);
  if constexpr (W >= 8) x += dpp_half_mirror(x);
  if constexpr (W >= 16) x += dpp_mirror(x);
  if constexpr (W >= 32) x += __shfl_xor(x, 16, 64);
  if constexpr (W >= 64) x += __shfl_xor(x, 32, 64);
  return x;
}
template <int W>
__device__ __forceinline__ float group_max(float x) {
  if constexpr (W >= 2) x = fmaxf(x, dpp_xor1(x));
  if constexpr (W >= 4) x = fmaxf(x, dpp_xor2(x));
  if constexpr (W >= 8) x = fmaxf(x, dpp_half_mirror(x));
  if constexpr (W >= 16) x = fmaxf(x, dpp_mirror(x));
  if constexpr (W >= 32) x = fmaxf(x, __shfl_xor(x, 16, 64));
  if constexpr (W >= 64) x = fmaxf(x, __shfl_xor(x, 32, 64));
  return x;
}

// Merge of two softmax partials (m, s) in the log2 domain: s = sum 2^(l - m).
__device__ __forceinline__ void merge_ms(float& m, float& s, float m2, float s2) {
  const float mn = fmaxf(m, m2);
  const float ref = mn == -INFINITY ? 0.0f : mn;  // both empty: stays (-inf, 0), no branch
  s = s * exp2f(m - ref) + s2 * exp2f(m2 - ref);
  m = mn;
}

// ---------------------------------------------------------------------------
// RoPE: per-pair cos/sin of delta * theta_i in fp64, theta_i = base^(-2i/D)
// (the table comes from the host, RopeTheta).  The 2x2 rotation is also done
// in fp64 and rounded once to the cache dtype, so a re-positioned key is the
// correctly rounded rotation of the stored one.
// ---------------------------------------------------------------------------
__device__ __forceinline__ double2 rope_cs(int64_t delta, double theta) {
  const double ang = static_cast<double>(delta) * theta;
  double s, c;
  sincos(ang, &s, &c);
  return make_double2(c, s);
}

// fp64 -> bf16 with one rounding to nearest even.  The hardware fp64 -> fp32
// conversion rounds to nearest; rounding that fp32 value to bf16 gives the
// correctly rounded result unless it landed exactly halfway between two bf16
// values while the fp64 value did not (every bf16 midpoint is an fp32 value,
// and any other fp32 value lies on the same side of the midpoints as x).  In
// that case the fp32 value moves one ulp toward x, which fixes the direction.
__device__ __forceinline__ float f64_to_bf16_ready(double x) {
  const float t = static_cast<float>(x);
  const uint32_t u = __float_as_uint(t);
  const double back = static_cast<double>(t);
  const bool fix = ((u & 0xffffu) == 0x8000u) & (back != x);
  const uint32_t step = fabs(x) > fabs(back) ? 1u : 0xffffffffu;
  return __uint_as_float(fix ? u + step : u);
}
__device__ __forceinline__ bf16_t f64_to_bf16(double x) {
  return f32_to_bf16(f64_to_bf16_ready(x));
}

template <typename T>
__device__ __forceinline__ uint4 pack16_f64(const double* in) {
  uint4 r;
  if constexpr (sizeof(T) == 4) {
    r.x = __float_as_uint(__double2float_rn(in[0])); r.y = __float_as_uint(__double2float_rn(in[1]));
    r.z = __float_as_uint(__double2float_rn(in[2])); r.w = __float_as_uint(__double2float_rn(in[3]));
  } else {
    // round to fp32 first; only a value that landed exactly on a bf16
    // midpoint (probability ~2^-16) needs the one-ulp fix of f64_to_bf16_ready
    float t[8];
    bool tie = false;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      t[e] = static_cast<float>(in[e]);
      tie |= (__float_as_uint(t[e]) & 0xffffu) == 0x8000u;
    }
    if (tie) {
#pragma unroll
      for (int e = 0; e < 8; ++e) t[e] = f64_to_bf16_ready(in[e]);
    }
    r.x = pack2_bf16(t[0], t[1]);
    r.y = pack2_bf16(t[2], t[3]);
    r.z = pack2_bf16(t[4], t[5]);
    r.w = pack2_bf16(t[6], t[7]);
  }
  return r;
}

// Rotate 16-byte vectors of a key row.  Half-split pairing: `ra` holds dims
// [d0, d0 + V) and `rb` the partner dims [d0 + D/2, ...); interleaved: `ra`
// holds V/2 whole pairs starting at dim d0 and `rb` is unused.  cs_at(e)
// gives the cos/sin of the pair that element e of `ra` belongs to (from an
// LDS table or from registers).
template <typename T, int STYLE, typename CsAt>
__device__ __forceinline__ void rope_rotate16_with(uint4& ra, uint4& rb, CsAt cs_at) {
  constexpr int V = Elem<T>::kPerVec;
  float a[V];
  double oa[V];
  unpack16<T>(ra, a);
  if constexpr (STYLE == KVSEL_ROPE_HALF) {
    float b[V];
    double ob[V];
    unpack16<T>(rb, b);
#pragma unroll
    for (int e = 0; e < V; ++e) {
      const double2 t = cs_at(e);
      const double x = a[e], y = b[e];
      oa[e] = fma(x, t.x, -y * t.y);
      ob[e] = fma(x, t.y, y * t.x);
    }
    rb = pack16_f64<T>(ob);
  } else {
#pragma unroll
    for (int e = 0; e < V; e += 2) {
      const double2 t = cs_at(e);
      const double x = a[e], y = a[e + 1];
      oa[e] = fma(x, t.x, -y * t.y);
      oa[e + 1] = fma(x, t.y, y * t.x);
    }
  }
  ra = pack16_f64<T>(oa);
}

// cs_at(e) = cos/sin of the pair of element e of the vector that starts at
// dimension d0: cs[d0 + e] (half-split) or cs[(d0 + e) / 2] (interleaved).
template <typename T, int STYLE>
__device__ __forceinline__ void rope_rotate16(uint4& ra, uint4& rb, int d0, const double2* cs) {
  if constexpr (STYLE == KVSEL_ROPE_HALF)
    rope_rotate16_with<T, STYLE>(ra, rb, [&](int e) { return cs[d0 + e]; });
  else
    rope_rotate16_with<T, STYLE>(ra, rb, [&](int e) { return cs[(d0 + e) >> 1]; });
}

// Record a launch failure; returns KVSEL_OK or KVSEL_ERR_HIP.
int check_launch(const char* what);
void set_error(const char* fmt, ...);

}  // namespace kvsel
