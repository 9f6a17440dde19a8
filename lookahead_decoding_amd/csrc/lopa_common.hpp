// Internal helpers shared by liblopa's kernels and entry points.
// gfx950 (CDNA4) only: wave64, MFMA bf16 with float32 accumulation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lopa.h"

namespace lopa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

// bf16 bit pattern -> float (exact).
__device__ __forceinline__ float bf16_bits_to_f32(unsigned short u) {
  return __uint_as_float(static_cast<unsigned>(u) << 16);
}

// float -> bf16 bit pattern, round to nearest, ties to even (finite inputs;
// NaN maps to a quiet NaN).
__device__ __forceinline__ unsigned short f32_to_bf16_bits(float f) {
  unsigned u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<unsigned short>(u >> 16);
}

template <typename T> struct Act;
template <> struct Act<float> {
  static __device__ __forceinline__ float load(const float* p, size_t i) { return p[i]; }
  static __device__ __forceinline__ void store(float* p, size_t i, float v) { p[i] = v; }
};
template <> struct Act<unsigned short> {
  static __device__ __forceinline__ float load(const unsigned short* p, size_t i) {
    return bf16_bits_to_f32(p[i]);
  }
  static __device__ __forceinline__ void store(unsigned short* p, size_t i, float v) {
    p[i] = f32_to_bf16_bits(v);
  }
};

// (max, index) pair ordering used by every argmax here: larger value wins,
// the lower index wins an exact tie.
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Online-softmax partial over a set of logits l: m = max l, s = sum
// exp(l - m), i = lowest index attaining m, t = sum exp(l - m) (l - m) (the
// entropy of softmax(l) is ln s - t / s).  The empty partial has s == 0.
struct Partial {
  float m;
  float s;
  int i;
  float t;
};

__device__ __forceinline__ Partial empty_partial() {
  return Partial{-INFINITY, 0.f, 0x7fffffff, 0.f};
}

// Merge of two partials over disjoint index sets; exact in (m, i), and the
// sums are rescaled to the larger max: with c = exp(m' - M),
// e^(l - M) = c e^(l - m') and (l - M) = (l - m') + (m' - M), so
// t -> c (t + (m' - M) s).
__device__ __forceinline__ Partial merge(Partial a, Partial b) {
  if (b.s == 0.f) return a;
  if (a.s == 0.f) return b;
  Partial r;
  if (better(b.m, b.i, a.m, a.i)) {
    r.m = b.m;
    r.i = b.i;
  } else {
    r.m = a.m;
    r.i = a.i;
  }
  const float da = a.m - r.m, db = b.m - r.m;
  const float ca = exp2f(da * kLog2e), cb = exp2f(db * kLog2e);
  r.s = a.s * ca + b.s * cb;
  r.t = ca * fmaf(da, a.s, a.t) + cb * fmaf(db, b.s, b.t);
  return r;
}

// Partial of the sampling LM head over the scaled logits z = l / T: m = max
// z, s = sum exp(z - m); (g, i, z_i) = the largest perturbed score z + G
// (Gumbel noise G), its index (lowest on a tie) and the scaled logit there.
// The empty partial has s == 0.
struct SPartial {
  float m;
  float s;
  int i;
  float g;
  float z;
};

__device__ __forceinline__ SPartial empty_spartial() {
  return SPartial{-INFINITY, 0.f, 0x7fffffff, -INFINITY, 0.f};
}

__device__ __forceinline__ SPartial merge(SPartial a, SPartial b) {
  if (b.s == 0.f) return a;
  if (a.s == 0.f) return b;
  SPartial r;
  r.m = fmaxf(a.m, b.m);
  r.s = a.s * exp2f((a.m - r.m) * kLog2e) + b.s * exp2f((b.m - r.m) * kLog2e);
  const bool tb = better(b.g, b.i, a.g, a.i);
  r.g = tb ? b.g : a.g;
  r.i = tb ? b.i : a.i;
  r.z = tb ? b.z : a.z;
  return r;
}

// Rows listed for the LM head, from the device-side branch count; both are
// clamped to the sizes the launch was planned for.
__device__ __forceinline__ int listed_rows(const int32_t* row_ptr, const int32_t* nb_ptr,
                                           int nb_max, int m_max) {
  int nb = *nb_ptr;
  nb = nb < 0 ? 0 : (nb > nb_max ? nb_max : nb);
  const int M = row_ptr[nb];
  return M < 0 ? 0 : (M > m_max ? m_max : M);
}

__device__ __forceinline__ SPartial shfl_xor(SPartial p, int o) {
  SPartial q;
  q.m = __shfl_xor(p.m, o, kWave);
  q.s = __shfl_xor(p.s, o, kWave);
  q.i = __shfl_xor(p.i, o, kWave);
  q.g = __shfl_xor(p.g, o, kWave);
  q.z = __shfl_xor(p.z, o, kWave);
  return q;
}

__device__ __forceinline__ Partial shfl_xor(Partial p, int o) {
  Partial q;
  q.m = __shfl_xor(p.m, o, kWave);
  q.s = __shfl_xor(p.s, o, kWave);
  q.i = __shfl_xor(p.i, o, kWave);
  q.t = __shfl_xor(p.t, o, kWave);
  return q;
}

}  // namespace lopa

// Host-side helpers
#define LOPA_LAUNCH_CHECK()                                   \
  do {                                                        \
    if (hipGetLastError() != hipSuccess) return LOPA_ERR_HIP; \
  } while (0)

int lopa_check_dims(const lopa_dims* d);   // defined in api.hip
