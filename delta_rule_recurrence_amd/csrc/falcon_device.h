// Device-side helpers shared by the Falcon kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace falcon {

// Compile-time variant tags (values match falcon_variant in falcon.h).
enum Variant : int { kF1 = 1, kF1A = 2, kF2 = 3, kF2A = 4 };

__host__ __device__ constexpr bool is_regression(int v) { return v == kF1 || v == kF2; }
__host__ __device__ constexpr bool is_per_column(int v) { return v == kF2 || v == kF2A; }

// ---- bf16 <-> f32 ---------------------------------------------------------
// bf16 is stored as its 16-bit pattern.  Widening is exact; narrowing is
// round-to-nearest-even via the hardware conversion.
struct bf16_t { uint16_t bits; };

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 h = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, h);
}

// Typed element access for the two I/O dtypes.
template <typename T> struct io;
template <> struct io<float> {
  __device__ __forceinline__ static float load(const float* p, int64_t i) { return p[i]; }
  __device__ __forceinline__ static void store(float* p, int64_t i, float x) { p[i] = x; }
};
template <> struct io<bf16_t> {
  __device__ __forceinline__ static float load(const bf16_t* p, int64_t i) {
    return bf16_to_f32(p[i].bits);
  }
  __device__ __forceinline__ static void store(bf16_t* p, int64_t i, float x) {
    p[i].bits = f32_to_bf16(x);
  }
};

// ---- step size and decay ----------------------------------------------------
// eta_t = beta_t / (E_t + lam_t + eps), eta := 0 when the denominator is 0
// or at the fresh-start sentinel (Eq. 3.4 and the Section 3 conventions).
__device__ __forceinline__ float nlms_eta(float beta, float energy, float lam, float eps,
                                          bool sentinel) {
  const float denom = energy + lam + eps;
  return (sentinel || denom == 0.0f) ? 0.0f : beta / denom;
}
// gamma = 1 - min(eta lam, 1 - eps_gamma) (Section 4.3 "Decay positivity"),
// formed as max(1 - eta lam, eps_gamma): the same number, but a binding
// clamp yields eps_gamma itself, where 1 minus the float nearest 1 - eps_gamma
// would be off by up to 5 % at eps_gamma = 1e-6 (1 - alpha is exact for
// alpha in [0.5, 2]).
__device__ __forceinline__ float clamped_gamma(float eta, float lam, float eps_gamma) {
  return fmaxf(1.0f - eta * lam, eps_gamma);
}
// log gamma in float32: log1p(-alpha), or log eps_gamma where the clamp binds
// (Section 4.3).
__device__ __forceinline__ float clamped_log_gamma(float eta, float lam, float eps_gamma) {
  const float a = eta * lam;
  return 1.0f - a >= eps_gamma ? log1pf(-a) : logf(eps_gamma);
}

}  // namespace falcon
