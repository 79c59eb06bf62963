// MFMA fragment helpers shared by the chunked kernels (gfx950, bf16 operands,
// float32 accumulation, 64-wide wavefronts).
//
// v_mfma_f32_16x16x32_bf16 takes, in lane l, row (l & 15) of A and column
// (l & 15) of B with eight k-values each; the result holds column (l & 15),
// rows 4 (l >> 4) .. +3.  "Contiguous" fragments give lane group g = l >> 4
// the k-values 8g..8g+7 of a 32-wide block (one 16-byte read of a row);
// "result-compatible" fragments give it {4g..4g+3, 16+4g..16+4g+3}, so two
// stacked result tiles are exactly the next operand fragment.  A and B
// always use the same order, so every sum is unchanged.
//
// Staged rows: 64 rows of 64 bf16 (128 bytes), the 16-byte segment q of row r
// stored at position q ^ ((r >> 1) & 7), which makes reads of 16 consecutive
// rows at one segment conflict-free.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "falcon_device.h"

namespace falcon {
namespace frag {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kRowElems = 64;     // elements per staged row

__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(s16x4 a, s16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ uint16_t bf(float f) { return f32_to_bf16(f); }
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// k offset (within a 32-wide block) of element e of lane group g in the
// result-compatible order.
__device__ __forceinline__ int kperm(int g, int e) { return e < 4 ? 4 * g + e : 12 + 4 * g + e; }

__device__ __forceinline__ int seg_pos(int r, int q) { return q ^ ((r & 15) >> 1); }

// Contiguous-order fragment: k = 32m + 8g .. +7 of row r of a ring matrix.
__device__ __forceinline__ bf16x8 ring_frag_c(const uint16_t* mat, int r, int m, int g) {
  const uint4 v = *reinterpret_cast<const uint4*>(mat + r * kRowElems + 8 * seg_pos(r, 4 * m + g));
  return __builtin_bit_cast(bf16x8, v);
}
// Result-compatible fragment: k = 32m + kperm(g, 0..7) of row r of a ring matrix.
__device__ __forceinline__ bf16x8 ring_frag_p(const uint16_t* mat, int r, int m, int g) {
  const int off = 4 * (g & 1);
  const uint2 a = *reinterpret_cast<const uint2*>(mat + r * kRowElems + 8 * seg_pos(r, 4 * m + (g >> 1)) + off);
  const uint2 b = *reinterpret_cast<const uint2*>(mat + r * kRowElems + 8 * seg_pos(r, 4 * m + 2 + (g >> 1)) + off);
  return __builtin_bit_cast(bf16x8, make_uint4(a.x, a.y, b.x, b.y));
}
// Result-compatible fragment of a bf16 row in a padded row-major array.
__device__ __forceinline__ bf16x8 frag_lds(const uint16_t* row, int kbase, int g) {
  const uint2 a = *reinterpret_cast<const uint2*>(row + kbase + 4 * g);
  const uint2 b = *reinterpret_cast<const uint2*>(row + kbase + 16 + 4 * g);
  return __builtin_bit_cast(bf16x8, make_uint4(a.x, a.y, b.x, b.y));
}
// Two stacked result tiles (k rows 0-15 and 16-31 of a block) as a fragment.
__device__ __forceinline__ bf16x8 frag_acc(f32x4 lo, f32x4 hi) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r[e] = static_cast<__bf16>(lo[e]);
    r[e + 4] = static_cast<__bf16>(hi[e]);
  }
  return r;
}
__device__ __forceinline__ bf16x8 load_frag(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}
__device__ __forceinline__ void store_frag(uint16_t* p, bf16x8 v) {
  *reinterpret_cast<uint4*>(p) = __builtin_bit_cast(uint4, v);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2 h = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, h);
}
__device__ __forceinline__ void store_half(uint16_t* p, f32x4 v) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
}
__device__ __forceinline__ f32x4 load_half(const uint16_t* p) {
  const uint2 v = *reinterpret_cast<const uint2*>(p);
  return f32x4{__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
               __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u)};
}
__device__ __forceinline__ s16x4 s16_acc(f32x4 v) {
  s16x4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = static_cast<short>(bf(v[e]));
  return r;
}
__device__ __forceinline__ f32x4 ld4(const float* p) {
  const float4 v = *reinterpret_cast<const float4*>(p);
  return f32x4{v.x, v.y, v.z, v.w};
}
// Contiguous-order B fragment of the selection matrix picking columns
// 16h..16h+15 of a 32-wide block (a product with it transposes a tile).
__device__ __forceinline__ bf16x8 select_frag(int h, int g, int c16) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = static_cast<__bf16>(8 * g + e == 16 * h + c16 ? 1.0f : 0.0f);
  return r;
}

// Value of lane l-n within the 16-lane row, 0 past the row start (DPP row_shr).
template <int N>
__device__ __forceinline__ float row_shr(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x110 + N, 0xf, 0xf, true));
}
__device__ __forceinline__ float lane_value(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}
// Lower 16x16 tiles (ib >= sb) of a 64x64 matrix, n = 0..9.
__device__ __forceinline__ void lower_tile(int n, int& ib, int& sb) {
  ib = n < 1 ? 0 : n < 3 ? 1 : n < 6 ? 2 : 3;
  sb = n - (ib * (ib + 1)) / 2;
}

// log gamma = log1p(-alpha), alpha = min(eta lam, 1 - eps_gamma) (Section
// 4.3), in float32 as ln(u) (-alpha) / (u - 1) with u = 1 - alpha rounded: the
// ratio cancels the rounding of u (Kahan's compensated log1p), so small alpha
// keeps its relative accuracy; ln is the hardware log2 times ln 2, and the
// division a hardware reciprocal (a few ulp in all).
__device__ __forceinline__ float fast_log_gamma(float eta, float lam, float eps_gamma) {
  // a binding clamp takes u = eps_gamma exactly and alpha = 1 - u, so that
  // the ratio below is 1 and the result log eps_gamma
  const float a = eta * lam;
  const bool unclamped = 1.0f - a >= eps_gamma;
  const float u = unclamped ? 1.0f - a : eps_gamma;
  const float alpha = unclamped ? a : 1.0f - u;
  const float d = u - 1.0f;
  return d == 0.0f ? -alpha
                   : __builtin_amdgcn_logf(u) * 0.6931471805599453f * (-alpha * __builtin_amdgcn_rcpf(d));
}

// Gates of one 64-token chunk (a1) from the staged key rows xs (64 swizzled
// rows in LDS) and the gates beta, lam of token `tok` = chunk start + l.
// Returns, for row l: eta_l (Eq. 3.4; 0 at the fresh start and past the
// sequence), the chunk-local inclusive prefix g_l of the clamped log decays
// (Section 4.3, "Decay positivity"; Section 4.4 log-space renormalisation
// applied per chunk), g_{l-1} (0 for l = 0) and g_63.
__device__ __forceinline__ void chunk_gates(const uint16_t* xs, float beta, float lam, int tok, int T,
                                            float eps, float eps_gamma, bool fresh, int l, float& eta,
                                            float& gi, float& gprev, float& glast) {
  const int g = l >> 4, c16 = l & 15;
  // energy of row l: lane l reads its own row (eight 16-byte segments)
  float energy = 0.f;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const bf16x8 v = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(xs + l * kRowElems + 8 * seg_pos(l, q)));
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const bf16x2 xv = {v[2 * k], v[2 * k + 1]};
      energy = __builtin_amdgcn_fdot2_f32_bf16(xv, xv, energy, false);
    }
  }
  // Eq. 3.4 with the hardware reciprocal; 0 at the fresh start, for a zero
  // denominator and past the sequence
  const float den = energy + lam + eps;
  const bool on = tok < T && !(fresh && tok == 0) && den != 0.0f;
  eta = on ? beta * __builtin_amdgcn_rcpf(den) : 0.0f;
  const float lg = tok < T ? fast_log_gamma(eta, lam, eps_gamma) : 0.0f;
  // inclusive prefix over the 64 rows: DPP shifts within 16-lane rows, then
  // the row totals carried across rows
  gi = lg;
  gi += row_shr<1>(gi);
  gi += row_shr<2>(gi);
  gi += row_shr<4>(gi);
  gi += row_shr<8>(gi);
  {
    const float r0 = lane_value(gi, 15), r1 = lane_value(gi, 31), r2 = lane_value(gi, 47);
    gi += (g >= 1 ? r0 : 0.0f) + (g >= 2 ? r1 : 0.0f) + (g >= 3 ? r2 : 0.0f);
  }
  gprev = row_shr<1>(gi);
  {
    const float e15 = lane_value(gi, 15), e31 = lane_value(gi, 31), e47 = lane_value(gi, 47);
    if (c16 == 0) gprev = g == 0 ? 0.0f : g == 1 ? e15 : g == 2 ? e31 : e47;
  }
  glast = lane_value(gi, 63);
}

// Column elimination for a unit lower-triangular 16x16 block: lane j holds
// column j of the negated strictly-lower part (ncol[i] = -A[i][j]) and of
// the inverse (t[i]).  Step S adds -A[i][S] t[S] to every row i > S, the
// factor broadcast from lane S of the 16-lane row by the multiply-add's own
// DPP source modifier (row_newbcast).  Each statement starts with two wait
// states, which covers the DPP read-after-VALU-write hazard on its sources.
#define FALCON_FMAC(D, A, S) "v_fmac_f32_dpp %" #D ", %" #A ", %" #S
#define FALCON_BCAST(N) " row_newbcast:" #N " row_mask:0xf bank_mask:0xf\n\t"
#define ELIM4(S, I)                                                                     \
  asm volatile("s_nop 1\n\t" FALCON_FMAC(0, 4, 8) FALCON_BCAST(S) FALCON_FMAC(1, 5, 8)   \
               FALCON_BCAST(S) FALCON_FMAC(2, 6, 8) FALCON_BCAST(S) FALCON_FMAC(3, 7, 8)   \
               FALCON_BCAST(S)                                                          \
               : "+v"(t[I]), "+v"(t[I + 1]), "+v"(t[I + 2]), "+v"(t[I + 3])              \
               : "v"(ncol[I]), "v"(ncol[I + 1]), "v"(ncol[I + 2]), "v"(ncol[I + 3]), "v"(t[S]))
#define ELIM3(S, I)                                                                     \
  asm volatile("s_nop 1\n\t" FALCON_FMAC(0, 3, 6) FALCON_BCAST(S) FALCON_FMAC(1, 4, 6)   \
               FALCON_BCAST(S) FALCON_FMAC(2, 5, 6) FALCON_BCAST(S)                      \
               : "+v"(t[I]), "+v"(t[I + 1]), "+v"(t[I + 2])                              \
               : "v"(ncol[I]), "v"(ncol[I + 1]), "v"(ncol[I + 2]), "v"(t[S]))
#define ELIM2(S, I)                                                                     \
  asm volatile("s_nop 1\n\t" FALCON_FMAC(0, 2, 4) FALCON_BCAST(S) FALCON_FMAC(1, 3, 4)   \
               FALCON_BCAST(S)                                                          \
               : "+v"(t[I]), "+v"(t[I + 1])                                             \
               : "v"(ncol[I]), "v"(ncol[I + 1]), "v"(t[S]))
#define ELIM1(S, I)                                                                     \
  asm volatile("s_nop 1\n\t" FALCON_FMAC(0, 1, 2) FALCON_BCAST(S)                        \
               : "+v"(t[I]) : "v"(ncol[I]), "v"(t[S]))

__device__ __forceinline__ void eliminate16(float (&t)[16], const float (&ncol)[16]) {
  ELIM4(0, 1); ELIM4(0, 5); ELIM4(0, 9); ELIM3(0, 13);
  ELIM4(1, 2); ELIM4(1, 6); ELIM4(1, 10); ELIM2(1, 14);
  ELIM4(2, 3); ELIM4(2, 7); ELIM4(2, 11); ELIM1(2, 15);
  ELIM4(3, 4); ELIM4(3, 8); ELIM4(3, 12);
  ELIM4(4, 5); ELIM4(4, 9); ELIM3(4, 13);
  ELIM4(5, 6); ELIM4(5, 10); ELIM2(5, 14);
  ELIM4(6, 7); ELIM4(6, 11); ELIM1(6, 15);
  ELIM4(7, 8); ELIM4(7, 12);
  ELIM4(8, 9); ELIM3(8, 13);
  ELIM4(9, 10); ELIM2(9, 14);
  ELIM4(10, 11); ELIM1(10, 15);
  ELIM4(11, 12);
  ELIM3(12, 13);
  ELIM2(13, 14);
  ELIM1(14, 15);
}
#undef ELIM4
#undef ELIM3
#undef ELIM2
#undef ELIM1
#undef FALCON_BCAST
#undef FALCON_FMAC

}  // namespace frag
}  // namespace falcon
