// Fused chunk-parallel Falcon-1 forward on MFMA (gfx950), bf16 I/O,
// dk = dv = 64, chunk C = 64.
//
// One workgroup owns one (batch, head) sequence.  Its waves split into two
// roles that run concurrently and meet in a ring of LDS slots:
//
//  * three FACTOR waves, each building the state-independent factors of one
//    chunk at a time (chunks f, f + 3, f + 6, ...), entirely from registers:
//      a1  x_i = phi(k_{t0+i-1}), E_i = ||x_i||^2, eta_i (Eq. 3.4 with the
//          fresh-start sentinel), log gamma_i = log1p(-min(eta_i lam_i,
//          1 - eps_gamma)) (Section 4.3) and the chunk-local prefix g_i
//          (log-space renormalisation of Section 4.4 applied per chunk);
//      a2  the decayed strictly-lower Gram matrix
//          A_{i,s} = eta_i e^{g_{i-1}-g_s} (x_i . x_s), T = (I + A)^{-1} by
//          blocked forward substitution (16x16 diagonal blocks by column
//          elimination in registers, off-diagonal blocks on MFMA), the
//          factor W = T Diag(eta e^{g_{s-1}}) X ("one multi-RHS TriSolve per
//          chunk" of the WY form), the decayed read mask
//          M_{i,s} = e^{g_i-g_s} (q_i . x_s) (s <= i, read after write) and
//          the decayed keys (Diag(e^{g_63-g}) X)^T;
//  * four CHAIN waves, wave w owning value columns 16w..16w+15 of the
//    float32 state S for the whole sequence:
//      a2  U = T Diag(eta) V for its columns;
//      a3  R = U - W S (rows eta_i r_i), S <- e^{g_63} S + (Diag(e^{g_63-g}) X)^T R;
//      a4  O = Diag(e^g) Q S + M R, stored as bf16.
//
// A slot is handed over with LDS flags (release/acquire at workgroup scope):
// full[slot] = chunk index when its factors are written, consumed[slot]
// counts chain waves done with it.  Every wait is bounded.
//
// Every input byte is read from HBM once (the chain waves re-read Q and V
// tiles that the factor waves touched moments before, from L2) and every
// output byte is written once.
//
// MFMA operand convention.  v_mfma_f32_16x16x32_bf16 takes, in lane l, row
// (l & 15) of A and column (l & 15) of B with eight k-values each; the
// result holds column (l & 15), rows 4 (l >> 4) .. +3.  Every product here
// feeds lane group g = l >> 4 the k-values {4g..4g+3, 16+4g..16+4g+3} of a
// 32-wide k block (the same for A and B, so the sum is unchanged).  With
// that choice two stacked result tiles are exactly the operand fragment of
// the next product, which keeps S and R in registers, and a product with
// the identity turns token-major rows into the feature-major fragments that
// contract over tokens.

#include "falcon_device.h"
#include "falcon_launch.h"

namespace falcon {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kC = 64;            // chunk length
constexpr int kD = 64;            // dk = dv
constexpr int kP = 72;            // bf16 row pitch of T in LDS (elements)
constexpr int kNF = 3;            // factor waves
constexpr int kNS = 4;            // ring slots
constexpr int kThreads = 64 * (4 + kNF);
constexpr int kSpinLimit = 1 << 22;

// Factors of one chunk, as consumed by the chain waves.
struct Slot {
  uint16_t wf[4 * 2 * 64 * 8];    // -W, A fragments [ib][m][lane][8]
  uint16_t mf[4 * 2 * 64 * 8];    // M^T, B fragments [ib][m][lane][8]
  uint16_t xh[4 * 2 * 64 * 8];    // (Diag(e^{g_63-g}) X)^T, A fragments [fb][m][lane][8]
  uint16_t tb[kC * kP];           // T = (I + A)^{-1}, row-major
  float eta[kC];                  // eta_s, token order
  float gexp_t[kC];               // e^{g_i} at [c16 * 4 + ib] for i = 16 ib + c16
  float glast[4];                 // e^{g_63}
};

// Per factor wave: the chunk's gates in the orders its lanes read them, and
// the diagonal 16x16 blocks of A.
struct FactorPrivate {
  float abt[4][16][16];           // [b][s][i] = A[16b+i][16b+s]
  float graw[kC];                 // g_s, token order
  float sxg[kC];                  // eta_s e^{g_{s-1}}
  float sxh[kC];                  // e^{g_63 - g_s}
  float eta_t[kC];                // eta_i at [c16 * 4 + ib]
  float gprev_t[kC];              // g_{i-1} at [c16 * 4 + ib]
  float graw_t[kC];               // g_i at [c16 * 4 + ib]
};

struct Smem {
  Slot slot[kNS];
  FactorPrivate fp[kNF];
  int full[kNS];
  int consumed[kNS];
  int abort_flag;
};

__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(s16x4 a, s16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ uint16_t bf(float f) { return f32_to_bf16(f); }
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// k offset (within a 32-wide block) of fragment element e of lane group g.
__device__ __forceinline__ int kperm(int g, int e) { return e < 4 ? 4 * g + e : 12 + 4 * g + e; }

// Fragment of a bf16 row: k = kbase + kperm(g, 0..7).
__device__ __forceinline__ bf16x8 frag_lds(const uint16_t* row, int kbase, int g) {
  const uint2 a = *reinterpret_cast<const uint2*>(row + kbase + 4 * g);
  const uint2 b = *reinterpret_cast<const uint2*>(row + kbase + 16 + 4 * g);
  return __builtin_bit_cast(bf16x8, make_uint4(a.x, a.y, b.x, b.y));
}
// Same from global memory, or zeros when the row does not exist.
__device__ __forceinline__ bf16x8 frag_global(const bf16_t* row, int kbase, int g, bool valid) {
  uint2 a = make_uint2(0, 0), b = make_uint2(0, 0);
  if (valid) {
    a = *reinterpret_cast<const uint2*>(row + kbase + 4 * g);
    b = *reinterpret_cast<const uint2*>(row + kbase + 16 + 4 * g);
  }
  return __builtin_bit_cast(bf16x8, make_uint4(a.x, a.y, b.x, b.y));
}
// Two stacked result tiles (k rows 0-15 and 16-31 of a block), scaled, as a fragment.
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
__device__ __forceinline__ void store_half(uint16_t* p, f32x4 v) {
  const uint32_t a = uint32_t(bf(v[0])) | (uint32_t(bf(v[1])) << 16);
  const uint32_t b = uint32_t(bf(v[2])) | (uint32_t(bf(v[3])) << 16);
  *reinterpret_cast<uint2*>(p) = make_uint2(a, b);
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
// B fragment of the 32x16 selection matrix picking columns 16h..16h+15 of a
// 32-wide k block (a product with it transposes a tile into the result layout).
__device__ __forceinline__ bf16x8 identity_frag(int h, int g, int c16) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = static_cast<__bf16>(kperm(g, e) == 16 * h + c16 ? 1.0f : 0.0f);
  return r;
}

// Lane n of each 16-lane row, broadcast to the row (DPP row_newbcast).
template <int N>
__device__ __forceinline__ float row_bcast(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x150 + N, 0xf, 0xf, false));
}
// Value of lane l-n within the 16-lane row, 0 past the row start (DPP row_shr).
template <int N>
__device__ __forceinline__ float row_shr(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x110 + N, 0xf, 0xf, true));
}
__device__ __forceinline__ float lane_value(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}
// Column elimination for a unit lower-triangular 16x16 block: lane j holds
// column j of the strictly-lower part (col[i] = A[i][j]) and of the inverse
// (t[i]); step S subtracts A[i][S] t[S] from every row i > S, with A[i][S]
// broadcast from lane S.
template <int S>
__device__ __forceinline__ void eliminate(float (&t)[16], const float (&col)[16]) {
  if constexpr (S < 15) {
#pragma unroll
    for (int i = S + 1; i < 16; ++i) t[i] = fmaf(-row_bcast<S>(col[i]), t[S], t[i]);
    eliminate<S + 1>(t, col);
  }
}

__device__ __forceinline__ bool wait_at_least(int* flag, int target, int* abort_flag) {
  for (int it = 0; it < kSpinLimit; ++it) {
    const int v = __hip_atomic_load(flag, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (__builtin_amdgcn_readfirstlane(v) >= target) return true;
    if (__hip_atomic_load(abort_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) return false;
    __builtin_amdgcn_s_sleep(1);
  }
  __hip_atomic_store(abort_flag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  return false;
}

// Lower 16x16 tiles (ib >= sb) of a 64x64 matrix.
__device__ __forceinline__ void lower_tile(int n, int& ib, int& sb) {
  ib = n < 1 ? 0 : n < 3 ? 1 : n < 6 ? 2 : 3;
  sb = n - (ib * (ib + 1)) / 2;
}

struct Seq {
  const bf16_t* K;
  const bf16_t* Q;
  const bf16_t* V;
  const float* beta;
  const float* lam;
  const bf16_t* k_prev;
  int T;
};

// ---------------------------------------------------------------------------
// Factor wave: builds the slot of chunk c.
// ---------------------------------------------------------------------------
struct FactorLoads {
  bf16x8 x[4][2];   // X rows, fragments [row block][k step]
  bf16x8 q[4][2];   // Q rows
  float beta, lam;
};

__device__ __forceinline__ void factor_load(FactorLoads& L, const Seq& sq, int c, int l) {
  const int g = l >> 4, c16 = l & 15;
  const int t0 = c * kC;
#pragma unroll
  for (int ib = 0; ib < 4; ++ib) {
    const int tok = t0 + 16 * ib + c16;
    const int kt = tok - 1;                               // x_i = phi(k_{t-1})
    const bool xv = (kt >= 0 && kt < sq.T) || (kt == -1 && sq.k_prev);
    const bf16_t* xrow = kt >= 0 ? sq.K + int64_t(kt) * kD : sq.k_prev;
    const bool qv = tok < sq.T;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      L.x[ib][m] = frag_global(xrow, 32 * m, g, xv);
      L.q[ib][m] = frag_global(sq.Q + int64_t(tok) * kD, 32 * m, g, qv);
    }
  }
  const int tok = t0 + l;
  L.beta = tok < sq.T ? sq.beta[tok] : 0.0f;
  L.lam = tok < sq.T ? sq.lam[tok] : 0.0f;
}

__device__ void factor_chunk(Smem& sm, FactorLoads& L, const Seq& sq, int c, int fw, int l,
                             float eps, float eps_gamma, bool fresh, int nchunks) {
  const int g = l >> 4, c16 = l & 15;
  const int t0 = c * kC;
  Slot& S = sm.slot[c % kNS];
  FactorPrivate& P = sm.fp[fw];

  // ---- a1: energies, step sizes, chunk-local log decays -------------------
  float part[4];
#pragma unroll
  for (int ib = 0; ib < 4; ++ib) {
    float e = 0.f;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float xv = static_cast<float>(L.x[ib][m][k]);
        e = fmaf(xv, xv, e);
      }
    part[ib] = e;
  }
#pragma unroll
  for (int ib = 0; ib < 4; ++ib) part[ib] += __shfl_xor(part[ib], 16);
#pragma unroll
  for (int ib = 0; ib < 4; ++ib) part[ib] += __shfl_xor(part[ib], 32);
  const float energy = g == 0 ? part[0] : g == 1 ? part[1] : g == 2 ? part[2] : part[3];
  const int tok = t0 + l;                                  // this lane's row is l
  float eta = 0.f, lg = 0.f;
  if (tok < sq.T) {
    eta = nlms_eta(L.beta, energy, L.lam, eps, fresh && tok == 0);
    lg = clamped_log_gamma(eta, L.lam, eps_gamma);
  }
  // inclusive prefix over the 64 rows: within 16-lane rows by DPP shifts,
  // then the row totals carried across rows
  float gi = lg;
  gi += row_shr<1>(gi);
  gi += row_shr<2>(gi);
  gi += row_shr<4>(gi);
  gi += row_shr<8>(gi);
  {
    const float r0 = lane_value(gi, 15), r1 = lane_value(gi, 31), r2 = lane_value(gi, 47);
    gi += (g >= 1 ? r0 : 0.0f) + (g >= 2 ? r1 : 0.0f) + (g >= 3 ? r2 : 0.0f);
  }
  float gprev = row_shr<1>(gi);
  if (c16 == 0) {
    const float e15 = lane_value(gi, 15), e31 = lane_value(gi, 31), e47 = lane_value(gi, 47);
    gprev = g == 0 ? 0.0f : g == 1 ? e15 : g == 2 ? e31 : e47;
  }
  const float glast = lane_value(gi, 63);

  // Gates in the orders the lanes read them back.
  P.graw[l] = gi;
  P.sxg[l] = eta * __expf(gprev);
  P.sxh[l] = __expf(glast - gi);
  P.eta_t[c16 * 4 + g] = eta;
  P.gprev_t[c16 * 4 + g] = gprev;
  P.graw_t[c16 * 4 + g] = gi;
  // i-role values (i = 16 ib + c16) and s-role values (s = 16 sb + 4 g + r)
  const f32x4 eta_i = ld4(&P.eta_t[c16 * 4]);
  const f32x4 gpv_i = ld4(&P.gprev_t[c16 * 4]);
  const f32x4 gra_i = ld4(&P.graw_t[c16 * 4]);
  f32x4 gs_s[4];
#pragma unroll
  for (int sb = 0; sb < 4; ++sb) gs_s[sb] = ld4(&P.graw[16 * sb + 4 * g]);

  // ---- decayed Gram: A^T tile (sb, ib) = X_sb X_ib^T, scaled --------------
  // lane holds A[16ib+c16][16sb+4g+r]; diagonal tiles go to LDS for the
  // elimination, off-diagonal tiles stay in registers as MFMA operands.
  s16x4 a10, a32;        // A blocks (1,0) and (3,2) as K=16 A fragments
  bf16x8 a2lo, a3lo;     // A rows 32-47 / 48-63, columns 0-31, as K=32 A fragments
  {
    f32x4 a_off[6];
#pragma unroll
    for (int n = 0; n < 10; ++n) {
      int ib, sb;
      lower_tile(n, ib, sb);
      f32x4 acc = mfma32(L.x[sb][0], L.x[ib][0], zero4());
      acc = mfma32(L.x[sb][1], L.x[ib][1], acc);
      const int i = 16 * ib + c16;
      f32x4 a;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int s_ = 16 * sb + 4 * g + r;
        a[r] = s_ < i ? eta_i[ib] * __expf(gpv_i[ib] - gs_s[sb][r]) * acc[r] : 0.0f;
      }
      if (ib == sb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) P.abt[ib][4 * g + r][c16] = a[r];
      } else {
        a_off[n - ib] = a;       // n - ib enumerates the off-diagonal tiles in order
      }
    }
    a10 = s16_acc(a_off[0]);
    a32 = s16_acc(a_off[5]);
    a2lo = frag_acc(a_off[1], a_off[2]);
    a3lo = frag_acc(a_off[3], a_off[4]);
  }
  // ---- T = (I + A)^{-1}: diagonal blocks by column elimination -----------
  float t[16];
  {
    const int b = g, j = c16;
    float col[16];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const f32x4 v = ld4(&P.abt[b][j][4 * q4]);          // A[16b+i][16b+j], all i
      col[4 * q4] = v[0]; col[4 * q4 + 1] = v[1]; col[4 * q4 + 2] = v[2]; col[4 * q4 + 3] = v[3];
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) t[i] = (i == j) ? 1.0f : 0.0f;
    eliminate<0>(t, col);
  }

  // The slot may still be read by the chain for chunk c - kNS.
  if (!wait_at_least(&sm.consumed[c % kNS], 4 * (c / kNS), &sm.abort_flag)) return;

#pragma unroll
  for (int i = 0; i < 16; ++i) S.tb[(16 * g + i) * kP + 16 * g + c16] = bf(t[i]);
  S.eta[l] = eta;
  S.gexp_t[c16 * 4 + g] = __expf(gi);
  if (l == 0) S.glast[0] = __expf(glast);

  // ---- off-diagonal 16x16 blocks: T_hl = -T_hh A_hl T_ll for (1,0), (3,2)
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int lo = 2 * p, hi = 2 * p + 1;
    s16x4 tl;
#pragma unroll
    for (int e = 0; e < 4; ++e) tl[e] = static_cast<short>(S.tb[(16 * lo + 4 * g + e) * kP + 16 * lo + c16]);
    const f32x4 y = mfma16(p == 0 ? a10 : a32, tl, zero4());
    const s16x4 th = __builtin_bit_cast(
        s16x4, *reinterpret_cast<const uint2*>(&S.tb[(16 * hi + c16) * kP + 16 * hi + 4 * g]));
    const f32x4 z = mfma16(th, s16_acc(y), zero4());
#pragma unroll
    for (int r = 0; r < 4; ++r) S.tb[(16 * hi + 4 * g + r) * kP + 16 * lo + c16] = bf(-z[r]);
  }
  // ---- lower-left 32x32 block: T_21 = -T_22 A_21 T_11 (2x2 block sense) --
  {
    bf16x8 tlo[2];
#pragma unroll
    for (int cj = 0; cj < 2; ++cj)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        tlo[cj][e] = __builtin_bit_cast(__bf16, S.tb[kperm(g, e) * kP + 16 * cj + c16]);
    const bf16x8 th2 = frag_lds(&S.tb[(32 + c16) * kP], 32, g);
    const bf16x8 th3 = frag_lds(&S.tb[(48 + c16) * kP], 32, g);
#pragma unroll
    for (int cj = 0; cj < 2; ++cj) {
      const f32x4 y2 = mfma32(a2lo, tlo[cj], zero4());     // rows 32-47
      const f32x4 y3 = mfma32(a3lo, tlo[cj], zero4());     // rows 48-63
      const bf16x8 yb = frag_acc(y2, y3);
      const f32x4 z2 = mfma32(th2, yb, zero4());
      const f32x4 z3 = mfma32(th3, yb, zero4());
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        S.tb[(32 + 4 * g + r) * kP + 16 * cj + c16] = bf(-z2[r]);
        S.tb[(48 + 4 * g + r) * kP + 16 * cj + c16] = bf(-z3[r]);
      }
    }
  }
  // ---- decayed read mask: M^T tile (sb, ib) = X_sb Q_ib^T ----------------
#pragma unroll
  for (int n = 0; n < 10; ++n) {
    int ib, sb;
    lower_tile(n, ib, sb);
    f32x4 acc = mfma32(L.x[sb][0], L.q[ib][0], zero4());
    acc = mfma32(L.x[sb][1], L.q[ib][1], acc);
    const int i = 16 * ib + c16;
    f32x4 mv;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int s_ = 16 * sb + 4 * g + r;
      mv[r] = s_ <= i ? __expf(gra_i[ib] - gs_s[sb][r]) * acc[r] : 0.0f;
    }
    store_half(&S.mf[((ib * 2 + (sb >> 1)) * 64 + l) * 8 + 4 * (sb & 1)], mv);
  }

  // ---- decayed key transposes on the matrix cores ------------------------
  // D(sb, fb) = X_sb I_fb; lane holds X[16sb+4g+r][16fb+c16].
  bf16x8 xg[4][2];                                         // (Diag(eta e^{g_{s-1}}) X)^T
  {
    f32x4 sxg_s[4], sxh_s[4];
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) {
      sxg_s[sb] = ld4(&P.sxg[16 * sb + 4 * g]);
      sxh_s[sb] = ld4(&P.sxh[16 * sb + 4 * g]);
    }
    const bf16x8 id0 = identity_frag(0, g, c16), id1 = identity_frag(1, g, c16);
#pragma unroll
    for (int fb = 0; fb < 4; ++fb) {
      f32x4 d[4];
#pragma unroll
      for (int sb = 0; sb < 4; ++sb)
        d[sb] = mfma32(L.x[sb][fb >> 1], (fb & 1) ? id1 : id0, zero4());
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        xg[fb][m] = frag_acc(d[2 * m] * sxg_s[2 * m], d[2 * m + 1] * sxg_s[2 * m + 1]);
        store_frag(&S.xh[((fb * 2 + m) * 64 + l) * 8],
                   frag_acc(d[2 * m] * sxh_s[2 * m], d[2 * m + 1] * sxh_s[2 * m + 1]));
      }
    }
  }
  // The chunk's rows are no longer needed: prefetch this wave's next chunk.
  if (c + kNF < nchunks) factor_load(L, sq, c + kNF, l);

  // ---- W^T tiles (fb, ib) = (Diag(eta e^{g_{s-1}}) X)^T T^T; store -W ----
  {
    bf16x8 tf[4][2];
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) {
      tf[ib][0] = frag_lds(&S.tb[(16 * ib + c16) * kP], 0, g);
      tf[ib][1] = frag_lds(&S.tb[(16 * ib + c16) * kP], 32, g);
    }
#pragma unroll
    for (int ib = 0; ib < 4; ++ib)
#pragma unroll
      for (int fb = 0; fb < 4; ++fb) {
        f32x4 acc = mfma32(xg[fb][0], tf[ib][0], zero4());
        if (ib >= 2) acc = mfma32(xg[fb][1], tf[ib][1], acc);  // T is lower triangular
        store_half(&S.wf[((ib * 2 + (fb >> 1)) * 64 + l) * 8 + 4 * (fb & 1)], -acc);
      }
  }
  if (l == 0) __hip_atomic_store(&sm.full[c % kNS], c, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// ---------------------------------------------------------------------------
// Chain wave: consumes the slot of chunk c for value columns 16w..16w+15.
// ---------------------------------------------------------------------------
struct ChainLoads {
  bf16x8 v[4];      // V rows of the four row blocks, k block covering columns 16w..
  bf16x8 q[4][2];   // Q rows, fragments [row block][k step]
};

__device__ __forceinline__ void chain_load_v(ChainLoads& L, const Seq& sq, int c, int w, int l) {
  const int g = l >> 4, c16 = l & 15;
#pragma unroll
  for (int sb = 0; sb < 4; ++sb) {
    const int tok = c * kC + 16 * sb + c16;
    L.v[sb] = frag_global(sq.V + int64_t(tok) * kD, 32 * (w >> 1), g, tok < sq.T);
  }
}
__device__ __forceinline__ void chain_load_q(ChainLoads& L, const Seq& sq, int c, int l) {
  const int g = l >> 4, c16 = l & 15;
#pragma unroll
  for (int ib = 0; ib < 4; ++ib) {
    const int tok = c * kC + 16 * ib + c16;
#pragma unroll
    for (int m = 0; m < 2; ++m) L.q[ib][m] = frag_global(sq.Q + int64_t(tok) * kD, 32 * m, g, tok < sq.T);
  }
}

__device__ bool chain_chunk(Smem& sm, ChainLoads& L, f32x4 (&Sst)[4], const Seq& sq, int c, int w,
                            int l, bf16_t* o_bh, int nchunks) {
  const int g = l >> 4, c16 = l & 15;
  const int t0 = c * kC;
  if (!wait_at_least(&sm.full[c % kNS], c, &sm.abort_flag)) return false;
  const Slot& S = sm.slot[c % kNS];

  // ---- wait done; first batch of slot reads: T rows, eta and -W fragments.
  bf16x8 tf[4][2], wfr[4][2];
  f32x4 eta_s[4];
#pragma unroll
  for (int ib = 0; ib < 4; ++ib) {
    tf[ib][0] = frag_lds(&S.tb[(16 * ib + c16) * kP], 0, g);
    if (ib >= 2) tf[ib][1] = frag_lds(&S.tb[(16 * ib + c16) * kP], 32, g);
  }
#pragma unroll
  for (int sb = 0; sb < 4; ++sb) eta_s[sb] = ld4(&S.eta[16 * sb + 4 * g]);
#pragma unroll
  for (int ib = 0; ib < 4; ++ib)
#pragma unroll
    for (int m = 0; m < 2; ++m) wfr[ib][m] = load_frag(&S.wf[((ib * 2 + m) * 64 + l) * 8]);

  // ---- U = T Diag(eta) V for columns 16w..: transpose the V tile on the matrix
  // cores, scale rows by eta_s, then contract over tokens.
  bf16x8 vt[2];
  {
    const bf16x8 id = identity_frag(w & 1, g, c16);
    f32x4 d[4];
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) d[sb] = mfma32(L.v[sb], id, zero4());
#pragma unroll
    for (int m = 0; m < 2; ++m) vt[m] = frag_acc(d[2 * m] * eta_s[2 * m], d[2 * m + 1] * eta_s[2 * m + 1]);
  }
  if (c + 1 < nchunks) chain_load_v(L, sq, c + 1, w, l);
  // ---- R = U - W S (rows eta_i r_i of this column block)
  const bf16x8 sb0 = frag_acc(Sst[0], Sst[1]);
  const bf16x8 sb1 = frag_acc(Sst[2], Sst[3]);
  f32x4 R[4];
#pragma unroll
  for (int ib = 0; ib < 4; ++ib) {
    f32x4 u = mfma32(tf[ib][0], vt[0], zero4());
    if (ib >= 2) u = mfma32(tf[ib][1], vt[1], u);
    u = mfma32(wfr[ib][0], sb0, u);
    R[ib] = mfma32(wfr[ib][1], sb1, u);
  }
  // ---- second batch: mask and decayed-key fragments, output and decay scales.
  bf16x8 mfr[4][2], xhr[4][2];
#pragma unroll
  for (int ib = 0; ib < 4; ++ib) {
    mfr[ib][0] = load_frag(&S.mf[((ib * 2 + 0) * 64 + l) * 8]);
    if (ib >= 2) mfr[ib][1] = load_frag(&S.mf[((ib * 2 + 1) * 64 + l) * 8]);
  }
#pragma unroll
  for (int fb = 0; fb < 4; ++fb)
#pragma unroll
    for (int m = 0; m < 2; ++m) xhr[fb][m] = load_frag(&S.xh[((fb * 2 + m) * 64 + l) * 8]);
  const f32x4 gexp_i = ld4(&S.gexp_t[c16 * 4]);
  const float glast = S.glast[0];
  // All slot data is in registers: hand the slot back to the factor waves.
  if (l == 0) __hip_atomic_fetch_add(&sm.consumed[c % kNS], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);

  const bf16x8 rb0 = frag_acc(R[0], R[1]);
  const bf16x8 rb1 = frag_acc(R[2], R[3]);
  // ---- O^T tiles: e^{g_i} S^T Q^T + R^T M^T; lane holds o[t0+16ib+c16][16w+4g+r].
#pragma unroll
  for (int ib = 0; ib < 4; ++ib) {
    f32x4 acc = mfma32(sb0, L.q[ib][0], zero4());
    acc = mfma32(sb1, L.q[ib][1], acc);
    acc = acc * gexp_i[ib];
    acc = mfma32(rb0, mfr[ib][0], acc);
    if (ib >= 2) acc = mfma32(rb1, mfr[ib][1], acc);
    const int tok = t0 + 16 * ib + c16;
    if (tok < sq.T) {
      const uint32_t p0 = uint32_t(bf(acc[0])) | (uint32_t(bf(acc[1])) << 16);
      const uint32_t p1 = uint32_t(bf(acc[2])) | (uint32_t(bf(acc[3])) << 16);
      *reinterpret_cast<uint2*>(o_bh + int64_t(tok) * kD + 16 * w + 4 * g) = make_uint2(p0, p1);
    }
  }
  if (c + 1 < nchunks) chain_load_q(L, sq, c + 1, l);
  // ---- S <- e^{g_63} S + (Diag(e^{g_63-g}) X)^T R
#pragma unroll
  for (int fb = 0; fb < 4; ++fb) {
    f32x4 acc = Sst[fb] * glast;
    acc = mfma32(xhr[fb][0], rb0, acc);
    Sst[fb] = mfma32(xhr[fb][1], rb1, acc);
  }
  return true;
}

__global__ void __launch_bounds__(kThreads)
falcon1_chunked_mfma_kernel(const bf16_t* __restrict__ phi_k, const bf16_t* __restrict__ phi_q,
                            const bf16_t* __restrict__ v, const float* __restrict__ beta,
                            const float* __restrict__ lam, const float* S0,
                            const bf16_t* __restrict__ k_prev, bf16_t* __restrict__ o,
                            float* S_T, int T, float eps, float eps_gamma) {
  __shared__ Smem sm;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int l = tid & 63;
  const int g = l >> 4, c16 = l & 15;
  const int64_t bh = blockIdx.x;
  Seq sq;
  sq.K = phi_k + bh * T * kD;
  sq.Q = phi_q + bh * T * kD;
  sq.V = v + bh * T * kD;
  sq.beta = beta + bh * T;
  sq.lam = lam + bh * T;
  sq.k_prev = k_prev ? k_prev + bh * kD : nullptr;
  sq.T = T;
  const int nchunks = (T + kC - 1) / kC;

  // T's upper blocks and the structurally-zero halves of the mask fragments
  // are never written afterwards and stay zero.
  for (int s = 0; s < kNS; ++s) {
    for (int e = tid; e < kC * kP; e += kThreads) sm.slot[s].tb[e] = 0;
    for (int e = tid; e < 4 * 2 * 64 * 8; e += kThreads) sm.slot[s].mf[e] = 0;
  }
  if (tid < kNS) {
    sm.full[tid] = -1;
    sm.consumed[tid] = 0;
  }
  if (tid == 0) sm.abort_flag = 0;
  __syncthreads();

  if (wave < 4) {
    const int w = wave;
    f32x4 Sst[4];
#pragma unroll
    for (int fb = 0; fb < 4; ++fb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        Sst[fb][r] = S0 ? S0[(bh * kD + 16 * fb + 4 * g + r) * kD + 16 * w + c16] : 0.0f;
    ChainLoads L;
    chain_load_v(L, sq, 0, w, l);
    chain_load_q(L, sq, 0, l);
    for (int c = 0; c < nchunks; ++c)
      if (!chain_chunk(sm, L, Sst, sq, c, w, l, o + bh * T * kD, nchunks)) break;
    if (S_T) {
#pragma unroll
      for (int fb = 0; fb < 4; ++fb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          S_T[(bh * kD + 16 * fb + 4 * g + r) * kD + 16 * w + c16] = Sst[fb][r];
    }
  } else {
    const int fw = wave - 4;
    const bool fresh = (k_prev == nullptr);
    FactorLoads L;
    if (fw < nchunks) factor_load(L, sq, fw, l);
    for (int c = fw; c < nchunks; c += kNF) {
      factor_chunk(sm, L, sq, c, fw, l, eps, eps_gamma, fresh, nchunks);
      if (__hip_atomic_load(&sm.abort_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) break;
    }
  }
}

}  // namespace

bool chunked_mfma_applies(const ProblemArgs& a) {
  return a.bf16 && a.variant == kF1 && a.dk == kD && a.dv == kD && a.C == kC;
}

hipError_t launch_chunked_mfma(const ProblemArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(falcon1_chunked_mfma_kernel, dim3(a.B * a.H), dim3(kThreads), 0, st,
                     static_cast<const bf16_t*>(a.phi_k), static_cast<const bf16_t*>(a.phi_q),
                     static_cast<const bf16_t*>(a.v), a.beta, a.lam, a.S0,
                     static_cast<const bf16_t*>(a.k_prev), static_cast<bf16_t*>(a.o), a.S_T, a.T,
                     a.eps, a.eps_gamma);
  return hipGetLastError();
}

}  // namespace falcon
