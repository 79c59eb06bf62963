// Chunked forward of the per-column rules (Falcon-2 and Falcon-2A) on gfx950,
// bf16 I/O, dk = dv = 64, chunk C = 64.
//
// Falcon-2 gives every value column j its own NLMS step size
// eta_{t,j} = beta_{t,j} / (||x_t||^2 + lam_t + eps) and decay
// gamma_{t,j} = 1 - min(eta_{t,j} lam_t, 1 - eps_gamma) (Section 4.2, Eq. 4.7,
// and the clamp of Section 4.3), so column j of S follows the scalar rule on
// its own.  Within a chunk with incoming state S, per column j (g_{i,j} the
// chunk-local prefix of log gamma):
//   rho_{i,j} + sum_{s<i} eta_{i,j} e^{g_{i-1,j}-g_{s,j}} (x_i.x_s) rho_{s,j}
//        = eta_{i,j} (v_{i,j} - e^{g_{i-1,j}} (X S)_{i,j})
// (the merged residual system of Section 4.2; rho_{i,j} = eta_{i,j} v_{i,j}
// for the additive Falcon-2A), and
//   o_{i,j} = e^{g_{i,j}} (Q S)_{i,j} + sum_{s<=i} e^{g_{i,j}-g_{s,j}} (q_i.x_s) rho_{s,j}
//   S'_{:,j} = e^{g_{63,j}} S_{:,j} + sum_s e^{g_{63,j}-g_{s,j}} x_s rho_{s,j}.
// The decays differ per column, so the triangular system is solved per
// column on the vector ALUs: with u_s = e^{g_{i-1}-g_s} rho_s carried from
// row to row (u_s <- gamma_i u_s after row i), every coefficient is a plain
// product and no exponential is evaluated; all factors are <= 1.  The
// products that are shared by all columns (x_i.x_s, q_i.x_s, X S, Q S and the
// state update) run on the matrix cores.
//
// One workgroup (one wave) per (batch, head, 16-column slice); four lanes per
// column split every row's sums (s = 4k + lane % 4) and combine them with
// DPP quad reductions.

#include "falcon_device.h"
#include "falcon_launch.h"
#include "falcon_mfma_frag.h"

namespace falcon {

namespace {

using namespace frag;

constexpr int kC = 64;
constexpr int kD = 64;
constexpr int kSlice = 16;

struct PcSmem {
  uint16_t x[kC * kD];            // keys phi(k_{t0+r-1}), swizzled rows
  uint16_t q[kC * kD];            // queries, swizzled rows
  float kq[kC][4][16];            // x_i.x_s at [i][s % 4][s / 4] for s < i, else 0
  float pq[kC][4][16];            // q_i.x_s at [i][s % 4][s / 4] for s <= i, else 0
  // per row i and column j: first {v, beta, (X S), (Q S)}, then, in place,
  // {rhs a, eta, gamma, e^{g_i} (Q S)}, and after the rows o_{i,j} in .x
  f32x4 rp[kC][kSlice];
  float en[kC];                   // ||x_i||^2
  float lm[kC];                   // lam_i
  uint16_t ut[kSlice][kC];        // e^{g_63-g_s} rho_s per column, bf16, [j][s]
  float e63[kSlice];              // e^{g_63} per column
};

__device__ __forceinline__ float quad_sum(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xf, 0xf, true));  // [1,0,3,2]
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xf, 0xf, true));  // [2,3,0,1]
  return v;
}

// Row I of one chunk for the lane's column (unrolled by recursion, so every
// bound and register index is a compile-time constant; the loop body reads
// LDS only, so the compiler is free to fetch later rows early).  On entry
// u[k] holds e^{g_{I-1}-g_s} rho_s for s = 4k + qq < I, on exit
// e^{g_I-g_s} rho_s for s <= I.  Row I's output is kept by the lane that owns
// s = I, in ov[I / 4].
template <bool kReg, int I>
__device__ __forceinline__ void solve_rows(const PcSmem& sm, int jc, int qq, float (&u)[16], float (&ov)[16]) {
  if constexpr (I < kC) {
    const f32x4 p = sm.rp[I][jc];                  // a_I, eta_I, gamma_I, e^{g_I} (Q S)_I
    float rho = p[0];
    if constexpr (kReg) {
      float dk = 0.f;
#pragma unroll
      for (int k = 0; 4 * k < I; ++k) dk = fmaf(sm.kq[I][qq][k], u[k], dk);
      rho = fmaf(-p[1], quad_sum(dk), rho);
    }
#pragma unroll
    for (int k = 0; 4 * k < I; ++k) u[k] *= p[2];
    const bool own = qq == (I & 3);
    if (own) u[I >> 2] = rho;
    float dp = 0.f;
#pragma unroll
    for (int k = 0; 4 * k <= I; ++k) dp = fmaf(sm.pq[I][qq][k], u[k], dp);
    dp = quad_sum(dp);
    if (own) ov[I >> 2] = p[3] + dp;
    solve_rows<kReg, I + 1>(sm, jc, qq, u, ov);
  }
}

// Inclusive product over the 64 lanes of a wave (DPP shifts within 16-lane
// rows, then the row totals carried across rows).
__device__ __forceinline__ float lane_prefix_product(float v, int g) {
#pragma unroll
  for (int sh = 1; sh < 16; sh <<= 1) {
    float w;
    switch (sh) {
      case 1: w = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, 1.0f), __builtin_bit_cast(int, v), 0x111, 0xf, 0xf, false)); break;
      case 2: w = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, 1.0f), __builtin_bit_cast(int, v), 0x112, 0xf, 0xf, false)); break;
      case 4: w = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, 1.0f), __builtin_bit_cast(int, v), 0x114, 0xf, 0xf, false)); break;
      default: w = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, 1.0f), __builtin_bit_cast(int, v), 0x118, 0xf, 0xf, false)); break;
    }
    v *= w;
  }
  const float r0 = lane_value(v, 15), r1 = lane_value(v, 31), r2 = lane_value(v, 47);
  return v * (g >= 1 ? r0 : 1.0f) * (g >= 2 ? r1 : 1.0f) * (g >= 3 ? r2 : 1.0f);
}

template <bool kReg>
__global__ void __launch_bounds__(64)
falcon2_chunked_kernel(const bf16_t* __restrict__ phi_k, const bf16_t* __restrict__ phi_q,
                       const bf16_t* __restrict__ v, const float* __restrict__ beta,
                       const float* __restrict__ lam, const float* S0,
                       const bf16_t* __restrict__ k_prev, bf16_t* __restrict__ o, float* S_T, int T,
                       float eps, float eps_gamma) {
  __shared__ PcSmem sm;
  const int l = threadIdx.x;
  const int g = l >> 4, c16 = l & 15;
  const int jc = l >> 2, qq = l & 3;              // recurrence layout: column jc, sub-lane qq
  const int64_t bh = blockIdx.x >> 2;
  const int j0 = (blockIdx.x & 3) * kSlice;
  const bool fresh = (k_prev == nullptr);
  const bf16_t* K = phi_k + bh * T * kD;
  const bf16_t* Q = phi_q + bh * T * kD;
  const bf16_t* V = v + bh * T * kD;
  const float* Bt = beta + bh * T * kD;
  const float* Lm = lam + bh * T;
  const bf16_t* kp = k_prev ? k_prev + bh * kD : nullptr;

  // upper parts of the Gram buffers are never written and stay zero
  for (int e = l; e < kC * 4 * 16; e += 64) {
    (&sm.kq[0][0][0])[e] = 0.f;
    (&sm.pq[0][0][0])[e] = 0.f;
  }
  // S[fb]: lane holds S[16fb+4g+r][j0+c16]
  f32x4 S[4];
#pragma unroll
  for (int fb = 0; fb < 4; ++fb)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      S[fb][r] = S0 ? S0[(bh * kD + 16 * fb + 4 * g + r) * kD + j0 + c16] : 0.0f;

  const int nchunks = (T + kC - 1) / kC;
  for (int c = 0; c < nchunks; ++c) {
    const int t0 = c * kC;
    // ---- stage: rows of keys and queries, this slice's values and gains --
    {
      bf16x8 xr[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int r = 8 * j + (l >> 3);
        const int kt = t0 + r - 1;
        const bf16_t* xsrc = kt < 0 ? (kp ? kp : K) : K + int64_t(kt < T ? kt : T - 1) * kD;
        const int tok = t0 + r < T ? t0 + r : T - 1;
        xr[j] = *reinterpret_cast<const bf16x8*>(xsrc + 8 * (l & 7));
        const bf16x8 qr = *reinterpret_cast<const bf16x8*>(Q + int64_t(tok) * kD + 8 * (l & 7));
        const int off = r * kD + 8 * seg_pos(r, l & 7);
        *reinterpret_cast<bf16x8*>(sm.x + off) = xr[j];
        *reinterpret_cast<bf16x8*>(sm.q + off) = qr;
      }
      // energies of rows 8 (l & 7) + (l >> 3) by a butterfly over 8 lanes
      float p[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float e = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const bf16x2 xv = {xr[j][2 * k], xr[j][2 * k + 1]};
          e = __builtin_amdgcn_fdot2_f32_bf16(xv, xv, e, false);
        }
        p[j] = e;
      }
      float q4[4], q2[2];
      {
        const bool b = (l & 4) != 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) q4[k] = (b ? p[k + 4] : p[k]) + __shfl_xor(b ? p[k] : p[k + 4], 4);
      }
      {
        const bool b = (l & 2) != 0;
#pragma unroll
        for (int k = 0; k < 2; ++k) q2[k] = (b ? q4[k + 2] : q4[k]) + __shfl_xor(b ? q4[k] : q4[k + 2], 2);
      }
      {
        const bool b = (l & 1) != 0;
        sm.en[8 * (l & 7) + (l >> 3)] = (b ? q2[1] : q2[0]) + __shfl_xor(b ? q2[0] : q2[1], 1);
      }
      const int tok = t0 + l < T ? t0 + l : T - 1;
      sm.lm[l] = Lm[tok];
      const bf16x8 va = *reinterpret_cast<const bf16x8*>(V + int64_t(tok) * kD + j0);
      const bf16x8 vb = *reinterpret_cast<const bf16x8*>(V + int64_t(tok) * kD + j0 + 8);
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const f32x4 bt = *reinterpret_cast<const f32x4*>(Bt + int64_t(tok) * kD + j0 + 4 * e4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = 4 * e4 + e;
          sm.rp[l][j][0] = static_cast<float>(j < 8 ? va[j] : vb[j - 8]);
          sm.rp[l][j][1] = bt[e];
        }
      }
    }
    // ---- shared products on the matrix cores -----------------------------
    // Gram and read tiles (ib, sb), sb <= ib: lane holds rows i = 16ib+4g+r,
    // column s = 16sb+c16
#pragma unroll
    for (int n = 0; n < 10; ++n) {
      int ib, sb;
      lower_tile(n, ib, sb);
      const bf16x8 xs0 = ring_frag_c(sm.x, 16 * sb + c16, 0, g), xs1 = ring_frag_c(sm.x, 16 * sb + c16, 1, g);
      f32x4 dk = zero4(), dp = zero4();
      if (kReg) {
        dk = mfma32(ring_frag_c(sm.x, 16 * ib + c16, 0, g), xs0, dk);
        dk = mfma32(ring_frag_c(sm.x, 16 * ib + c16, 1, g), xs1, dk);
      }
      dp = mfma32(ring_frag_c(sm.q, 16 * ib + c16, 0, g), xs0, dp);
      dp = mfma32(ring_frag_c(sm.q, 16 * ib + c16, 1, g), xs1, dp);
      const int s = 16 * sb + c16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * ib + 4 * g + r;
        if (kReg) sm.kq[i][s & 3][s >> 2] = s < i ? dk[r] : 0.0f;
        sm.pq[i][s & 3][s >> 2] = s <= i ? dp[r] : 0.0f;
      }
    }
    // X S and Q S for this slice: lane holds rows 16ib+4g+r, column j0+c16
    {
      const bf16x8 s0 = frag_acc(S[0], S[1]);
      const bf16x8 s1 = frag_acc(S[2], S[3]);
#pragma unroll
      for (int ib = 0; ib < 4; ++ib) {
        const int i = 16 * ib + c16;
        f32x4 aq = mfma32(ring_frag_p(sm.q, i, 0, g), s0, zero4());
        aq = mfma32(ring_frag_p(sm.q, i, 1, g), s1, aq);
        f32x4 ax = zero4();
        if (kReg) {
          ax = mfma32(ring_frag_p(sm.x, i, 0, g), s0, ax);
          ax = mfma32(ring_frag_p(sm.x, i, 1, g), s1, ax);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          sm.rp[16 * ib + 4 * g + r][c16][3] = aq[r];
          if (kReg) sm.rp[16 * ib + 4 * g + r][c16][2] = ax[r];
        }
      }
    }
    // ---- per row and column: step sizes, decays, right-hand sides ---------
    // lane l owns row i = l; e^{g_{i,j}} is the product of the row decays
    {
      const int t = t0 + l;
      const bool live = t < T;
      const float en = sm.en[l], lmi = sm.lm[l];
      const float den = en + lmi + eps;
      const float inv = (live && !(fresh && t == 0) && den != 0.0f) ? 1.0f / den : 0.0f;
#pragma unroll 4
      for (int j = 0; j < kSlice; ++j) {
        const f32x4 in = sm.rp[l][j];                // v, beta, (X S), (Q S)
        const float eta = in[1] * inv;
        const float gam = live ? clamped_gamma(eta, lmi, eps_gamma) : 1.0f;
        const float e_inc = lane_prefix_product(gam, g);
        float e_exc = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
            __builtin_bit_cast(int, 1.0f), __builtin_bit_cast(int, e_inc), 0x111, 0xf, 0xf, false));
        {
          const float c15 = lane_value(e_inc, 15), c31 = lane_value(e_inc, 31), c47 = lane_value(e_inc, 47);
          if (c16 == 0) e_exc = g == 0 ? 1.0f : g == 1 ? c15 : g == 2 ? c31 : c47;
        }
        const float a = kReg ? eta * (in[0] - e_exc * in[2]) : eta * in[0];
        sm.rp[l][j] = f32x4{a, eta, gam, e_inc * in[3]};
        if (l == 63) sm.e63[j] = e_inc;
      }
    }
    // ---- per-column rows: residual system, weights, outputs --------------
    float u[16], ov[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) { u[k] = 0.f; ov[k] = 0.f; }
    solve_rows<kReg, 0>(sm, jc, qq, u, ov);
#pragma unroll
    for (int k = 0; k < 16; ++k) sm.rp[4 * k + qq][jc][0] = ov[k];
    // ---- outputs (row l of the slice) and the state update -----------------
    {
      const int tok = t0 + l;
      if (tok < T) {
        uint32_t w[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e] = pack_bf16x2(sm.rp[l][2 * e][0], sm.rp[l][2 * e + 1][0]);
        uint4* dst = reinterpret_cast<uint4*>(o + (bh * T + tok) * kD + j0);
        dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
        dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
      }
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) sm.ut[jc][4 * k + qq] = bf(u[k]);
    {
      const float dec = sm.e63[c16];
      const bf16x8 u0 = frag_lds(&sm.ut[c16][0], 0, g);
      const bf16x8 u1 = frag_lds(&sm.ut[c16][0], 32, g);
#pragma unroll
      for (int fb = 0; fb < 4; ++fb) {
        const bf16x8 sel = select_frag(fb & 1, g, c16);
        f32x4 d[4];
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) d[sb] = mfma32(ring_frag_c(sm.x, 16 * sb + c16, fb >> 1, g), sel, zero4());
        f32x4 acc = S[fb] * dec;
        acc = mfma32(frag_acc(d[0], d[1]), u0, acc);
        S[fb] = mfma32(frag_acc(d[2], d[3]), u1, acc);
      }
    }
  }
  if (S_T) {
#pragma unroll
    for (int fb = 0; fb < 4; ++fb)
#pragma unroll
      for (int r = 0; r < 4; ++r) S_T[(bh * kD + 16 * fb + 4 * g + r) * kD + j0 + c16] = S[fb][r];
  }
}

}  // namespace

bool chunked_percol_applies(const ProblemArgs& a) {
  return a.bf16 && (a.variant == kF2 || a.variant == kF2A) && a.dk == kD && a.dv == kD && a.C == kC;
}

hipError_t launch_chunked_percol(const ProblemArgs& a, hipStream_t st) {
  const dim3 grid(unsigned(int64_t(a.B) * a.H * (kD / kSlice)));
  if (a.variant == kF2)
    hipLaunchKernelGGL(falcon2_chunked_kernel<true>, grid, dim3(64), 0, st,
                       static_cast<const bf16_t*>(a.phi_k), static_cast<const bf16_t*>(a.phi_q),
                       static_cast<const bf16_t*>(a.v), a.beta, a.lam, a.S0,
                       static_cast<const bf16_t*>(a.k_prev), static_cast<bf16_t*>(a.o), a.S_T, a.T, a.eps,
                       a.eps_gamma);
  else
    hipLaunchKernelGGL(falcon2_chunked_kernel<false>, grid, dim3(64), 0, st,
                       static_cast<const bf16_t*>(a.phi_k), static_cast<const bf16_t*>(a.phi_q),
                       static_cast<const bf16_t*>(a.v), a.beta, a.lam, a.S0,
                       static_cast<const bf16_t*>(a.k_prev), static_cast<bf16_t*>(a.o), a.S_T, a.T, a.eps,
                       a.eps_gamma);
  return hipGetLastError();
}

}  // namespace falcon
