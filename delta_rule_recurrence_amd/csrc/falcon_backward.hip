// Backward of the chunked Falcon-1 forward (gfx950), float32 gradients.
//
// Forward, per 32-token chunk with incoming state S (g_i the chunk-local
// prefix of log gamma, gp_i = g_{i-1}, G = g_31; x_i, q_i, v_i the chunk's
// shifted keys, queries and values):
//   A_{is} = eta_i e^{gp_i-g_s} (x_i.x_s) (s < i),  W = (I + A)^{-1} Diag(eta e^{gp}) X,
//   U = (I + A)^{-1} Diag(eta) V,  Xh = Diag(e^{G-g}) X,  M_{is} = (q_i.x_s) e^{g_i-g_s} (s <= i),
//   S' = P S + H,  O = Qt S + Ot   with
//   P = e^G I - Xh^T W,  H = Xh^T U,  Qt = Diag(e^g) Q - M W,  Ot = M U
// (the chunk-parallel form of Section 4.2 with the log-space renormalisation
// of Section 4.4 applied per chunk; exact up to rounding).  Training
// differentiates through the update (Section 3), so for L = <dO, O> +
// <dS_T, S_T> the backward is:
//   1. chunk maps P, H, Qt, Ot for every chunk (chunk-parallel);
//   2. forward state chain, saving the state S_c entering each chunk;
//   3. reverse adjoint chain: with Lam_c = dL/dS at the end of chunk c,
//      Lam_{c-1} = P_c^T Lam_c + Qt_c^T dO_c, and dS0 = the last Lam;
//   4. per chunk (chunk-parallel), reverse mode through the chunk maps from
//      dP = Lam S_c^T, dH = Lam, dQt = dO S_c^T, dOt = dO:
//        dW = -Xh dP - M^T dQt,  dU = Xh Lam + M^T dO,  dXh = -W dP^T + U Lam^T,
//        dM = -dQt W^T + dO U^T,  dQ = Diag(e^g) dQt + (dM o D) X,
//        dY = (I + A)^{-T} dW,  dZ = (I + A)^{-T} dU,  dA = -dY W^T - dZ U^T,
//      then the Gram, the decays and the gates (eta, the clamped log decay,
//      the prefix sums) by the chain rule, and the key shift x_t = phi(k_{t-1}).
// Every product runs on the matrix cores in float32 (v_mfma_f32_16x16x4f32)
// with operands in LDS; the triangular solves run one column per thread.

#include "falcon_device.h"
#include "falcon_launch.h"

namespace falcon {

namespace {

constexpr int kBC = 32;        // chunk length of the backward
constexpr int kD = 64;         // dk = dv
constexpr int kPW = 68;        // float pitch of 64-wide LDS matrices
constexpr int kPN = 36;        // float pitch of 32-wide LDS matrices
constexpr int kThreads = 256;  // four waves
constexpr int kMapFloats = kD * kD * 2 + kBC * kD * 2;   // P, H, Qt, Ot

typedef float f32x4 __attribute__((ext_vector_type(4)));

// D (M x N) = op(A) op(B) on the matrix cores in float32; A is M x K (stored
// K x M when TA), B is K x N (stored N x K when TB), both in LDS with float
// pitches pa, pb.  The 16x16 output tiles go round-robin to the four waves
// (the same lane always gets the same output element for a given M, N), and
// epi(row, col, value) receives each result.
template <int M, int N, int K, bool TA, bool TB, typename Epi>
__device__ __forceinline__ void mm(const float* A, int pa, const float* B, int pb, int w, int l, Epi epi) {
  const int g = l >> 4, c16 = l & 15;
  constexpr int TN = N / 16;
  static_assert((M / 16) * TN % 4 == 0, "tiles must split evenly over the four waves");
#pragma unroll
  for (int it = 0; it < (M / 16) * TN / 4; ++it) {
    const int tile = w + 4 * it;
    const int tm = tile / TN, tn = tile % TN;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < K / 4; ++kb) {
      const int k = 4 * kb + g;
      const float a = TA ? A[k * pa + 16 * tm + c16] : A[(16 * tm + c16) * pa + k];
      const float b = TB ? B[(16 * tn + c16) * pb + k] : B[k * pb + 16 * tn + c16];
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) epi(16 * tm + 4 * g + r, 16 * tn + c16, acc[r]);
  }
}

// out = (I + A)^{-1} r and out = (I + A)^{-T} r for A strictly lower (32 x 32
// in LDS); r(i) gives row i of the right-hand side's column.
template <typename R>
__device__ __forceinline__ void solve_lower(const float (*AA)[kPN], R r, float (&out)[kBC]) {
#pragma unroll
  for (int i = 0; i < kBC; ++i) {
    float acc = r(i);
#pragma unroll
    for (int s = 0; s < i; ++s) acc = fmaf(-AA[i][s], out[s], acc);
    out[i] = acc;
  }
}
template <typename R>
__device__ __forceinline__ void solve_lower_t(const float (*AA)[kPN], R r, float (&out)[kBC]) {
#pragma unroll
  for (int i = kBC - 1; i >= 0; --i) {
    float acc = r(i);
#pragma unroll
    for (int s = i + 1; s < kBC; ++s) acc = fmaf(-AA[s][i], out[s], acc);
    out[i] = acc;
  }
}

struct BwdArgs {
  const void* phi_k;
  const void* phi_q;
  const void* v;
  const float* beta;
  const float* lam;
  const float* S0;
  const void* k_prev;
  const void* dO;
  const float* dS_T;
  float* dphi_k;
  float* dphi_q;
  float* dv;
  float* dbeta;
  float* dlam;
  float* dS0;
  float* dk_prev;
  float* maps;     // per chunk: P [64][64], H [64][64], Qt [32][64], Ot [32][64]
  float* ckpt;     // per chunk: S entering the chunk [64][64]
  float* adj;      // per chunk: dL/dS at the end of the chunk [64][64]
  int T, nchunks;
  float eps, eps_gamma;
};

// The forward quantities of one chunk, in LDS.
struct ChunkCore {
  float X[kBC][kPW];     // x_i = phi(k_{t0+i-1}); 0 at a fresh start and past T
  float Q[kBC][kPW];     // q_i; 0 past T
  float KX[kBC][kPN];    // x_i . x_s
  float AA[kBC][kPN];    // A, strictly lower
  float MM[kBC][kPN];    // M, lower with the diagonal
  float W[kBC][kPW];
  float U[kBC][kPW];
  float eta[kBC], g[kBC], gp[kBC], lg[kBC], lamv[kBC], betav[kBC], den[kBC];
  int flags[kBC];        // 1: eta from the formula, 2: the clamp binds, 4: live row
  float G;
};

template <typename IO>
__device__ __forceinline__ float ld_row(const IO* base, int64_t row, int col) {
  return io<IO>::load(base, row * kD + col);
}

// Loads the chunk's keys, queries and gate inputs; derives the gates; forms
// the Gram, A, M and (by two triangular solves) W and U.
template <typename IO>
__device__ void chunk_forward(ChunkCore& cc, const BwdArgs& a, int64_t bh, int c, int tid, int w, int l) {
  const int T = a.T;
  const int t0 = c * kBC;
  const bool fresh = (a.k_prev == nullptr);
  const IO* K = static_cast<const IO*>(a.phi_k) + bh * T * kD;
  const IO* Qp = static_cast<const IO*>(a.phi_q) + bh * T * kD;
  const IO* V = static_cast<const IO*>(a.v) + bh * T * kD;
  const IO* kp = a.k_prev ? static_cast<const IO*>(a.k_prev) + bh * kD : nullptr;
  for (int e = tid; e < kBC * kD; e += kThreads) {
    const int i = e >> 6, f = e & 63;
    const int t = t0 + i;
    float xv = 0.f, qv = 0.f;
    if (t < T) {
      if (t >= 1) xv = ld_row(K, t - 1, f);
      else if (kp) xv = io<IO>::load(kp, f);
      qv = ld_row(Qp, t, f);
    }
    cc.X[i][f] = xv;
    cc.Q[i][f] = qv;
  }
  if (tid < kBC) {
    const int t = t0 + tid;
    cc.betav[tid] = t < T ? a.beta[bh * T + t] : 0.f;
    cc.lamv[tid] = t < T ? a.lam[bh * T + t] : 0.f;
  }
  __syncthreads();
  if (tid < kBC) {
    // gates of row i (Eq. 3.4; Section 4.3 clamp; Section 3 fresh-start sentinel)
    const int i = tid, t = t0 + i;
    float en = 0.f;
#pragma unroll 16
    for (int f = 0; f < kD; ++f) en = fmaf(cc.X[i][f], cc.X[i][f], en);
    const bool live = t < T;
    const float lamv = cc.lamv[i];
    const float den = en + lamv + a.eps;
    const bool on = live && !(fresh && t == 0) && den != 0.0f;
    const float eta = on ? cc.betav[i] / den : 0.0f;
    const float alpha = eta * lamv;
    const bool clamped = alpha > 1.0f - a.eps_gamma;
    const float lg = live ? log1pf(-fminf(alpha, 1.0f - a.eps_gamma)) : 0.0f;
    cc.eta[i] = eta;
    cc.den[i] = den;
    cc.lg[i] = lg;
    cc.flags[i] = (on ? 1 : 0) | (clamped ? 2 : 0) | (live ? 4 : 0);
  }
  __syncthreads();
  if (tid < kBC) {
    // chunk-local prefix sums of the log decays
    const int i = tid;
    float gi = 0.f, gpv = 0.f;
    for (int r = 0; r <= i; ++r) {
      gpv = gi;
      gi += cc.lg[r];
    }
    cc.g[i] = gi;
    cc.gp[i] = gpv;
    if (i == kBC - 1) cc.G = gi;
  }
  __syncthreads();
  // Gram, A and M
  mm<kBC, kBC, kD, false, true>(&cc.X[0][0], kPW, &cc.X[0][0], kPW, w, l, [&](int r, int s, float v) {
    cc.KX[r][s] = v;
    cc.AA[r][s] = s < r ? cc.eta[r] * __expf(cc.gp[r] - cc.g[s]) * v : 0.f;
  });
  mm<kBC, kBC, kD, false, true>(&cc.Q[0][0], kPW, &cc.X[0][0], kPW, w, l, [&](int r, int s, float v) {
    cc.MM[r][s] = s <= r ? __expf(cc.g[r] - cc.g[s]) * v : 0.f;
  });
  __syncthreads();
  // W = (I + A)^{-1} Diag(eta e^{gp}) X and U = (I + A)^{-1} Diag(eta) V, a column per thread
  if (tid < 2 * kD) {
    const int j = tid & 63;
    float col[kBC];
    if (tid < kD) {
      solve_lower(cc.AA, [&](int i) { return cc.eta[i] * __expf(cc.gp[i]) * cc.X[i][j]; }, col);
#pragma unroll
      for (int i = 0; i < kBC; ++i) cc.W[i][j] = col[i];
    } else {
      solve_lower(cc.AA, [&](int i) { return t0 + i < T ? cc.eta[i] * ld_row(V, t0 + i, j) : 0.f; }, col);
#pragma unroll
      for (int i = 0; i < kBC; ++i) cc.U[i][j] = col[i];
    }
  }
  __syncthreads();
}

// ---- launch 1: chunk maps --------------------------------------------------------
struct MapSmem {
  ChunkCore cc;
  float XH[kBC][kPW];    // Diag(e^{G-g}) X
};

template <typename IO>
__global__ void __launch_bounds__(kThreads) falcon1_bwd_maps_kernel(BwdArgs a) {
  __shared__ MapSmem sm;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;   // wave-uniform
  const int64_t bh = blockIdx.x / a.nchunks;
  const int c = blockIdx.x % a.nchunks;
  ChunkCore& cc = sm.cc;
  chunk_forward<IO>(cc, a, bh, c, tid, w, l);
  for (int e = tid; e < kBC * kD; e += kThreads) {
    const int i = e >> 6, f = e & 63;
    sm.XH[i][f] = __expf(cc.G - cc.g[i]) * cc.X[i][f];
  }
  __syncthreads();
  float* out = a.maps + int64_t(blockIdx.x) * kMapFloats;
  const float eG = __expf(cc.G);
  // P = e^G I - Xh^T W, H = Xh^T U
  mm<kD, kD, kBC, true, false>(&sm.XH[0][0], kPW, &cc.W[0][0], kPW, w, l,
                               [&](int r, int s, float v) { out[r * kD + s] = (r == s ? eG : 0.f) - v; });
  mm<kD, kD, kBC, true, false>(&sm.XH[0][0], kPW, &cc.U[0][0], kPW, w, l,
                               [&](int r, int s, float v) { out[kD * kD + r * kD + s] = v; });
  // Qt = Diag(e^g) Q - M W, Ot = M U
  mm<kBC, kD, kBC, false, false>(&cc.MM[0][0], kPN, &cc.W[0][0], kPW, w, l, [&](int r, int s, float v) {
    out[2 * kD * kD + r * kD + s] = __expf(cc.g[r]) * cc.Q[r][s] - v;
  });
  mm<kBC, kD, kBC, false, false>(&cc.MM[0][0], kPN, &cc.U[0][0], kPW, w, l,
                                 [&](int r, int s, float v) { out[2 * kD * kD + kBC * kD + r * kD + s] = v; });
}

// ---- launches 2 and 3: the state chain and the adjoint chain -------------------
struct ChainSmem {
  float S[2][kD][kPW];   // state (or adjoint), double-buffered
  float P[kD][kPW];      // this chunk's P
  float B[kD][kPW];      // this chunk's H (state chain) or Qt in rows 0..31 (adjoint chain)
  float O[kBC][kPW];     // this chunk's dO (adjoint chain)
};

// State chain: S_c into ckpt[c], then S <- P_c S + H_c.
__global__ void __launch_bounds__(kThreads) falcon1_bwd_state_kernel(BwdArgs a) {
  __shared__ ChainSmem sm;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;
  const int64_t bh = blockIdx.x;
  for (int e = tid; e < kD * kD; e += kThreads)
    sm.S[0][e >> 6][e & 63] = a.S0 ? a.S0[bh * kD * kD + e] : 0.f;
  int cur = 0;
  for (int c = 0; c < a.nchunks; ++c) {
    const float* mp = a.maps + (bh * a.nchunks + c) * kMapFloats;
    float* ck = a.ckpt + (bh * a.nchunks + c) * kD * kD;
    for (int e = tid; e < kD * kD; e += kThreads) {
      sm.P[e >> 6][e & 63] = mp[e];
      sm.B[e >> 6][e & 63] = mp[kD * kD + e];
    }
    __syncthreads();
    float (*S)[kPW] = sm.S[cur];
    float (*Sn)[kPW] = sm.S[cur ^ 1];
    for (int e = tid; e < kD * kD; e += kThreads) ck[e] = S[e >> 6][e & 63];
    mm<kD, kD, kD, false, false>(&sm.P[0][0], kPW, &S[0][0], kPW, w, l,
                                 [&](int r, int s, float v) { Sn[r][s] = v + sm.B[r][s]; });
    __syncthreads();
    cur ^= 1;
  }
}

// Adjoint chain: adj[c] = Lam at the end of chunk c, then
// Lam <- P_c^T Lam + Qt_c^T dO_c; finally dS0 = Lam.
template <typename IO>
__global__ void __launch_bounds__(kThreads) falcon1_bwd_adjoint_kernel(BwdArgs a) {
  __shared__ ChainSmem sm;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;
  const int64_t bh = blockIdx.x;
  const int T = a.T;
  const IO* dO = static_cast<const IO*>(a.dO) + bh * T * kD;
  for (int e = tid; e < kD * kD; e += kThreads)
    sm.S[0][e >> 6][e & 63] = a.dS_T ? a.dS_T[bh * kD * kD + e] : 0.f;
  int cur = 0;
  for (int c = a.nchunks - 1; c >= 0; --c) {
    const float* mp = a.maps + (bh * a.nchunks + c) * kMapFloats;
    float* ad = a.adj + (bh * a.nchunks + c) * kD * kD;
    for (int e = tid; e < kD * kD; e += kThreads) sm.P[e >> 6][e & 63] = mp[e];
    for (int e = tid; e < kBC * kD; e += kThreads) {
      const int i = e >> 6, f = e & 63, t = c * kBC + i;
      sm.B[i][f] = mp[2 * kD * kD + e];
      sm.O[i][f] = t < T ? ld_row(dO, t, f) : 0.f;
    }
    __syncthreads();
    float (*S)[kPW] = sm.S[cur];
    float (*Sn)[kPW] = sm.S[cur ^ 1];
    for (int e = tid; e < kD * kD; e += kThreads) ad[e] = S[e >> 6][e & 63];
    mm<kD, kD, kD, true, false>(&sm.P[0][0], kPW, &S[0][0], kPW, w, l,
                                [&](int r, int s, float v) { Sn[r][s] = v; });
    mm<kD, kD, kBC, true, false>(&sm.B[0][0], kPW, &sm.O[0][0], kPW, w, l,
                                 [&](int r, int s, float v) { Sn[r][s] += v; });
    __syncthreads();
    cur ^= 1;
  }
  if (a.dS0)
    for (int e = tid; e < kD * kD; e += kThreads) a.dS0[bh * kD * kD + e] = sm.S[cur][e >> 6][e & 63];
}

// ---- launch 4: reverse mode through one chunk ----------------------------------
struct GradSmem {
  ChunkCore cc;
  float SC[kD][kPW];     // S entering the chunk; later dXh in rows 0..31
  float LL[kD][kPW];     // dL/dS at the end of the chunk
  float DP[kD][kPW];     // dP
  float DO[kBC][kPW];    // dO
  float DQT[kBC][kPW];   // dQt
  float DW[kBC][kPW];    // dW, then dY
  float DU[kBC][kPW];    // dU, then dZ
  float DM[kBC][kPN];    // dM, then dM o D, then dA, then its decayed, eta-scaled form
  float DX[kBC][kPW];    // dX accumulator
  float dg[kBC], dgp[kBC], deta[kBC], dgt[kBC];
  float dG;
};

template <typename IO>
__global__ void __launch_bounds__(kThreads) falcon1_bwd_chunk_kernel(BwdArgs a) {
  __shared__ GradSmem sm;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;
  const int64_t bh = blockIdx.x / a.nchunks;
  const int c = blockIdx.x % a.nchunks;
  const int T = a.T;
  const int t0 = c * kBC;
  ChunkCore& cc = sm.cc;
  const IO* dO = static_cast<const IO*>(a.dO) + bh * T * kD;
  const IO* V = static_cast<const IO*>(a.v) + bh * T * kD;
  {
    const float* ck = a.ckpt + (bh * a.nchunks + c) * kD * kD;
    const float* ad = a.adj + (bh * a.nchunks + c) * kD * kD;
    for (int e = tid; e < kD * kD; e += kThreads) {
      sm.SC[e >> 6][e & 63] = ck[e];
      sm.LL[e >> 6][e & 63] = ad[e];
    }
    for (int e = tid; e < kBC * kD; e += kThreads) {
      const int i = e >> 6, f = e & 63, t = t0 + i;
      sm.DO[i][f] = t < T ? ld_row(dO, t, f) : 0.f;
    }
  }
  chunk_forward<IO>(cc, a, bh, c, tid, w, l);
  const float eG = __expf(cc.G);
  auto xs = [&](int i) { return __expf(cc.G - cc.g[i]); };
  // dP = Lam S_c^T, dQt = dO S_c^T
  mm<kD, kD, kD, false, true>(&sm.LL[0][0], kPW, &sm.SC[0][0], kPW, w, l,
                              [&](int r, int s, float v) { sm.DP[r][s] = v; });
  mm<kBC, kD, kD, false, true>(&sm.DO[0][0], kPW, &sm.SC[0][0], kPW, w, l,
                               [&](int r, int s, float v) { sm.DQT[r][s] = v; });
  __syncthreads();
  float (*DXH)[kPW] = sm.SC;   // S_c is no longer needed
  // dW = -Xh dP - M^T dQt, dU = Xh Lam + M^T dO
  mm<kBC, kD, kD, false, false>(&cc.X[0][0], kPW, &sm.DP[0][0], kPW, w, l,
                                [&](int r, int s, float v) { sm.DW[r][s] = -xs(r) * v; });
  mm<kBC, kD, kBC, true, false>(&cc.MM[0][0], kPN, &sm.DQT[0][0], kPW, w, l,
                                [&](int r, int s, float v) { sm.DW[r][s] -= v; });
  mm<kBC, kD, kD, false, false>(&cc.X[0][0], kPW, &sm.LL[0][0], kPW, w, l,
                                [&](int r, int s, float v) { sm.DU[r][s] = xs(r) * v; });
  mm<kBC, kD, kBC, true, false>(&cc.MM[0][0], kPN, &sm.DO[0][0], kPW, w, l,
                                [&](int r, int s, float v) { sm.DU[r][s] += v; });
  // dXh = -W dP^T + U Lam^T, dM = -dQt W^T + dO U^T
  mm<kBC, kD, kD, false, true>(&cc.W[0][0], kPW, &sm.DP[0][0], kPW, w, l,
                               [&](int r, int s, float v) { DXH[r][s] = -v; });
  mm<kBC, kD, kD, false, true>(&cc.U[0][0], kPW, &sm.LL[0][0], kPW, w, l,
                               [&](int r, int s, float v) { DXH[r][s] += v; });
  mm<kBC, kBC, kD, false, true>(&sm.DQT[0][0], kPW, &cc.W[0][0], kPW, w, l,
                                [&](int r, int s, float v) { sm.DM[r][s] = -v; });
  mm<kBC, kBC, kD, false, true>(&sm.DO[0][0], kPW, &cc.U[0][0], kPW, w, l,
                                [&](int r, int s, float v) { sm.DM[r][s] += v; });
  __syncthreads();
  // decay terms of M, Qt and Xh; dG from P = e^G I + ...
  if (tid < kBC) {
    const int i = tid;
    float qd = 0.f, xd = 0.f;
#pragma unroll 16
    for (int f = 0; f < kD; ++f) {
      qd = fmaf(cc.Q[i][f], sm.DQT[i][f], qd);
      xd = fmaf(cc.X[i][f], DXH[i][f], xd);
    }
    float rowm = 0.f, colm = 0.f;
#pragma unroll 8
    for (int s = 0; s < kBC; ++s) {
      rowm = fmaf(sm.DM[i][s], cc.MM[i][s], rowm);
      colm = fmaf(sm.DM[s][i], cc.MM[s][i], colm);
    }
    const float z = xs(i) * xd;
    sm.dg[i] = __expf(cc.g[i]) * qd + rowm - colm - z;
    sm.dgt[i] = z;
  }
  __syncthreads();
  if (tid == 0) {
    float tr = 0.f, zs = 0.f;
    for (int f = 0; f < kD; ++f) tr += sm.DP[f][f];
    for (int i = 0; i < kBC; ++i) zs += sm.dgt[i];
    sm.dG = eG * tr + zs;
  }
  // dM o D, D_{is} = e^{g_i-g_s} for s <= i
  for (int e = tid; e < kBC * kBC; e += kThreads) {
    const int i = e >> 5, s = e & 31;
    sm.DM[i][s] = s <= i ? sm.DM[i][s] * __expf(cc.g[i] - cc.g[s]) : 0.f;
  }
  __syncthreads();
  // dQ = Diag(e^g) dQt + (dM o D) X;  dX = Diag(e^{G-g}) dXh + (dM o D)^T Q
  float* dq_out = a.dphi_q + bh * T * kD;
  mm<kBC, kD, kBC, false, false>(&sm.DM[0][0], kPN, &cc.X[0][0], kPW, w, l, [&](int r, int s, float v) {
    if (t0 + r < T) dq_out[int64_t(t0 + r) * kD + s] = __expf(cc.g[r]) * sm.DQT[r][s] + v;
  });
  mm<kBC, kD, kBC, true, false>(&sm.DM[0][0], kPN, &cc.Q[0][0], kPW, w, l,
                                [&](int r, int s, float v) { sm.DX[r][s] = xs(r) * DXH[r][s] + v; });
  __syncthreads();
  // dY = (I + A)^{-T} dW, dZ = (I + A)^{-T} dU (in place), a column per thread
  if (tid < 2 * kD) {
    const int j = tid & 63;
    float (*D)[kPW] = tid < kD ? sm.DW : sm.DU;
    float col[kBC];
    solve_lower_t(cc.AA, [&](int i) { return D[i][j]; }, col);
#pragma unroll
    for (int i = 0; i < kBC; ++i) D[i][j] = col[i];
  }
  __syncthreads();
  // dA = -dY W^T - dZ U^T (strictly lower part used)
  mm<kBC, kBC, kD, false, true>(&sm.DW[0][0], kPW, &cc.W[0][0], kPW, w, l,
                                [&](int r, int s, float v) { sm.DM[r][s] = -v; });
  mm<kBC, kBC, kD, false, true>(&sm.DU[0][0], kPW, &cc.U[0][0], kPW, w, l,
                                [&](int r, int s, float v) { sm.DM[r][s] -= v; });
  // Y = Diag(eta e^{gp}) X, Z = Diag(eta) V
  float* dv_out = a.dv + bh * T * kD;
  for (int e = tid; e < kBC * kD; e += kThreads) {
    const int i = e >> 6, f = e & 63;
    sm.DX[i][f] = fmaf(cc.eta[i] * __expf(cc.gp[i]), sm.DW[i][f], sm.DX[i][f]);
    if (t0 + i < T) dv_out[int64_t(t0 + i) * kD + f] = cc.eta[i] * sm.DU[i][f];
  }
  if (tid < kBC) {
    const int i = tid;
    float xy = 0.f, vz = 0.f;
    for (int f = 0; f < kD; ++f) {
      xy = fmaf(cc.X[i][f], sm.DW[i][f], xy);
      if (t0 + i < T) vz = fmaf(ld_row(V, t0 + i, f), sm.DU[i][f], vz);
    }
    const float egp = __expf(cc.gp[i]);
    sm.deta[i] = egp * xy + vz;
    sm.dgp[i] = cc.eta[i] * egp * xy;
  }
  __syncthreads();
  // A_{is} = eta_i e^{gp_i-g_s} k_{is}: D2 = dA o e^{gp_i-g_s} (s < i)
  for (int e = tid; e < kBC * kBC; e += kThreads) {
    const int i = e >> 5, s = e & 31;
    sm.DM[i][s] = s < i ? sm.DM[i][s] * __expf(cc.gp[i] - cc.g[s]) : 0.f;
  }
  __syncthreads();
  if (tid < kBC) {
    const int i = tid;
    float row = 0.f, col = 0.f;
    for (int s = 0; s < kBC; ++s) {
      row = fmaf(sm.DM[i][s], cc.KX[i][s], row);
      col = fmaf(cc.eta[s] * sm.DM[s][i], cc.KX[s][i], col);
    }
    sm.deta[i] += row;
    sm.dgp[i] += cc.eta[i] * row;
    sm.dg[i] -= col;
  }
  __syncthreads();
  // dK = Diag(eta) D2 (strictly lower), dX += (dK + dK^T) X
  for (int e = tid; e < kBC * kBC; e += kThreads) {
    const int i = e >> 5, s = e & 31;
    sm.DM[i][s] *= cc.eta[i];
  }
  __syncthreads();
  mm<kBC, kD, kBC, false, false>(&sm.DM[0][0], kPN, &cc.X[0][0], kPW, w, l,
                                 [&](int r, int s, float v) { sm.DX[r][s] += v; });
  mm<kBC, kD, kBC, true, false>(&sm.DM[0][0], kPN, &cc.X[0][0], kPW, w, l,
                                [&](int r, int s, float v) { sm.DX[r][s] += v; });
  __syncthreads();
  // gates: g -> log decay -> (eta, lam); eta -> (beta, lam, ||x||^2)
  if (tid < kBC) {
    const int i = tid;
    sm.dgt[i] = sm.dg[i] + (i + 1 < kBC ? sm.dgp[i + 1] : 0.f) + (i == kBC - 1 ? sm.dG : 0.f);
  }
  __syncthreads();
  if (tid < kBC) {
    const int i = tid;
    float dlg = 0.f;
    for (int r = i; r < kBC; ++r) dlg += sm.dgt[r];
    const int fl = cc.flags[i];
    const float eta = cc.eta[i], lamv = cc.lamv[i];
    float deta = sm.deta[i], dlam = 0.f;
    if ((fl & 4) && !(fl & 2)) {
      const float dalpha = -dlg / (1.0f - eta * lamv);
      deta += dalpha * lamv;
      dlam += dalpha * eta;
    }
    float dbeta = 0.f, dE = 0.f;
    if (fl & 1) {
      const float den = cc.den[i];
      dbeta = deta / den;
      const float dden = -deta * eta / den;
      dlam += dden;
      dE = dden;
    }
    const int t = t0 + i;
    if (t < T) {
      a.dbeta[bh * T + t] = dbeta;
      a.dlam[bh * T + t] = dlam;
    }
    sm.deta[i] = dE;     // reused: d||x_i||^2
  }
  __syncthreads();
  // x_t = phi(k_{t-1}): row i of dX is the gradient of key t0 + i - 1
  float* dk_out = a.dphi_k + bh * T * kD;
  const bool fresh = (a.k_prev == nullptr);
  for (int e = tid; e < kBC * kD; e += kThreads) {
    const int i = e >> 6, f = e & 63, t = t0 + i;
    const float dx = fmaf(2.0f * sm.deta[i], cc.X[i][f], sm.DX[i][f]);
    if (t >= 1 && t < T) dk_out[int64_t(t - 1) * kD + f] = dx;
    if (t == 0 && !fresh && a.dk_prev) a.dk_prev[bh * kD + f] = dx;
  }
  // the last key feeds no token of this call
  if (c == a.nchunks - 1)
    for (int f = tid; f < kD; f += kThreads) dk_out[int64_t(T - 1) * kD + f] = 0.f;
}

}  // namespace

size_t bwd_workspace_bytes(const ProblemArgs& p) {
  const int64_t nchunks = (int64_t(p.T) + kBC - 1) / kBC;
  const int64_t n = int64_t(p.B) * p.H * nchunks;
  return size_t(n) * (kMapFloats + 2 * kD * kD) * sizeof(float);
}

hipError_t launch_bwd(const ProblemArgs& p, const BwdBuffers& b, hipStream_t st) {
  const int64_t BH = int64_t(p.B) * p.H;
  const int nchunks = (p.T + kBC - 1) / kBC;
  BwdArgs a;
  a.phi_k = p.phi_k; a.phi_q = p.phi_q; a.v = p.v; a.beta = p.beta; a.lam = p.lam; a.S0 = p.S0;
  a.k_prev = p.k_prev; a.dO = b.dO; a.dS_T = b.dS_T;
  a.dphi_k = b.dphi_k; a.dphi_q = b.dphi_q; a.dv = b.dv; a.dbeta = b.dbeta; a.dlam = b.dlam;
  a.dS0 = b.dS0; a.dk_prev = b.dk_prev;
  float* ws = static_cast<float*>(p.workspace);
  const int64_t n = BH * nchunks;
  a.maps = ws;
  a.ckpt = ws + n * kMapFloats;
  a.adj = a.ckpt + n * kD * kD;
  a.T = p.T; a.nchunks = nchunks; a.eps = p.eps; a.eps_gamma = p.eps_gamma;
  if (p.bf16) {
    hipLaunchKernelGGL(falcon1_bwd_maps_kernel<bf16_t>, dim3(unsigned(n)), dim3(kThreads), 0, st, a);
    hipLaunchKernelGGL(falcon1_bwd_state_kernel, dim3(unsigned(BH)), dim3(kThreads), 0, st, a);
    hipLaunchKernelGGL(falcon1_bwd_adjoint_kernel<bf16_t>, dim3(unsigned(BH)), dim3(kThreads), 0, st, a);
    hipLaunchKernelGGL(falcon1_bwd_chunk_kernel<bf16_t>, dim3(unsigned(n)), dim3(kThreads), 0, st, a);
  } else {
    hipLaunchKernelGGL(falcon1_bwd_maps_kernel<float>, dim3(unsigned(n)), dim3(kThreads), 0, st, a);
    hipLaunchKernelGGL(falcon1_bwd_state_kernel, dim3(unsigned(BH)), dim3(kThreads), 0, st, a);
    hipLaunchKernelGGL(falcon1_bwd_adjoint_kernel<float>, dim3(unsigned(BH)), dim3(kThreads), 0, st, a);
    hipLaunchKernelGGL(falcon1_bwd_chunk_kernel<float>, dim3(unsigned(n)), dim3(kThreads), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace falcon
