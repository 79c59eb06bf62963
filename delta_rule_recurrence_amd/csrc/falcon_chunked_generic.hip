// Chunk-parallel Falcon forward, general-shape float32 kernel (gfx950).
//
// Serves every (variant, dtype, dk, dv, C) combination that has no MFMA path
// (the bf16 cases with dk = dv = 64 and C = 64 have their own kernels).
// All arithmetic is float32 on the vector ALUs; intermediates live in LDS.
//
// Chunk algebra (derived from the Section 4 summary rules with the chunk-
// local log-space renormalisation of Section 4.4, "Algorithm 3 realizes
// Eq. (4.16) chunk-locally via log-prefix decays", taken with window B = 1).
// For a chunk with local rows i = 0..C-1, incoming state S and per value
// column j (scalar rules use one gate column for all j):
//   g_i      = sum_{r<=i} log gamma_r             (float32, all exponents <= 0)
//   rho_i    = eta_i r_i  (scaled residual, regression rules) solves the
//              merged residual system
//              rho_i + sum_{s<i} eta_i e^{g_{i-1}-g_s} (x_i.x_s) rho_s
//                    = eta_i (v_i - e^{g_{i-1}} (X S)_i)
//              ("injected-value and projected-history paths share this
//              triangular factor ... one merged residual system", §4.2);
//   rho_i    = eta_i v_i                            (inner-product rules)
//   o_i      = e^{g_i} (Q S)_i + sum_{s<=i} e^{g_i-g_s} (q_i.x_s) rho_s
//   S_next   = e^{g_{C-1}} S + sum_s e^{g_{C-1}-g_s} x_s rho_s^T
// Rows past the end of the sequence get eta = 0 and log gamma = 0, so a
// ragged last chunk needs no special case.

#include <algorithm>

#include "falcon_device.h"
#include "falcon_launch.h"

namespace falcon {

namespace {

constexpr int kThreads = 256;

struct GenericLayout {
  int C, dk, nv, ng;   // chunk, key width, value tile, gate columns (1 or nv)
  int xp;              // padded row pitch of X and Q
  int off_x, off_q, off_p, off_g, off_r, off_o, off_s, off_eta, off_lg, total;
  __host__ __device__ GenericLayout(int C_, int dk_, int nv_, int ng_)
      : C(C_), dk(dk_), nv(nv_), ng(ng_), xp(dk_ + 1) {
    off_x = 0;
    off_q = off_x + C * xp;
    off_p = off_q + C * xp;
    off_g = off_p + C * C;
    off_r = off_g + C * C;
    off_o = off_r + C * nv;
    off_s = off_o + C * nv;
    off_eta = off_s + dk * nv;
    off_lg = off_eta + C * ng;
    total = off_lg + C * ng;
  }
};

template <typename IO, int VARIANT>
__global__ void __launch_bounds__(kThreads)
chunked_generic_kernel(const IO* __restrict__ phi_k, const IO* __restrict__ phi_q,
                       const IO* __restrict__ v, const float* __restrict__ beta,
                       const float* __restrict__ lam, const float* S0,
                       const IO* __restrict__ k_prev, IO* __restrict__ o, float* S_T, int T,
                       int dk, int dv, int C, int nv, float eps, float eps_gamma) {
  constexpr bool kPerCol = is_per_column(VARIANT);
  constexpr bool kReg = is_regression(VARIANT);
  extern __shared__ float lds[];
  const int ng = kPerCol ? nv : 1;
  const GenericLayout L(C, dk, nv, ng);
  float* Xs = lds + L.off_x;      // [C][xp]  shifted keys x_i
  float* Qs = lds + L.off_q;      // [C][xp]  queries
  float* Ps = lds + L.off_p;      // [C][C]   q_i.x_s, then decayed mask
  float* Gs = lds + L.off_g;      // [C][C]   x_i.x_s, then coupling matrix
  float* Rs = lds + L.off_r;      // [C][nv]  -X S, then rhs, then rho
  float* Os = lds + L.off_o;      // [C][nv]  Q S, then scratch
  float* Ss = lds + L.off_s;      // [dk][nv] state tile
  float* Eta = lds + L.off_eta;   // [C][ng]  eta, later e^{g_{C-1}-g_s}
  float* Lg = lds + L.off_lg;     // [C][ng]  log gamma -> inclusive prefix g

  const int tid = threadIdx.x;
  const int64_t bh = blockIdx.x;
  const int j0 = blockIdx.y * nv;
  const bool fresh = (k_prev == nullptr);

  for (int e = tid; e < dk * nv; e += kThreads) {
    const int f = e / nv, j = e % nv;
    Ss[e] = S0 ? S0[(bh * dk + f) * dv + j0 + j] : 0.0f;
  }

  const int nchunks = (T + C - 1) / C;
  for (int c = 0; c < nchunks; ++c) {
    const int t0 = c * C;
    __syncthreads();  // previous chunk finished with every buffer
    // ---- load: shifted keys and queries (values are read with the gates) --
    for (int e = tid; e < C * dk; e += kThreads) {
      const int i = e / dk, f = e % dk;
      const int t = t0 + i;
      float xv = 0.f, qv = 0.f;
      if (t < T) {
        qv = io<IO>::load(phi_q, (bh * T + t) * dk + f);
        if (t >= 1) xv = io<IO>::load(phi_k, (bh * T + t - 1) * dk + f);
        else if (!fresh) xv = io<IO>::load(k_prev, bh * dk + f);
      }
      Xs[i * L.xp + f] = xv;
      Qs[i * L.xp + f] = qv;
    }
    __syncthreads();
    // ---- a1: energies, step sizes, log decays --------------------------
    for (int e = tid; e < C * ng; e += kThreads) {
      const int i = e / ng, cc = e % ng;
      const int t = t0 + i;
      float eta = 0.f, lg = 0.f;
      if (t < T) {
        float en = 0.f;
        for (int f = 0; f < dk; ++f) en = fmaf(Xs[i * L.xp + f], Xs[i * L.xp + f], en);
        const float lt = lam[bh * T + t];
        const float bt = kPerCol ? beta[(bh * T + t) * dv + j0 + cc] : beta[bh * T + t];
        eta = nlms_eta(bt, en, lt, eps, fresh && t == 0);
        lg = clamped_log_gamma(eta, lt, eps_gamma);
      }
      Eta[e] = eta;
      Lg[e] = lg;
    }
    __syncthreads();
    for (int cc = tid; cc < ng; cc += kThreads) {   // inclusive prefix over rows
      float acc = 0.f;
      for (int i = 0; i < C; ++i) { acc += Lg[i * ng + cc]; Lg[i * ng + cc] = acc; }
    }
    // ---- a2 (products that do not need the state) ----------------------
    for (int e = tid; e < C * C; e += kThreads) {
      const int i = e / C, s = e % C;
      float pq = 0.f, px = 0.f;
      if (s <= i) {
        for (int f = 0; f < dk; ++f) pq = fmaf(Qs[i * L.xp + f], Xs[s * L.xp + f], pq);
        if (kReg && s < i)
          for (int f = 0; f < dk; ++f) px = fmaf(Xs[i * L.xp + f], Xs[s * L.xp + f], px);
      }
      Ps[e] = pq;
      Gs[e] = px;
    }
    for (int e = tid; e < C * nv; e += kThreads) {  // Q S and X S with the incoming state
      const int i = e / nv, j = e % nv;
      float qs = 0.f, xs = 0.f;
      for (int f = 0; f < dk; ++f) {
        const float sv = Ss[f * nv + j];
        qs = fmaf(Qs[i * L.xp + f], sv, qs);
        if (kReg) xs = fmaf(Xs[i * L.xp + f], sv, xs);
      }
      Os[e] = qs;
      if (kReg) Rs[e] = -xs;   // stash -(X S)_ij until the gates are ready
      else (void)xs;
    }
    __syncthreads();
    // right-hand side: rho (inner product) or the merged residual rhs
    for (int e = tid; e < C * nv; e += kThreads) {
      const int i = e / nv, j = e % nv;
      const int t = t0 + i;
      const int cc = kPerCol ? j : 0;
      const float eta = Eta[i * ng + cc];
      const float vt = t < T ? io<IO>::load(v, (bh * T + t) * dv + j0 + j) : 0.0f;
      if (kReg) {
        const float gprev = i > 0 ? Lg[(i - 1) * ng + cc] : 0.0f;
        Rs[e] = eta * fmaf(expf(gprev), Rs[e], vt);   // eta (v - e^{g_{i-1}} X S)
      } else {
        Rs[e] = eta * vt;
      }
    }
    if (kReg && !kPerCol) {   // shared coupling matrix eta_i e^{g_{i-1}-g_s} x_i.x_s
      for (int e = tid; e < C * C; e += kThreads) {
        const int i = e / C, s = e % C;
        if (s < i) Gs[e] *= Eta[i] * expf(Lg[i - 1] - Lg[s]);
      }
    }
    __syncthreads();
    // ---- a2/a3: forward substitution of the merged residual system -------
    if (kReg) {
      const int per = kThreads / nv;            // threads per value column
      const int j = tid / per, p = tid % per;
      const int cc = kPerCol ? j : 0;
      for (int i = 1; i < C; ++i) {
        float part = 0.f;
        if (kPerCol) {
          const float ei = Eta[i * ng + cc], gi = Lg[(i - 1) * ng + cc];
          for (int s = p; s < i; s += per)
            part = fmaf(ei * expf(gi - Lg[s * ng + cc]) * Gs[i * C + s], Rs[s * nv + j], part);
        } else {
          for (int s = p; s < i; s += per) part = fmaf(Gs[i * C + s], Rs[s * nv + j], part);
        }
        for (int m = 1; m < per; m <<= 1) part += __shfl_xor(part, m);
        // Every lane of the column group holds the same sum; one writes rho_i.
        if (p == i % per) Rs[i * nv + j] -= part;
        __syncthreads();
      }
    }
    // ---- a4: outputs ---------------------------------------------------
    for (int e = tid; e < C * nv; e += kThreads) {
      const int i = e / nv, j = e % nv;
      const int t = t0 + i;
      if (t >= T) continue;
      const int cc = kPerCol ? j : 0;
      const float gi = Lg[i * ng + cc];
      float acc = expf(gi) * Os[e];
      for (int s = 0; s <= i; ++s)
        acc = fmaf(expf(gi - Lg[s * ng + cc]) * Ps[i * C + s], Rs[s * nv + j], acc);
      io<IO>::store(o, (bh * T + t) * dv + j0 + j, acc);
    }
    __syncthreads();
    // ---- a3: state update S = e^{g_{C-1}} S + sum_s e^{g_{C-1}-g_s} x_s rho_s^T
    for (int e = tid; e < C * ng; e += kThreads) {
      const int s = e / ng, cc = e % ng;
      Eta[e] = expf(Lg[(C - 1) * ng + cc] - Lg[s * ng + cc]);
    }
    __syncthreads();
    for (int e = tid; e < dk * nv; e += kThreads) {
      const int f = e / nv, j = e % nv;
      const int cc = kPerCol ? j : 0;
      float acc = expf(Lg[(C - 1) * ng + cc]) * Ss[e];
      for (int s = 0; s < C; ++s)
        acc = fmaf(Xs[s * L.xp + f] * Eta[s * ng + cc], Rs[s * nv + j], acc);
      Ss[e] = acc;
    }
  }
  __syncthreads();
  if (S_T) {
    for (int e = tid; e < dk * nv; e += kThreads) {
      const int f = e / nv, j = e % nv;
      S_T[(bh * dk + f) * dv + j0 + j] = Ss[e];
    }
  }
}

template <typename IO, int VARIANT>
hipError_t launch_generic_t(const ProblemArgs& a, int nv, size_t lds, hipStream_t st) {
  auto kern = chunked_generic_kernel<IO, VARIANT>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(lds));
  if (e != hipSuccess) return e;
  dim3 grid(a.B * a.H, a.dv / nv);
  hipLaunchKernelGGL(kern, grid, dim3(kThreads), lds, st, static_cast<const IO*>(a.phi_k),
                     static_cast<const IO*>(a.phi_q), static_cast<const IO*>(a.v), a.beta,
                     a.lam, a.S0, static_cast<const IO*>(a.k_prev), static_cast<IO*>(a.o),
                     a.S_T, a.T, a.dk, a.dv, a.C, nv, a.eps, a.eps_gamma);
  return hipGetLastError();
}

template <typename IO>
hipError_t dispatch_generic(const ProblemArgs& a, int nv, size_t lds, hipStream_t st) {
  switch (a.variant) {
    case kF1: return launch_generic_t<IO, kF1>(a, nv, lds, st);
    case kF1A: return launch_generic_t<IO, kF1A>(a, nv, lds, st);
    case kF2: return launch_generic_t<IO, kF2>(a, nv, lds, st);
    default: return launch_generic_t<IO, kF2A>(a, nv, lds, st);
  }
}

}  // namespace

// Largest value tile (64, 32 or 16 columns) whose LDS footprint fits.
int generic_tile(const ProblemArgs& a, size_t* lds_bytes) {
  for (int nv = std::min(a.dv, 64); nv >= 16; nv /= 2) {
    const GenericLayout L(a.C, a.dk, nv, is_per_column(a.variant) ? nv : 1);
    const size_t bytes = sizeof(float) * L.total;
    if (bytes <= 160 * 1024) {
      *lds_bytes = bytes;
      return nv;
    }
  }
  *lds_bytes = 0;
  return 0;
}

hipError_t launch_chunked_generic(const ProblemArgs& a, hipStream_t st) {
  size_t lds = 0;
  const int nv = generic_tile(a, &lds);
  if (nv == 0) return hipErrorInvalidValue;
  return a.bf16 ? dispatch_generic<bf16_t>(a, nv, lds, st) : dispatch_generic<float>(a, nv, lds, st);
}

__global__ void state_copy_kernel(const float* __restrict__ src, float* __restrict__ dst,
                                  int64_t n) {
  for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < n;
       i += int64_t(gridDim.x) * blockDim.x)
    dst[i] = src ? src[i] : 0.0f;
}

hipError_t launch_state_copy(const float* S0, float* S_T, int64_t n, hipStream_t st) {
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(state_copy_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, S0,
                     S_T, n);
  return hipGetLastError();
}

}  // namespace falcon
