// Recurrent form and single-token decode of the Falcon rules (gfx950).
//
// Both kernels hold the float32 state on-chip in registers and make exactly
// one pass over their inputs.  Thread layout: a thread owns 16 consecutive
// state rows of one value column (recurrent) or of four value columns
// (decode); the dk/16 threads that share a column reduce their partial dot
// products with cross-lane shuffles (recurrent) or through LDS (decode).
//
// Paper: "Fast Weight Attention for Continual Learning", Section 4 naming and
// formula summary (the rules), Eq. (3.4) (step size), Section 4.3 "Decay
// positivity" (clamp); the per-token order follows the Falcon-1 step listing
// of the rcap.io post (residual from the pre-update state, read after write).

#include "falcon_device.h"
#include "falcon_launch.h"

namespace falcon {

namespace {

constexpr int kRows = 16;  // state rows held by one thread

template <typename IO>
__device__ __forceinline__ void load16(const IO* p, float out[kRows]) {
#pragma unroll
  for (int i = 0; i < kRows; ++i) out[i] = io<IO>::load(p, i);
}
template <>
__device__ __forceinline__ void load16<bf16_t>(const bf16_t* p, float out[kRows]) {
  const uint4* q = reinterpret_cast<const uint4*>(p);
  const uint4 a = q[0], b = q[1];
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
template <>
__device__ __forceinline__ void load16<float>(const float* p, float out[kRows]) {
  const float4* q = reinterpret_cast<const float4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 a = q[i];
    out[4 * i] = a.x; out[4 * i + 1] = a.y; out[4 * i + 2] = a.z; out[4 * i + 3] = a.w;
  }
}

__device__ __forceinline__ float group_sum(float v, int rs) {
  for (int m = 1; m < rs; m <<= 1) v += __shfl_xor(v, m);
  return v;
}

// One workgroup per (b*h, value-column tile).  blockDim.x = ncols * rs with
// rs = dk / 16; thread tid = col * rs + r owns rows [16 r, 16 r + 16) of
// column col of the tile.
template <typename IO, int VARIANT>
__global__ void __launch_bounds__(512)
recurrent_kernel(const IO* __restrict__ phi_k, const IO* __restrict__ phi_q,
                 const IO* __restrict__ v, const float* __restrict__ beta,
                 const float* __restrict__ lam, const float* S0, const IO* __restrict__ k_prev,
                 IO* __restrict__ o, float* S_T, int T, int dk, int dv, float eps,
                 float eps_gamma) {
  const int rs = dk / kRows;
  const int ncols = blockDim.x / rs;
  const int r = threadIdx.x % rs;
  const int col = blockIdx.y * ncols + threadIdx.x / rs;
  const int64_t bh = blockIdx.x;
  const IO* K = phi_k + bh * T * dk + r * kRows;
  const IO* Q = phi_q + bh * T * dk + r * kRows;
  const IO* V = v + bh * T * dv + col;
  const float* Lm = lam + bh * T;
  const float* Bt = beta + (is_per_column(VARIANT) ? bh * T * dv + col : bh * T);
  const int bstride = is_per_column(VARIANT) ? dv : 1;

  float S[kRows];
#pragma unroll
  for (int i = 0; i < kRows; ++i)
    S[i] = S0 ? S0[(bh * dk + r * kRows + i) * dv + col] : 0.0f;

  const bool fresh = (k_prev == nullptr);
  float x[kRows], q[kRows];
  if (fresh) {
#pragma unroll
    for (int i = 0; i < kRows; ++i) x[i] = 0.0f;
  } else {
    load16<IO>(k_prev + bh * dk + r * kRows, x);
  }
  load16<IO>(Q, q);
  float vt = io<IO>::load(V, 0), bt = Bt[0], lt = Lm[0];

  for (int t = 0; t < T; ++t) {
    // Prefetch step t+1 (its key is this step's k_t).
    float xn[kRows], qn[kRows];
    float vn = 0.f, bn = 0.f, ln = 0.f;
    const bool more = (t + 1 < T);
    if (more) {
      load16<IO>(K + int64_t(t) * dk, xn);
      load16<IO>(Q + int64_t(t + 1) * dk, qn);
      vn = io<IO>::load(V, int64_t(t + 1) * dv);
      bn = Bt[int64_t(t + 1) * bstride];
      ln = Lm[t + 1];
    }

    float e = 0.f;
#pragma unroll
    for (int i = 0; i < kRows; ++i) e = fmaf(x[i], x[i], e);
    e = group_sum(e, rs);
    const float eta = nlms_eta(bt, e, lt, eps, fresh && t == 0);
    const float gamma = clamped_gamma(eta, lt, eps_gamma);

    float target = vt;
    if constexpr (is_regression(VARIANT)) {
      float p = 0.f;
#pragma unroll
      for (int i = 0; i < kRows; ++i) p = fmaf(S[i], x[i], p);
      target = vt - group_sum(p, rs);             // r_t = v_t - S_{t-1}^T x_t
    }
    const float w = eta * target;
    float po = 0.f;
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
      S[i] = fmaf(gamma, S[i], w * x[i]);         // S_t = gamma S + eta x r^T
      po = fmaf(S[i], q[i], po);
    }
    po = group_sum(po, rs);                       // o_t = S_t^T q_t
    if (r == 0) io<IO>::store(o, (bh * T + t) * dv + col, po);

    if (more) {
#pragma unroll
      for (int i = 0; i < kRows; ++i) { x[i] = xn[i]; q[i] = qn[i]; }
      vt = vn; bt = bn; lt = ln;
    }
  }
  if (S_T) {
#pragma unroll
    for (int i = 0; i < kRows; ++i) S_T[(bh * dk + r * kRows + i) * dv + col] = S[i];
  }
}

// Decode: one workgroup per (b, h).  Thread (rg, cg) with tid = rg * ncg + cg
// owns rows rg + nrg * i (i < 16) of the four columns 4 cg .. 4 cg + 3, so a
// wave reads whole state rows (coalesced 16-byte accesses).
template <typename IO, int VARIANT>
__global__ void __launch_bounds__(256)
decode_kernel(const IO* __restrict__ x_in, const IO* __restrict__ q_in,
              const IO* __restrict__ v_in, const float* __restrict__ beta,
              const float* __restrict__ lam, float* __restrict__ S,
              const uint8_t* __restrict__ is_first, IO* __restrict__ o, int H, int dk, int dv,
              float eps, float eps_gamma) {
  extern __shared__ float red[];                  // [nrg][2*dv + 4]
  const int ncg = dv / 4;
  const int nrg = dk / kRows;
  const int cg = threadIdx.x % ncg;
  const int rg = threadIdx.x / ncg;
  const int64_t bh = blockIdx.x;
  const int b = static_cast<int>(bh / H);
  const IO* X = x_in + bh * dk;
  const IO* Qv = q_in + bh * dk;
  float* Sp = S + bh * dk * dv + 4 * cg;

  float4 s[kRows];
  float px[4] = {0, 0, 0, 0}, pq[4] = {0, 0, 0, 0};
  float pe = 0.f, pxq = 0.f;
#pragma unroll
  for (int i = 0; i < kRows; ++i)
    s[i] = *reinterpret_cast<const float4*>(Sp + int64_t(rg + nrg * i) * dv);
#pragma unroll
  for (int i = 0; i < kRows; ++i) {
    const int row = rg + nrg * i;
    const float xr = io<IO>::load(X, row), qr = io<IO>::load(Qv, row);
    px[0] = fmaf(s[i].x, xr, px[0]); px[1] = fmaf(s[i].y, xr, px[1]);
    px[2] = fmaf(s[i].z, xr, px[2]); px[3] = fmaf(s[i].w, xr, px[3]);
    pq[0] = fmaf(s[i].x, qr, pq[0]); pq[1] = fmaf(s[i].y, qr, pq[1]);
    pq[2] = fmaf(s[i].z, qr, pq[2]); pq[3] = fmaf(s[i].w, qr, pq[3]);
    pe = fmaf(xr, xr, pe);
    pxq = fmaf(xr, qr, pxq);
  }
  const int ld = 2 * dv + 4;                      // keeps float4 rows aligned
  float* mine = red + rg * ld;
  *reinterpret_cast<float4*>(mine + 4 * cg) = make_float4(px[0], px[1], px[2], px[3]);
  *reinterpret_cast<float4*>(mine + dv + 4 * cg) = make_float4(pq[0], pq[1], pq[2], pq[3]);
  if (cg == 0) { mine[2 * dv] = pe; mine[2 * dv + 1] = pxq; }
  __syncthreads();
  float4 sx = make_float4(0, 0, 0, 0), sq = make_float4(0, 0, 0, 0);
  float e = 0.f, xq = 0.f;
  for (int g = 0; g < nrg; ++g) {
    const float* p = red + g * ld;
    const float4 a = *reinterpret_cast<const float4*>(p + 4 * cg);
    const float4 c = *reinterpret_cast<const float4*>(p + dv + 4 * cg);
    sx.x += a.x; sx.y += a.y; sx.z += a.z; sx.w += a.w;
    sq.x += c.x; sq.y += c.y; sq.z += c.z; sq.w += c.w;
    e += p[2 * dv];
    xq += p[2 * dv + 1];
  }
  const bool sentinel = is_first != nullptr && is_first[b] != 0;
  const float lt = lam[bh];
  float eta[4], gam[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const float bt = is_per_column(VARIANT) ? beta[bh * dv + 4 * cg + c] : beta[bh];
    eta[c] = nlms_eta(bt, e, lt, eps, sentinel);
    gam[c] = clamped_gamma(eta[c], lt, eps_gamma);
  }
  const float sxa[4] = {sx.x, sx.y, sx.z, sx.w};
  const float sqa[4] = {sq.x, sq.y, sq.z, sq.w};
  float w[4], oc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const float vt = io<IO>::load(v_in, bh * dv + 4 * cg + c);
    const float tgt = is_regression(VARIANT) ? vt - sxa[c] : vt;
    w[c] = eta[c] * tgt;
    // o_t = S_t^T q = gamma S_{t-1}^T q + eta (x . q) target
    oc[c] = fmaf(gam[c], sqa[c], w[c] * xq);
  }
  if (rg == 0) {
#pragma unroll
    for (int c = 0; c < 4; ++c) io<IO>::store(o, bh * dv + 4 * cg + c, oc[c]);
  }
#pragma unroll
  for (int i = 0; i < kRows; ++i) {
    const float xr = io<IO>::load(X, rg + nrg * i);
    float4 n;
    n.x = fmaf(gam[0], s[i].x, w[0] * xr);
    n.y = fmaf(gam[1], s[i].y, w[1] * xr);
    n.z = fmaf(gam[2], s[i].z, w[2] * xr);
    n.w = fmaf(gam[3], s[i].w, w[3] * xr);
    *reinterpret_cast<float4*>(Sp + int64_t(rg + nrg * i) * dv) = n;
  }
}

template <typename IO, int VARIANT>
hipError_t launch_recurrent_t(const ProblemArgs& a, hipStream_t st) {
  const int rs = a.dk / kRows;
  const int ncols = a.dv < 64 ? a.dv : 64;
  dim3 grid(a.B * a.H, a.dv / ncols), block(ncols * rs);
  hipLaunchKernelGGL((recurrent_kernel<IO, VARIANT>), grid, block, 0, st,
                     static_cast<const IO*>(a.phi_k), static_cast<const IO*>(a.phi_q),
                     static_cast<const IO*>(a.v), a.beta, a.lam, a.S0,
                     static_cast<const IO*>(a.k_prev), static_cast<IO*>(a.o), a.S_T, a.T,
                     a.dk, a.dv, a.eps, a.eps_gamma);
  return hipGetLastError();
}

template <typename IO, int VARIANT>
hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t st) {
  const int threads = (a.dk / kRows) * (a.dv / 4);
  const size_t lds = sizeof(float) * (a.dk / kRows) * (2 * a.dv + 4);
  hipLaunchKernelGGL((decode_kernel<IO, VARIANT>), dim3(a.B * a.H), dim3(threads), lds, st,
                     static_cast<const IO*>(a.x), static_cast<const IO*>(a.q),
                     static_cast<const IO*>(a.v), a.beta, a.lam, a.S, a.is_first,
                     static_cast<IO*>(a.o), a.H, a.dk, a.dv, a.eps, a.eps_gamma);
  return hipGetLastError();
}

template <typename IO>
hipError_t dispatch_recurrent(const ProblemArgs& a, hipStream_t st) {
  switch (a.variant) {
    case kF1: return launch_recurrent_t<IO, kF1>(a, st);
    case kF1A: return launch_recurrent_t<IO, kF1A>(a, st);
    case kF2: return launch_recurrent_t<IO, kF2>(a, st);
    default: return launch_recurrent_t<IO, kF2A>(a, st);
  }
}
template <typename IO>
hipError_t dispatch_decode(const DecodeArgs& a, hipStream_t st) {
  switch (a.variant) {
    case kF1: return launch_decode_t<IO, kF1>(a, st);
    case kF1A: return launch_decode_t<IO, kF1A>(a, st);
    case kF2: return launch_decode_t<IO, kF2>(a, st);
    default: return launch_decode_t<IO, kF2A>(a, st);
  }
}

}  // namespace

hipError_t launch_recurrent(const ProblemArgs& a, hipStream_t st) {
  return a.bf16 ? dispatch_recurrent<bf16_t>(a, st) : dispatch_recurrent<float>(a, st);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st) {
  return a.bf16 ? dispatch_decode<bf16_t>(a, st) : dispatch_decode<float>(a, st);
}

}  // namespace falcon
