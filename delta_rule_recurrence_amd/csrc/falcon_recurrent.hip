// Recurrent form and single-token decode of the Falcon rules (gfx950).
//
// Both kernels hold the float32 state on-chip in registers and make exactly
// one pass over their inputs.  Thread layout: a thread owns 16 consecutive
// state rows of one value column (recurrent) or of four value columns
// (decode); the dk/16 threads that share a column reduce their partial dot
// products with DPP lane moves (recurrent) or through LDS (decode).
//
// Paper: "Fast Weight Attention for Continual Learning", Section 4 naming and
// formula summary (the rules: the residual is taken against the state before
// the write, Eq. 3.3, and the read comes after the write), Eq. (3.4) (step
// size), Section 4.3 "Decay positivity" (clamp).

#include "falcon_device.h"
#include "falcon_launch.h"

namespace falcon {

namespace {

constexpr int kRows = 16;  // state rows held by one decode thread

// Sum over the RS consecutive lanes (RS <= 16, aligned) that share a value
// column: lanes l ^ 1 and l ^ 2 by quad permutes; then, with every quad
// holding its sum, the mirror inside 8 lanes pairs each quad with the other
// one, and the mirror inside 16 lanes pairs the two halves.
template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
template <int RS>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (RS >= 2) v = dpp_add<0xb1>(v);    // quad_perm [1, 0, 3, 2]
  if constexpr (RS >= 4) v = dpp_add<0x4e>(v);    // quad_perm [2, 3, 0, 1]
  if constexpr (RS >= 8) v = dpp_add<0x141>(v);   // row_half_mirror
  if constexpr (RS >= 16) v = dpp_add<0x140>(v);  // row_mirror
  return v;
}

// ---- recurrent form ----------------------------------------------------------
// One workgroup per (b*h, 32-column tile) with NCOLS * RS threads, RS = dk / 8:
// thread tid = col * RS + r owns rows [8 r, 8 r + 8) of column col of the tile.
// The inputs come through LDS in blocks of 32 (or 16) tokens: while a block is
// swept, the next one is loaded straight from global memory into the other
// LDS buffer (direct-to-LDS loads, 16 bytes per lane), so no step waits for
// global memory.  After a block lands, one pass widens bf16 keys and queries
// to float32 (one LDS region, read by the steps) and forms each token's gates:
// eta_t and gamma_t, or for per-column gains 1 / (||x_t||^2 + lam_t + eps)
// (0 where the step size is 0).  The per-step work is then the state's dot
// products and update, with the cross-lane sums in DPP.

// Tokens per staged block: 32, or 16 for rows of 256 bytes and more, so the
// two buffers stay within 64 KB of LDS.
__host__ __device__ constexpr int block_tokens(int dk, int io_bytes) { return dk * io_bytes >= 256 ? 16 : 32; }

typedef __attribute__((address_space(3))) void lds_void;

// Byte layout of one LDS buffer of tc tokens (every part a multiple of 16
// bytes), and of the float32 keys and queries of the block being swept
// (bf16 inputs only), which follow the two buffers.
struct RecLayout {
  int x, q, v, b, l, g, bytes;           // g: per token (eta, gamma), or (1 / (||x||^2 + lam + eps), -)
  int xf, qf, total;
  __host__ __device__ RecLayout(int tc, int dk, int ncols, int io_bytes, bool per_col) {
    x = 0;
    q = x + tc * dk * io_bytes;
    v = q + tc * dk * io_bytes;
    b = v + tc * ncols * io_bytes;
    l = b + tc * (per_col ? ncols : 1) * 4;
    g = l + tc * 4;
    bytes = g + tc * 8;
    xf = 2 * bytes;
    qf = xf + (io_bytes == 2 ? tc * dk * 4 : 0);
    total = qf + (io_bytes == 2 ? tc * dk * 4 : 0);
  }
};

// Direct-to-LDS staging: lane l of an instruction writes bytes
// [16 l, 16 l + 16) (or [4 l, 4 l + 4)) after the wave-uniform LDS address.
// `wl` lanes per wave (the whole block when it is smaller than a wave) and
// `nw` waves cover the units in turn.
//
// Rows [0, tc) of a slab whose row t starts at base + row_of(t) * stride,
// row_bytes each (a multiple of 16), into dense LDS rows at dst.  Rows past
// the sequence read a valid row (row_of clamps); their values are never used.
template <typename RowOf>
__device__ __forceinline__ void stage_rows(char* dst, const char* base, int64_t stride_bytes, int row_bytes,
                                           int tc, RowOf row_of, int wave, int nw, int wl, int lane) {
  const int per_row = row_bytes / 16;
  const int units = tc * per_row;
  for (int u0 = wl * wave; u0 < units; u0 += wl * nw) {
    const int u = u0 + lane;
    const int t = u / per_row, piece = u - t * per_row;
    const char* src = base + row_of(t) * stride_bytes + piece * 16;
    if (u < units) __builtin_amdgcn_global_load_lds(src, (lds_void*)(dst + 16 * u0), 16, 0, 0);
  }
}
// One 4-byte value per row (the per-token gates).
template <typename RowOf>
__device__ __forceinline__ void stage_words(char* dst, const char* base, int64_t stride_bytes, int tc,
                                            RowOf row_of, int wave, int nw, int wl, int lane) {
  for (int u0 = wl * wave; u0 < tc; u0 += wl * nw) {
    const int u = u0 + lane;
    if (u < tc) __builtin_amdgcn_global_load_lds(base + row_of(u) * stride_bytes, (lds_void*)(dst + 4 * u0), 4, 0, 0);
  }
}

constexpr int kRowsR = 8;  // state rows per thread in the recurrent form

template <typename IO>
__device__ __forceinline__ void lds8(const char* p, float out[kRowsR]) {
  if constexpr (sizeof(IO) == 2) {
    const uint4 a = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(w[i] << 16);
      out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const float4 a = reinterpret_cast<const float4*>(p)[i];
      out[4 * i] = a.x; out[4 * i + 1] = a.y; out[4 * i + 2] = a.z; out[4 * i + 3] = a.w;
    }
  }
}
template <typename IO>
__device__ __forceinline__ float lds1(const char* p, int i) {
  if constexpr (sizeof(IO) == 2) return __uint_as_float(uint32_t(reinterpret_cast<const uint16_t*>(p)[i]) << 16);
  else return reinterpret_cast<const float*>(p)[i];
}

template <typename IO, int VARIANT, int RS>
__global__ void __launch_bounds__(1024)
recurrent_kernel(const IO* __restrict__ phi_k, const IO* __restrict__ phi_q,
                 const IO* __restrict__ v, const float* __restrict__ beta,
                 const float* __restrict__ lam, const float* S0, const IO* __restrict__ k_prev,
                 IO* __restrict__ o, float* S_T, int T, int dv, float eps, float eps_gamma) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int dk = RS * kRowsR;
  constexpr int io_bytes = sizeof(IO);
  constexpr bool per_col = is_per_column(VARIANT);
  constexpr int tc = block_tokens(dk, io_bytes);
  const int ncols = blockDim.x / RS;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int nw = (blockDim.x + 63) >> 6;
  const int wl = blockDim.x < 64 ? blockDim.x : 64;
  const int r = tid % RS;
  const int cl = tid / RS;                          // column within the tile
  const int col0 = blockIdx.y * ncols;
  const int col = col0 + cl;
  const int64_t bh = blockIdx.x;
  const RecLayout L(tc, dk, ncols, io_bytes, per_col);
  const bool fresh = (k_prev == nullptr);

  float S[kRowsR];
#pragma unroll
  for (int i = 0; i < kRowsR; ++i)
    S[i] = S0 ? S0[(bh * dk + r * kRowsR + i) * dv + col] : 0.0f;

  const char* Kb = reinterpret_cast<const char*>(phi_k + bh * int64_t(T) * dk);
  const char* Qb = reinterpret_cast<const char*>(phi_q + bh * int64_t(T) * dk);
  const char* Vb = reinterpret_cast<const char*>(v + bh * int64_t(T) * dv + col0);
  const char* Bb = reinterpret_cast<const char*>(beta + (per_col ? bh * int64_t(T) * dv + col0 : bh * int64_t(T)));
  const char* Lb = reinterpret_cast<const char*>(lam + bh * int64_t(T));
  const char* KP = k_prev ? reinterpret_cast<const char*>(k_prev + bh * dk) : nullptr;

  // block j's inputs into buffer j & 1
  auto stage = [&](int j) {
    char* buf = smem + (j & 1) * L.bytes;
    const int t0 = j * tc;
    auto tok = [&](int t) { const int g = t0 + t; return int64_t(g < T ? g : T - 1); };
    // x_t = phi(k_{t-1}); x_0 is the previous key, or (fresh start, step size
    // 0) any valid row
    {
      const int per_row = dk * io_bytes / 16;
      const int units = tc * per_row;
      for (int u0 = wl * wave; u0 < units; u0 += wl * nw) {
        const int u = u0 + lane;
        const int t = u / per_row, piece = u - t * per_row;
        const int g = t0 + t - 1;
        const char* src = (g < 0 && KP) ? KP + piece * 16
                                        : Kb + int64_t(g < 0 ? 0 : (g < T ? g : T - 1)) * dk * io_bytes + piece * 16;
        if (u < units) __builtin_amdgcn_global_load_lds(src, (lds_void*)(buf + L.x + 16 * u0), 16, 0, 0);
      }
    }
    stage_rows(buf + L.q, Qb, int64_t(dk) * io_bytes, dk * io_bytes, tc, tok, wave, nw, wl, lane);
    stage_rows(buf + L.v, Vb, int64_t(dv) * io_bytes, ncols * io_bytes, tc, tok, wave, nw, wl, lane);
    if constexpr (per_col) stage_rows(buf + L.b, Bb, int64_t(dv) * 4, ncols * 4, tc, tok, wave, nw, wl, lane);
    else stage_words(buf + L.b, Bb, 4, tc, tok, wave, nw, wl, lane);
    stage_words(buf + L.l, Lb, 4, tc, tok, wave, nw, wl, lane);
  };

  const int nblocks = (T + tc - 1) / tc;
  if (nblocks > 0) stage(0);
  for (int j = 0; j < nblocks; ++j) {
    char* buf = smem + (j & 1) * L.bytes;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this thread's loads of block j have landed
    __syncthreads();                                   // all of block j landed; block j - 1 is done
    if (j + 1 < nblocks) stage(j + 1);
    // bf16 keys and queries widened once, 8 per thread and pass
    if constexpr (io_bytes == 2) {
      for (int u = tid; u < tc * dk / 8; u += blockDim.x) {
        const uint4 kx = reinterpret_cast<const uint4*>(buf + L.x)[u];
        const uint4 kq = reinterpret_cast<const uint4*>(buf + L.q)[u];
        const uint32_t wx[4] = {kx.x, kx.y, kx.z, kx.w}, wq[4] = {kq.x, kq.y, kq.z, kq.w};
        float4* fx = reinterpret_cast<float4*>(smem + L.xf) + 2 * u;
        float4* fq = reinterpret_cast<float4*>(smem + L.qf) + 2 * u;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          fx[h] = make_float4(__uint_as_float(wx[2 * h] << 16), __uint_as_float(wx[2 * h] & 0xffff0000u),
                              __uint_as_float(wx[2 * h + 1] << 16), __uint_as_float(wx[2 * h + 1] & 0xffff0000u));
          fq[h] = make_float4(__uint_as_float(wq[2 * h] << 16), __uint_as_float(wq[2 * h] & 0xffff0000u),
                              __uint_as_float(wq[2 * h + 1] << 16), __uint_as_float(wq[2 * h + 1] & 0xffff0000u));
        }
      }
    }
    // gates per token: rd = 1 / (||x_t||^2 + lam_t + eps), 0 where the step
    // size is 0 (a zero denominator, or the first step of a fresh start); with
    // one gain per token also eta_t = beta_t rd (Eq. 3.4) and gamma_t
    for (int t = tid; t < tc; t += blockDim.x) {
      float e = 0.f;
      const char* xr = buf + L.x + t * dk * io_bytes;
#pragma unroll
      for (int i = 0; i < dk; ++i) {
        const float xv = lds1<IO>(xr, i);
        e = fmaf(xv, xv, e);
      }
      const float lt = reinterpret_cast<const float*>(buf + L.l)[t];
      const float den = e + lt + eps;
      const bool off = den == 0.0f || (fresh && j * tc + t == 0);
      const float rd = off ? 0.0f : 1.0f / den;
      float2 gt = make_float2(rd, 0.0f);
      if constexpr (!per_col) {
        const float eta = reinterpret_cast<const float*>(buf + L.b)[t] * rd;
        gt = make_float2(eta, clamped_gamma(eta, lt, eps_gamma));
      }
      reinterpret_cast<float2*>(buf + L.g)[t] = gt;
    }
    __syncthreads();
    const int t0 = j * tc;
    const int nt = T - t0 < tc ? T - t0 : tc;
    for (int t = 0; t < nt; ++t) {
      float x[kRowsR], q[kRowsR];
      if constexpr (io_bytes == 2) {
        lds8<float>(smem + L.xf + (t * dk + r * kRowsR) * 4, x);
        lds8<float>(smem + L.qf + (t * dk + r * kRowsR) * 4, q);
      } else {
        lds8<IO>(buf + L.x + (t * dk + r * kRowsR) * io_bytes, x);
        lds8<IO>(buf + L.q + (t * dk + r * kRowsR) * io_bytes, q);
      }
      const float vt = lds1<IO>(buf + L.v, t * ncols + cl);
      const float2 gt = reinterpret_cast<const float2*>(buf + L.g)[t];
      float eta, gamma;
      if constexpr (per_col) {
        eta = reinterpret_cast<const float*>(buf + L.b)[t * ncols + cl] * gt.x;   // Eq. 3.4
        gamma = clamped_gamma(eta, reinterpret_cast<const float*>(buf + L.l)[t], eps_gamma);
      } else {
        eta = gt.x;
        gamma = gt.y;
      }
      float target = vt;
      if constexpr (is_regression(VARIANT)) {
        float p0 = 0.f, p1 = 0.f, p2 = 0.f, p3 = 0.f;
#pragma unroll
        for (int i = 0; i < kRowsR; i += 4) {
          p0 = fmaf(S[i], x[i], p0);
          p1 = fmaf(S[i + 1], x[i + 1], p1);
          p2 = fmaf(S[i + 2], x[i + 2], p2);
          p3 = fmaf(S[i + 3], x[i + 3], p3);
        }
        target = vt - group_sum<RS>((p0 + p1) + (p2 + p3));   // r_t = v_t - S_{t-1}^T x_t
      }
      const float w = eta * target;
      float o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;
#pragma unroll
      for (int i = 0; i < kRowsR; i += 4) {
        S[i] = fmaf(gamma, S[i], w * x[i]);                 // S_t = gamma S + eta x r^T
        S[i + 1] = fmaf(gamma, S[i + 1], w * x[i + 1]);
        S[i + 2] = fmaf(gamma, S[i + 2], w * x[i + 2]);
        S[i + 3] = fmaf(gamma, S[i + 3], w * x[i + 3]);
        o0 = fmaf(S[i], q[i], o0);
        o1 = fmaf(S[i + 1], q[i + 1], o1);
        o2 = fmaf(S[i + 2], q[i + 2], o2);
        o3 = fmaf(S[i + 3], q[i + 3], o3);
      }
      const float po = group_sum<RS>((o0 + o1) + (o2 + o3));  // o_t = S_t^T q_t
      if (r == 0) io<IO>::store(o, (bh * T + t0 + t) * dv + col, po);
    }
  }
  if (S_T) {
#pragma unroll
    for (int i = 0; i < kRowsR; ++i) S_T[(bh * dk + r * kRowsR + i) * dv + col] = S[i];
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

template <typename IO, int VARIANT, int RS>
hipError_t launch_recurrent_rs(const ProblemArgs& a, hipStream_t st) {
  // 32-column tiles: twice the workgroups of 64-column ones, one wave per SIMD
  const int ncols = a.dv < 32 ? a.dv : 32;
  const RecLayout L(block_tokens(RS * kRowsR, int(sizeof(IO))), RS * kRowsR, ncols, int(sizeof(IO)),
                    is_per_column(VARIANT));
  dim3 grid(a.B * a.H, a.dv / ncols), block(ncols * RS);
  hipLaunchKernelGGL((recurrent_kernel<IO, VARIANT, RS>), grid, block, size_t(L.total), st,
                     static_cast<const IO*>(a.phi_k), static_cast<const IO*>(a.phi_q),
                     static_cast<const IO*>(a.v), a.beta, a.lam, a.S0,
                     static_cast<const IO*>(a.k_prev), static_cast<IO*>(a.o), a.S_T, a.T, a.dv,
                     a.eps, a.eps_gamma);
  return hipGetLastError();
}

template <typename IO, int VARIANT>
hipError_t launch_recurrent_t(const ProblemArgs& a, hipStream_t st) {
  switch (a.dk) {
    case 16: return launch_recurrent_rs<IO, VARIANT, 2>(a, st);
    case 32: return launch_recurrent_rs<IO, VARIANT, 4>(a, st);
    case 64: return launch_recurrent_rs<IO, VARIANT, 8>(a, st);
    default: return launch_recurrent_rs<IO, VARIANT, 16>(a, st);
  }
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
