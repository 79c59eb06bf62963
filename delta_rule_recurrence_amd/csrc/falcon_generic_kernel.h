// Chunk-parallel Falcon forward, general-shape float32 kernel (gfx950).
//
// Serves every (variant, dtype, dk, dv, C) combination that has no dedicated
// kernel (the bf16 cases with dk = dv = 64 and C = 64 have their own).  All
// arithmetic is float32: the chunk's four contractions on the fp32 matrix
// cores (16- and 32-column value tiles) or on the vector ALUs (64-column
// tiles), everything else on the vector ALUs; intermediates live in LDS.
// The kernel template is instantiated once per chunk size, each in a source
// file of its own (falcon_chunked_generic_c16/c32/c64.hip) so the three
// compile in parallel; falcon_chunked_generic.hip picks the value tile and
// dispatches.
//
// Chunk algebra (derived from the Section 4 summary rules with the log-space
// renormalisation of Section 4.4, Eq. (4.16), applied per chunk with decays
// taken from chunk-local log prefixes, at window B = 1).
// For a chunk with local rows i = 0..C-1, incoming state S and per value
// column j (scalar rules use one gate column for all j):
//   g_i      = sum_{r<=i} log gamma_r             (float32, all exponents <= 0;
//              held in base-2 units, so each decay is one exp2)
//   rho_i    = eta_i r_i  (scaled residual, regression rules) solves the
//              merged residual system
//              rho_i + sum_{s<i} eta_i e^{g_{i-1}-g_s} (x_i.x_s) rho_s
//                    = eta_i (v_i - e^{g_{i-1}} (X S)_i)
//              (Section 4.2: the new values and the carried state's
//              prediction enter through the same unit-lower triangular
//              operator, so one solve per chunk covers both);
//   rho_i    = eta_i v_i                            (inner-product rules)
//   o_i      = e^{g_i} (Q S)_i + sum_{s<=i} e^{g_i-g_s} (q_i.x_s) rho_s
//   S_next   = e^{g_{C-1}} S + sum_s e^{g_{C-1}-g_s} x_s rho_s^T
// Rows past the end of the sequence get eta = 0 and log gamma = 0, so a
// ragged last chunk needs no special case.
//
// Mapping.  One workgroup of 256 threads owns one sequence and one tile of
// nv = 16 NB value columns and walks its chunks in order.  On the matrix
// cores the chunk's products are 16 x 16 tiles dealt round-robin to the four
// waves.  Elsewhere the threads form a 16 x 16 grid (ty, tx); a contraction
// gives a thread the rows ty + 16 a and the columns tx + 16 b of its output,
// so a wave reads four operand rows that sit in distinct LDS banks (row
// pitches are a multiple of 4 words plus 4) and sixteen consecutive words of
// the other operand.  Operands that run along the contraction index are read
// as float4.  Per-thread tiles have
// compile-time shapes (C / 16 chunk rows, NB value columns; key rows in
// groups of four), so no multiply-add sits behind a run-time guard.  Each
// chunk's inputs are loaded into registers in one batch at the top of the
// chunk and staged into LDS.  The substitution runs one thread per value
// column in 16-row blocks, the block's unknowns in registers; per-column
// rules also keep the solved unknowns scaled by the decay to their block's
// last row, so sums over a whole earlier block take one exp2 per column.
// Sums stop at the diagonal (s <= i), never multiplying a masked zero by a
// later row's value, so a non-finite input reaches no earlier output.
#pragma once

#include <type_traits>

#include "falcon_device.h"
#include "falcon_generic.h"

namespace falcon {

namespace generic_detail {

// Four consecutive I/O elements, loaded raw and widened when staged into LDS.
template <typename T> struct quad;
template <> struct quad<float> {
  using raw = float4;
  __device__ __forceinline__ static raw load(const float* p, int i) {
    return *reinterpret_cast<const float4*>(p + i);
  }
  __device__ __forceinline__ static raw zero() { return make_float4(0.f, 0.f, 0.f, 0.f); }
  __device__ __forceinline__ static float4 widen(raw r) { return r; }
};
template <> struct quad<bf16_t> {
  using raw = uint2;
  __device__ __forceinline__ static raw load(const bf16_t* p, int i) {
    return *reinterpret_cast<const uint2*>(p + i);
  }
  __device__ __forceinline__ static raw zero() { return make_uint2(0u, 0u); }
  __device__ __forceinline__ static float4 widen(raw r) {
    return make_float4(__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xffff0000u),
                       __uint_as_float(r.y << 16), __uint_as_float(r.y & 0xffff0000u));
  }
};

__device__ __forceinline__ float4 ld4(const float* p) {
  return *reinterpret_cast<const float4*>(p);
}
__device__ __forceinline__ void st4(float* p, float4 x) { *reinterpret_cast<float4*>(p) = x; }
__device__ __forceinline__ float dot4(float4 a, float4 b, float acc) {
  return fmaf(a.w, b.w, fmaf(a.z, b.z, fmaf(a.y, b.y, fmaf(a.x, b.x, acc))));
}
__device__ __forceinline__ float comp(float4 a, int k) {
  return k == 0 ? a.x : k == 1 ? a.y : k == 2 ? a.z : a.w;
}

typedef float f32x4v __attribute__((ext_vector_type(4)));

// Product tiles of one chunk, in order: P (MC (MC + 1) / 2 tiles on and below
// the diagonal, row-major), G (same, regression rules only), Q S (MC x NB),
// X S (regression rules only).  Tile t (wave-uniform) -> kind, row tile ta,
// column tile tb.
enum TileKind : int { kTileP = 0, kTileG = 1, kTileQS = 2, kTileXS = 3 };
template <int MC, int NB, bool kReg>
__device__ __forceinline__ void decode_tile(int t, int& kind, int& ta, int& tb) {
  constexpr int nPt = MC * (MC + 1) / 2, nSt = MC * NB;
  int u = t;
  if (u < nPt) {
    kind = kTileP;
  } else if (kReg && u < 2 * nPt) {
    kind = kTileG;
    u -= nPt;
  } else {
    u -= kReg ? 2 * nPt : nPt;
    kind = u < nSt ? kTileQS : kTileXS;
    if (u >= nSt) u -= nSt;
    ta = u / NB;
    tb = u % NB;
    return;
  }
  ta = 0;
  while ((ta + 1) * (ta + 2) / 2 <= u) ++ta;
  tb = u - ta * (ta + 1) / 2;
}

// LDS-only workgroup barrier: orders the workgroup's LDS traffic without
// waiting for its outstanding global stores.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <typename IO, int VARIANT, int C, int NB>
__global__ void __launch_bounds__(kGenericThreads)
chunked_generic_kernel(const IO* __restrict__ phi_k, const IO* __restrict__ phi_q,
                       const IO* __restrict__ v, const float* __restrict__ beta,
                       const float* __restrict__ lam, const float* S0,
                       const IO* __restrict__ k_prev, IO* __restrict__ o, float* S_T, int T,
                       int dk, int dv, int64_t BH, float eps, float eps_gamma) {
  constexpr int kThreads = kGenericThreads;
  constexpr bool kPerCol = is_per_column(VARIANT);
  constexpr bool kReg = is_regression(VARIANT);
  constexpr int MC = C / 16;                      // chunk rows (and columns) per thread
  constexpr int nv = 16 * NB;                     // value columns of the tile
  constexpr int ng = kPerCol ? nv : 1;            // gate columns
  constexpr int kXQ = C * 128 / (4 * kThreads);   // float4 groups of X (and of Q) per thread, dk <= 128
  constexpr int kV = (C * nv / 4 + kThreads - 1) / kThreads;   // float4 groups of v per thread
  constexpr int nvq = C * nv / 4;
  constexpr int lv = NB == 1 ? 2 : NB == 2 ? 3 : 4;            // log2(nv / 4)
  using Q4 = quad<IO>;
  extern __shared__ float4 lds4[];
  float* lds = reinterpret_cast<float*>(lds4);
  const GenericLayout L(C, dk, nv, ng, kReg);
  float* Xs = lds + L.off_x;      // [C][xp]  shifted keys x_i
  float* Qs = lds + L.off_q;      // [C][xp]  queries; after the products Q S as [C][nv]
  float* Ps = lds + L.off_p;      // [C][pp]  q_i.x_s for s <= i (decayed for scalar gates)
  float* Gs = lds + L.off_g;      // [C][pp]  x_i.x_s for s < i (the coupling for scalar gates)
  float* Rs = lds + L.off_r;      // [C][nv]  v, then the right-hand side, then rho
  float* St = lds + L.off_s;      // [nv][sp] state tile, transposed (S^T)
  float* Eta = lds + L.off_eta;   // [C][ng]  beta, then eta
  float* Lg = lds + L.off_lg;     // [C][ng]  inclusive prefix g of log2 gamma
  float* En = lds + L.off_en;     // [C]      energies x_i.x_i, then 2^{g_{C-1}-g_s}
  float* Lm = lds + L.off_lm;     // [C]      lam
  // [C][nv], per-column rules: Y_s = rho_s 2^{g_{P0+15}-g_s} for s in the
  // 16-row block starting at P0 (every factor <= 1), so a sum over a whole
  // earlier block needs one exp2 per column instead of one per term
  float* Ys = lds + L.off_y;

  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  // The value tiles of one sequence are workgroups 8k + x for one x: consecutive
  // workgroups go to different XCDs, so the tiles share an XCD and its L2, and
  // the keys and queries every tile reads come from HBM once.
  const int ntile = dv / nv;
  const int kk8 = blockIdx.x >> 3;
  const int64_t bh = int64_t(kk8 / ntile) * 8 + (blockIdx.x & 7);
  const int j0 = (kk8 % ntile) * nv;
  if (bh >= BH) return;
  const bool fresh = (k_prev == nullptr);
  const int mk = dk >> 4;
  const int lq = __builtin_ctz(dk >> 2);
  const int nxq = (C * dk) >> 2;

  for (int e = tid; e < dk * nv; e += kThreads) {
    const int f = e / nv, j = e % nv;
    St[j * L.sp + f] = S0 ? S0[(bh * dk + f) * dv + j0 + j] : 0.0f;
  }

  typename Q4::raw xr[kXQ], qr[kXQ], vr[kV];
  float4 br[kPerCol ? kV : 1];
  float bs = 0.f, ls = 0.f;
  // Loads of one chunk: row t0 + i of the sequence, offsets within the chunk
  // (at most C * 128 elements) from a base pointer that is uniform.
  auto fetch = [&](int t0) {
    const int rows = min(C, T - t0);
    const int64_t row0 = bh * T + t0;
    const IO* Kc = phi_k + row0 * dk;   // x_i = phi_k row t0 + i - 1: offset off - dk
    const IO* Qc = phi_q + row0 * dk;
#pragma unroll
    for (int u = 0; u < kXQ; ++u) {
      const int e = tid + u * kThreads;
      const int i = e >> lq, off = e << 2;     // i * dk + f
      xr[u] = Q4::zero();
      qr[u] = Q4::zero();
      if (e < nxq && i < rows) {
        qr[u] = Q4::load(Qc, off);
        if (t0 + i >= 1) xr[u] = Q4::load(Kc, off - dk);
        else if (!fresh) xr[u] = Q4::load(k_prev + bh * dk, off);
      }
    }
    const IO* Vc = v + row0 * dv + j0;
    const float* Bc = beta + row0 * dv + j0;
#pragma unroll
    for (int u = 0; u < kV; ++u) {
      const int e = tid + u * kThreads;
      const int i = e >> lv, j = (e & (nv / 4 - 1)) << 2;
      vr[u] = Q4::zero();
      if constexpr (kPerCol) br[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (e < nvq && i < rows) {
        vr[u] = Q4::load(Vc, i * dv + j);
        if constexpr (kPerCol) br[u] = *reinterpret_cast<const float4*>(Bc + i * dv + j);
      }
    }
    bs = 0.f;
    ls = 0.f;
    if (tid < rows) {
      if constexpr (!kPerCol) bs = beta[row0 + tid];
      ls = lam[row0 + tid];
    }
  };

  const int nchunks = (T + C - 1) / C;
  for (int c = 0; c < nchunks; ++c) {
    const int t0 = c * C;
    fetch(t0);
    lds_barrier();  // the previous chunk is done with every buffer
    // ---- stage this chunk --------------------------------------------------
#pragma unroll
    for (int u = 0; u < kXQ; ++u) {
      const int e = tid + u * kThreads;
      if (e < nxq) {
        const int i = e >> lq, f = (e & ((dk >> 2) - 1)) << 2;
        st4(Xs + i * L.xp + f, Q4::widen(xr[u]));
        st4(Qs + i * L.xp + f, Q4::widen(qr[u]));
      }
    }
#pragma unroll
    for (int u = 0; u < kV; ++u) {
      const int e = tid + u * kThreads;
      if (e < nvq) {
        const int i = e >> lv, j = (e & (nv / 4 - 1)) << 2;
        st4(Rs + i * nv + j, Q4::widen(vr[u]));
        if constexpr (kPerCol) st4(Eta + i * nv + j, br[u]);
      }
    }
    if (tid < C) {
      if constexpr (!kPerCol) Eta[tid] = bs;
      Lm[tid] = ls;
    }
    lds_barrier();

    constexpr float kLog2e = 1.44269504088896341f;
    // ---- a1, scalar gates: wave 0 forms the energies, step sizes and the
    // prefix g (one row per lane, scan across the wave) before its share of
    // the products, so the decays fold into P and G as they are stored
    if constexpr (!kPerCol) {
      if (tid < 64) {
        float eta = 0.f, lg = 0.f;
        const int t = t0 + tid;
        if (tid < C && t < T) {
          float en = 0.f;
          for (int f = 0; f < dk; f += 4) {
            const float4 x = ld4(Xs + tid * L.xp + f);
            en = dot4(x, x, en);
          }
          eta = nlms_eta(Eta[tid], en, Lm[tid], eps, fresh && t == 0);
          lg = clamped_log_gamma(eta, Lm[tid], eps_gamma) * kLog2e;
        }
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
          const float y = __shfl_up(lg, d, 64);
          if (tid >= d) lg += y;
        }
        const float glast = __shfl(lg, C - 1, 64);
        if (tid < C) {
          Eta[tid] = eta;
          Lg[tid] = lg;
          En[tid] = exp2f(glast - lg);   // state-update weight 2^{g_{C-1}-g_s}
        }
      }
    }

    // ---- products on the matrix cores: P = Q X^T and G = X X^T (16 x 16
    // tiles on and below the diagonal), Q S and X S; tiles dealt round-robin
    // to the waves.  Each lane reads four consecutive k of its A row and of its
    // B column, so four MFMAs cover 16 k (A and B share that k permutation, so
    // every dot product is unchanged).
    // 64-column tiles (NB = 4) keep the products on the vector ALUs: with 13
    // MFMA tiles per wave their register needs slowed the later phases more
    // than the matrix cores saved here.
    constexpr bool kMfma = NB <= 2;
    constexpr int nPt = MC * (MC + 1) / 2;             // tiles of P (and of G)
    constexpr int nSt = MC * NB;                       // tiles of Q S (and of X S)
    constexpr int nTiles = (nPt + nSt) * (kReg ? 2 : 1);
    constexpr int kPerWave = (nTiles + 3) / 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), ln = tid & 63;
    const int lr = ln & 15, lk = 4 * (ln >> 4);
    f32x4v tacc[kMfma ? kPerWave : 1];
#pragma unroll
    for (int q = 0; q < (kMfma ? kPerWave : 1); ++q) tacc[q] = f32x4v{0.f, 0.f, 0.f, 0.f};
    // one code path per wave, so that each unrolled tile number is a constant
    // and the tile's kind and place fold at compile time
    auto products = [&](auto wave) {
      constexpr int W = decltype(wave)::value;
#pragma unroll
      for (int q = 0; q < kPerWave; ++q) {
        const int t = W + 4 * q;
        if (t < nTiles) {
          int kind, ta, tb;
          decode_tile<MC, NB, kReg>(t, kind, ta, tb);
          const float* Ap = (kind == kTileP || kind == kTileQS ? Qs : Xs) + (16 * ta + lr) * L.xp + lk;
          const float* Bp = kind <= kTileG ? Xs + (16 * tb + lr) * L.xp + lk
                                           : St + (16 * tb + lr) * L.sp + lk;
#pragma unroll 2
          for (int f = 0; f < dk; f += 16) {
            const float4 av = ld4(Ap + f), bv = ld4(Bp + f);
            tacc[q] = __builtin_amdgcn_mfma_f32_16x16x4f32(av.x, bv.x, tacc[q], 0, 0, 0);
            tacc[q] = __builtin_amdgcn_mfma_f32_16x16x4f32(av.y, bv.y, tacc[q], 0, 0, 0);
            tacc[q] = __builtin_amdgcn_mfma_f32_16x16x4f32(av.z, bv.z, tacc[q], 0, 0, 0);
            tacc[q] = __builtin_amdgcn_mfma_f32_16x16x4f32(av.w, bv.w, tacc[q], 0, 0, 0);
          }
        }
      }
    };
    // register tiles (vector ALUs): rows ty + 16 a, columns tx + 16 b
    float pa[MC][MC], ga[MC][MC], qs[MC][NB], xs[MC][NB];
    if constexpr (kMfma) {
      switch (w) {
        case 0: products(std::integral_constant<int, 0>{}); break;
        case 1: products(std::integral_constant<int, 1>{}); break;
        case 2: products(std::integral_constant<int, 2>{}); break;
        default: products(std::integral_constant<int, 3>{}); break;
      }
    } else {
#pragma unroll
      for (int a = 0; a < MC; ++a) {
#pragma unroll
        for (int b = 0; b < MC; ++b) pa[a][b] = ga[a][b] = 0.f;
#pragma unroll
        for (int b = 0; b < NB; ++b) qs[a][b] = xs[a][b] = 0.f;
      }
      for (int f = 0; f < dk; f += 4) {
        float4 qi[MC], xi[MC], xc[MC], sv[NB];
#pragma unroll
        for (int a = 0; a < MC; ++a) {
          qi[a] = ld4(Qs + (ty + 16 * a) * L.xp + f);
          if (kReg) xi[a] = ld4(Xs + (ty + 16 * a) * L.xp + f);
          xc[a] = ld4(Xs + (tx + 16 * a) * L.xp + f);
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) sv[b] = ld4(St + (tx + 16 * b) * L.sp + f);
#pragma unroll
        for (int a = 0; a < MC; ++a) {
#pragma unroll
          for (int b = 0; b <= a; ++b) {   // tiles with b > a lie above the diagonal
            pa[a][b] = dot4(qi[a], xc[b], pa[a][b]);
            if (kReg) ga[a][b] = dot4(xi[a], xc[b], ga[a][b]);
          }
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            qs[a][b] = dot4(qi[a], sv[b], qs[a][b]);
            if (kReg) xs[a][b] = dot4(xi[a], sv[b], xs[a][b]);
          }
        }
      }
    }

    if constexpr (kPerCol) {
      // ---- per-column gates follow the products ------------------------------
      if (tid < C) {
        float en = 0.f;
        for (int f = 0; f < dk; f += 4) {
          const float4 x = ld4(Xs + tid * L.xp + f);
          en = dot4(x, x, en);
        }
        En[tid] = en;
      }
      lds_barrier();
      for (int e = tid; e < C * ng; e += kThreads) {
        const int i = e >> (lv + 2);
        const int t = t0 + i;
        float eta = 0.f, lg = 0.f;
        if (t < T) {
          eta = nlms_eta(Eta[e], En[i], Lm[i], eps, fresh && t == 0);
          lg = clamped_log_gamma(eta, Lm[i], eps_gamma) * kLog2e;
        }
        Eta[e] = eta;
        Lg[e] = lg;
      }
      lds_barrier();
      if (tid < ng) {
        float acc = 0.f;
        for (int i = 0; i < C; ++i) {
          acc += Lg[i * ng + tid];
          Lg[i * ng + tid] = acc;
        }
      }
    }
    lds_barrier();   // gates and prefix visible

    // ---- tiles to LDS: P and G masked (and, for scalar gates, decayed), Q S;
    // X S becomes the right-hand side eta (v - 2^{g_{i-1}} X S) in place
    // (tile element r of a lane: row 16 ta + lk + r, column 16 tb + lr)
    auto store_tiles = [&](auto wave) {
      constexpr int W = decltype(wave)::value;
#pragma unroll
      for (int q = 0; q < kPerWave; ++q) {
        const int t = W + 4 * q;
        if (t < nTiles) {
          int kind, ta, tb;
          decode_tile<MC, NB, kReg>(t, kind, ta, tb);
          const int col = 16 * tb + lr;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = 16 * ta + lk + r;
            const float v = tacc[q][r];
            if (kind == kTileP) {
              float p = 0.f;
              if (col <= i) p = kPerCol ? v : v * exp2f(Lg[i] - Lg[col]);
              Ps[i * L.pp + col] = p;
            } else if (kind == kTileG) {
              float g = 0.f;
              if (col < i) g = kPerCol ? v : v * Eta[i] * exp2f(Lg[max(i - 1, 0)] - Lg[col]);
              Gs[i * L.pp + col] = g;
            } else if (kind == kTileQS) {
              Qs[i * nv + col] = v;
            } else {
              const int cc = kPerCol ? col : 0;
              const float gprev = i > 0 ? Lg[(i - 1) * ng + cc] : 0.0f;
              float& rr = Rs[i * nv + col];
              rr = Eta[i * ng + cc] * fmaf(exp2f(gprev), -v, rr);
            }
          }
        }
      }
    };
    if constexpr (kMfma) {
      switch (w) {
        case 0: store_tiles(std::integral_constant<int, 0>{}); break;
        case 1: store_tiles(std::integral_constant<int, 1>{}); break;
        case 2: store_tiles(std::integral_constant<int, 2>{}); break;
        default: store_tiles(std::integral_constant<int, 3>{}); break;
      }
    } else {
#pragma unroll
      for (int a = 0; a < MC; ++a) {
        const int i = ty + 16 * a;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const int j = tx + 16 * b;
          Qs[i * nv + j] = qs[a][b];
          if (kReg) {
            const int cc = kPerCol ? j : 0;
            const float gprev = i > 0 ? Lg[(i - 1) * ng + cc] : 0.0f;
            float& r = Rs[i * nv + j];
            r = Eta[i * ng + cc] * fmaf(exp2f(gprev), -xs[a][b], r);
          }
        }
        const float gi = kPerCol ? 0.f : Lg[i * ng];
        const float gi1 = kPerCol ? 0.f : Lg[max(i - 1, 0) * ng];
        const float ei = kPerCol ? 0.f : Eta[i * ng];
#pragma unroll
        for (int b = 0; b < MC; ++b) {
          const int s2 = tx + 16 * b;
          float p = 0.f, g = 0.f;
          if (b <= a && s2 <= i) p = kPerCol ? pa[a][b] : pa[a][b] * exp2f(gi - Lg[s2 * ng]);
          if (kReg && b <= a && s2 < i) g = kPerCol ? ga[a][b] : ga[a][b] * ei * exp2f(gi1 - Lg[s2 * ng]);
          Ps[i * L.pp + s2] = p;
          if (kReg) Gs[i * L.pp + s2] = g;
        }
      }
    }
    if constexpr (!kReg) {
#pragma unroll
      for (int a = 0; a < MC; ++a) {
        const int i = ty + 16 * a;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const int j = tx + 16 * b;
          const int cc = kPerCol ? j : 0;
          float& r = Rs[i * nv + j];
          r = Eta[i * ng + cc] * r;   // rho = eta v
          if (kPerCol) Ys[i * nv + j] = r * exp2f(Lg[(16 * a + 15) * ng + j] - Lg[i * ng + j]);
        }
      }
    }
    lds_barrier();

    // ---- a2/a3: forward substitution of the merged residual system --------
    // 16-row blocks.  Before block B0 is solved, all threads subtract the
    // contributions of the solved rows s < B0 from its right-hand sides (row
    // B0 + ty, columns tx + 16 b); then one thread per value column solves the
    // block's 16 x 16 lower triangle in registers.
    if constexpr (kReg) {
      for (int B0 = 0; B0 < C; B0 += 16) {
        if (B0 > 0) {
          const int i = B0 + ty;
          float acc[NB], gref[NB];
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            acc[b] = 0.f;
            // per-column gates: 2^{g_{i-1}-g_s} = 2^{g_{i-1}-g_ref} 2^{g_ref-g_s} with
            // g_ref = g_{B0-1}; both factors are <= 1 since g never increases
            gref[b] = kPerCol ? Lg[(B0 - 1) * ng + tx + 16 * b] : 0.f;
          }
          for (int P0 = 0; P0 < B0; P0 += 16) {
            float sc[NB];   // per-column gates: 2^{g_ref-g_{P0+15}} <= 1 rescales Y
#pragma unroll
            for (int b = 0; b < NB; ++b)
              sc[b] = kPerCol ? exp2f(gref[b] - Lg[(P0 + 15) * ng + tx + 16 * b]) : 1.f;
#pragma unroll
            for (int s0 = P0; s0 < P0 + 16; s0 += 4) {
              const float4 g = ld4(Gs + i * L.pp + s0);
#pragma unroll
              for (int k = 0; k < 4; ++k)
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                  const int j = tx + 16 * b;
                  const float rv = kPerCol ? Ys[(s0 + k) * nv + j] * sc[b] : Rs[(s0 + k) * nv + j];
                  acc[b] = fmaf(comp(g, k), rv, acc[b]);
                }
            }
          }
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            const int j = tx + 16 * b;
            if (kPerCol) acc[b] *= Eta[i * ng + j] * exp2f(Lg[(i - 1) * ng + j] - gref[b]);
            Rs[i * nv + j] -= acc[b];
          }
          lds_barrier();
        }
        if (tid < nv) {
          const int j = tid;
          float r[16], eB[16], gB[16];
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) {
            const int i = B0 + rr;
            r[rr] = Rs[i * nv + j];
            if (kPerCol) {
              eB[rr] = Eta[i * ng + j];
              gB[rr] = i > 0 ? Lg[(i - 1) * ng + j] : 0.f;
            }
          }
          if constexpr (kPerCol) {
            // per-column gates: the decay 2^{g_{i-1}-g_s} between two rows of
            // the block is the product of the gammas of rows s+1..i-1; each row
            // walks its terms from s = i-1 down, extending the product, so the
            // decays never wait on the unknowns.  gm[m] = gamma of row B0 + m.
            float gm[16];
#pragma unroll
            for (int m = 1; m < 15; ++m) gm[m] = exp2f(gB[m + 1] - gB[m]);
            gm[0] = 1.f;
#pragma unroll
            for (int rr = 1; rr < 16; ++rr) {
              const float* gi = Gs + (B0 + rr) * L.pp + B0;
              float4 gv[4];
#pragma unroll
              for (int q = 0; q < 4; ++q)
                if (4 * q < rr) gv[q] = ld4(gi + 4 * q);
              float d = eB[rr], a0 = 0.f, a1 = 0.f;
#pragma unroll
              for (int ss = rr - 1; ss >= 0; --ss) {
                const float cf = comp(gv[ss >> 2], ss & 3) * d;
                if (ss & 1) a1 = fmaf(cf, r[ss], a1);
                else a0 = fmaf(cf, r[ss], a0);
                if (ss > 0) d *= gm[ss];
              }
              r[rr] -= a0 + a1;
            }
            // decay-scaled copy: Y_{B0+ss} = r_ss prod_{m=ss+1..15} gamma_{B0+m}
            gm[15] = exp2f(Lg[(B0 + 15) * ng + j] - gB[15]);
            float fsc = 1.f;
            Ys[(B0 + 15) * nv + j] = r[15];
#pragma unroll
            for (int ss = 14; ss >= 0; --ss) {
              fsc *= gm[ss + 1];
              Ys[(B0 + ss) * nv + j] = r[ss] * fsc;
            }
          } else {
#pragma unroll
            for (int rr = 1; rr < 16; ++rr) {
              const float* gi = Gs + (B0 + rr) * L.pp + B0;
              float a0 = 0.f, a1 = 0.f;
#pragma unroll
              for (int s4 = 0; s4 < rr; s4 += 4) {
                const float4 g = ld4(gi + s4);
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                  if (s4 + k < rr) {
                    if (k & 1) a1 = fmaf(comp(g, k), r[s4 + k], a1);
                    else a0 = fmaf(comp(g, k), r[s4 + k], a0);
                  }
                }
              }
              r[rr] -= a0 + a1;
            }
          }
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) Rs[(B0 + rr) * nv + j] = r[rr];
        }
        lds_barrier();
      }
    }

    // ---- a4: outputs, and for scalar gates the state update of key rows
    // 4 ty + a (a < 4) in the same walk over the rows of rho (16- and 32-column
    // tiles; with 64 columns the extra registers cost more than the shared
    // loads save) ---------------------------------------------------------------
    constexpr bool kFuse = !kPerCol && NB <= 2;
    const int fb0 = (4 * ty) & (dk - 1);
    float sacc0[4][NB];
    if constexpr (kFuse) {
      const float dl = exp2f(Lg[C - 1]);
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const float4 s4v = ld4(St + (tx + 16 * b) * L.sp + fb0);
#pragma unroll
        for (int a = 0; a < 4; ++a) sacc0[a][b] = dl * comp(s4v, a);
      }
    }
    {
      float acc[MC][NB], gi[MC][NB];
#pragma unroll
      for (int a = 0; a < MC; ++a)
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const int i = ty + 16 * a, j = tx + 16 * b;
          gi[a][b] = Lg[i * ng + (kPerCol ? j : 0)];
          acc[a][b] = exp2f(gi[a][b]) * Qs[i * nv + j];   // Q S
        }
      if constexpr (!kPerCol) {
        // P carries the decays: plain sums, the select only in the diagonal block
#pragma unroll 1
        for (int sb = 0; sb < MC; ++sb) {
#pragma unroll 4
          for (int s4 = 0; s4 < 16; s4 += 4) {
            const int s = 16 * sb + s4;
            float rv[4][NB];
#pragma unroll
            for (int k = 0; k < 4; ++k)
#pragma unroll
              for (int b = 0; b < NB; ++b) rv[k][b] = Rs[(s + k) * nv + tx + 16 * b];
#pragma unroll
            for (int a = 0; a < MC; ++a) {
              if (a < sb) continue;   // above the diagonal (static index, uniform skip)
              const float4 p = ld4(Ps + (ty + 16 * a) * L.pp + s);
#pragma unroll
              for (int k = 0; k < 4; ++k) {
                // in the diagonal block only the columns s <= i take part
                const bool on = a > sb || s4 + k <= ty;
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                  const float nx = fmaf(comp(p, k), rv[k][b], acc[a][b]);
                  acc[a][b] = on ? nx : acc[a][b];
                }
              }
            }
            // state rows 4 ty + a: S += 2^{g_{C-1}-g_s} x_s rho_s^T for these four s
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const float4 xv = ld4(Xs + (s + k) * L.xp + fb0);
              const float w = En[s + k];
#pragma unroll
              for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < NB; ++b)
                  sacc0[a][b] = fmaf(comp(xv, a) * w, rv[k][b], sacc0[a][b]);
            }
          }
        }
      } else {
        // per-column gates: an earlier block sb contributes
        // 2^{g_i - g_end} sum_s P_is Y_s (g_end = g_{16 sb + 15}, one exp2 per
        // block and column); the diagonal block takes one exp2 per term
#pragma unroll 1
        for (int sb = 0; sb < MC; ++sb) {
          float gend[NB], part[MC][NB];
#pragma unroll
          for (int b = 0; b < NB; ++b) gend[b] = Lg[(16 * sb + 15) * ng + tx + 16 * b];
#pragma unroll
          for (int a = 0; a < MC; ++a)
#pragma unroll
            for (int b = 0; b < NB; ++b) part[a][b] = 0.f;
#pragma unroll 2
          for (int s4 = 0; s4 < 16; s4 += 4) {
            const int s = 16 * sb + s4;
            float yv[4][NB], rv[4][NB], gs[4][NB];
#pragma unroll
            for (int k = 0; k < 4; ++k)
#pragma unroll
              for (int b = 0; b < NB; ++b) {
                const int j = tx + 16 * b;
                yv[k][b] = Ys[(s + k) * nv + j];
                rv[k][b] = Rs[(s + k) * nv + j];
                gs[k][b] = Lg[(s + k) * ng + j];
              }
#pragma unroll
            for (int a = 0; a < MC; ++a) {
              if (a < sb) continue;   // above the diagonal (static index, uniform skip)
              const float4 p = ld4(Ps + (ty + 16 * a) * L.pp + s);
              if (a > sb) {
#pragma unroll
                for (int k = 0; k < 4; ++k)
#pragma unroll
                  for (int b = 0; b < NB; ++b) part[a][b] = fmaf(comp(p, k), yv[k][b], part[a][b]);
              } else {
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                  const bool on = s4 + k <= ty;   // columns s <= i only
#pragma unroll
                  for (int b = 0; b < NB; ++b) {
                    const float cf = comp(p, k) * exp2f(gi[a][b] - gs[k][b]);
                    const float nx = fmaf(cf, rv[k][b], acc[a][b]);
                    acc[a][b] = on ? nx : acc[a][b];
                  }
                }
              }
            }
          }
#pragma unroll
          for (int a = 0; a < MC; ++a)
            if (a > sb) {
#pragma unroll
              for (int b = 0; b < NB; ++b)
                acc[a][b] = fmaf(exp2f(gi[a][b] - gend[b]), part[a][b], acc[a][b]);
            }
        }
      }
#pragma unroll
      for (int a = 0; a < MC; ++a) {
        const int t = t0 + ty + 16 * a;
        if (t < T) {
#pragma unroll
          for (int b = 0; b < NB; ++b)
            io<IO>::store(o, (bh * T + t) * dv + j0 + tx + 16 * b, acc[a][b]);
        }
      }
    }

    // ---- a3: state update S = 2^{g_{C-1}} S + sum_s 2^{g_{C-1}-g_s} x_s rho_s^T
    // (reads X, rho and the weights, all final; each thread owns its S entries:
    // key rows f0 + 4 ty + a, a < 4, for f0 = 0, 64; rows past dk wrap onto
    // valid ones and are not stored)
    {
      float glast[NB], dlast[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        glast[b] = Lg[(C - 1) * ng + (kPerCol ? tx + 16 * b : 0)];
        dlast[b] = exp2f(glast[b]);
      }
      if constexpr (kFuse) {
        if (4 * ty < dk) {
#pragma unroll
          for (int b = 0; b < NB; ++b)
            st4(St + (tx + 16 * b) * L.sp + fb0,
                make_float4(sacc0[0][b], sacc0[1][b], sacc0[2][b], sacc0[3][b]));
        }
      }
      for (int f0 = kFuse ? 64 : 0; f0 < dk; f0 += 64) {
        const bool own = f0 + 4 * ty < dk;
        const int fb = (f0 + 4 * ty) & (dk - 1);
        float sacc[4][NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const float4 s4v = ld4(St + (tx + 16 * b) * L.sp + fb);
#pragma unroll
          for (int a = 0; a < 4; ++a) sacc[a][b] = dlast[b] * comp(s4v, a);
        }
        for (int P0 = 0; P0 < C; P0 += 16) {
          float sc[NB];   // per-column gates: 2^{g_{C-1}-g_{P0+15}} <= 1 rescales Y
#pragma unroll
          for (int b = 0; b < NB; ++b)
            sc[b] = kPerCol ? exp2f(glast[b] - Lg[(P0 + 15) * ng + tx + 16 * b]) : 1.f;
#pragma unroll 4
          for (int s = P0; s < P0 + 16; ++s) {
            float rw[NB];
#pragma unroll
            for (int b = 0; b < NB; ++b) {
              const int j = tx + 16 * b;
              rw[b] = kPerCol ? Ys[s * nv + j] * sc[b] : Rs[s * nv + j] * En[s];
            }
            const float4 xv = ld4(Xs + s * L.xp + fb);
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
              for (int b = 0; b < NB; ++b) sacc[a][b] = fmaf(comp(xv, a), rw[b], sacc[a][b]);
          }
        }
        if (own) {
#pragma unroll
          for (int b = 0; b < NB; ++b)
            st4(St + (tx + 16 * b) * L.sp + fb,
                make_float4(sacc[0][b], sacc[1][b], sacc[2][b], sacc[3][b]));
        }
      }
    }
  }
  __syncthreads();
  if (S_T) {
    for (int e = tid; e < dk * nv; e += kThreads) {
      const int f = e / nv, j = e % nv;
      S_T[(bh * dk + f) * dv + j0 + j] = St[j * L.sp + f];
    }
  }
}

template <typename IO, int VARIANT, int C, int NB>
hipError_t launch_one(const ProblemArgs& a, size_t lds, hipStream_t st) {
  auto kern = chunked_generic_kernel<IO, VARIANT, C, NB>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(lds));
  if (e != hipSuccess) return e;
  const int64_t BH = int64_t(a.B) * a.H;
  const int64_t blocks = (BH + 7) / 8 * 8 * (a.dv / (16 * NB));
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(blocks)), dim3(kGenericThreads), lds, st,
                     static_cast<const IO*>(a.phi_k), static_cast<const IO*>(a.phi_q),
                     static_cast<const IO*>(a.v), a.beta, a.lam, a.S0,
                     static_cast<const IO*>(a.k_prev), static_cast<IO*>(a.o), a.S_T, a.T, a.dk,
                     a.dv, BH, a.eps, a.eps_gamma);
  return hipGetLastError();
}

template <typename IO, int VARIANT, int C>
hipError_t launch_tile(const ProblemArgs& a, int nv, size_t lds, hipStream_t st) {
  switch (nv) {
    case 16: return launch_one<IO, VARIANT, C, 1>(a, lds, st);
    case 32: return launch_one<IO, VARIANT, C, 2>(a, lds, st);
    default: return launch_one<IO, VARIANT, C, 4>(a, lds, st);
  }
}

template <typename IO, int C>
hipError_t launch_variant(const ProblemArgs& a, int nv, size_t lds, hipStream_t st) {
  switch (a.variant) {
    case kF1: return launch_tile<IO, kF1, C>(a, nv, lds, st);
    case kF1A: return launch_tile<IO, kF1A, C>(a, nv, lds, st);
    case kF2: return launch_tile<IO, kF2, C>(a, nv, lds, st);
    default: return launch_tile<IO, kF2A, C>(a, nv, lds, st);
  }
}

}  // namespace generic_detail

template <int C>
hipError_t launch_generic_c(const ProblemArgs& a, int nv, size_t lds, hipStream_t st) {
  return a.bf16 ? generic_detail::launch_variant<bf16_t, C>(a, nv, lds, st)
                : generic_detail::launch_variant<float, C>(a, nv, lds, st);
}

}  // namespace falcon
