// Chunked Falcon-1 forward (gfx950, bf16 I/O, dk = dv = 64, chunk C = 64),
// in one launch by default or in two.
//
// The chunk form (the log-space renormalisation of Section 4.4 with window 1,
// applied per chunk; g_i the chunk-local prefix of log gamma):
//   A_{i,s} = eta_i e^{g_{i-1}-g_s} (x_i . x_s) for s < i,   T = (I + A)^{-1}
//   W = T Diag(eta e^{g_{s-1}}) X,   U = T Diag(eta) V,   R = U - W S
//   S' = e^{g_63} S + Xh^T R,   Xh = Diag(e^{g_63-g}) X
//   O = Diag(e^g) Q S + M R,    M = tril0(Q X^T) o [e^{g_i-g_s}].
// W and U depend only on the chunk's own keys, values and gates (the "WY"
// factors of Section 4.2's chunk-parallel implementation), and so do the
// products that carry S through the chunk.  Substituting R:
//   S' = e^{g_63} S + K S + H,   K = -Xh^T W,   H = Xh^T U
//   O  = Qt S + Ot,              Qt = Diag(e^g) Q - M W,   Ot = M U.
// Chunk workgroups build K, H, Qt and Ot for every chunk of every sequence at
// once (one workgroup per chunk) and write them to the workspace in MFMA
// operand order.  The short sequential part runs per sequence: per chunk, one
// 64x64x64 product for the state and one for the outputs, reading the chunk
// matrices back.  In the one-launch form (the default) chain workgroups run
// beside the chunk workgroups and take each chunk as soon as it is announced;
// in the two-launch form all chunk matrices come first.  The state is rounded
// to bf16 only as the operand of K S and Qt S; its decay term stays in
// float32.

#include <stdint.h>
#include <stdlib.h>

#include <vector>

#include "falcon_device.h"
#include "falcon_launch.h"
#include "falcon_mfma_frag.h"

namespace falcon {

namespace {

using namespace frag;

constexpr int kC = 64;
constexpr int kD = 64;
constexpr int kP = 72;                  // bf16 row pitch of T in LDS
// Per-chunk block in the workspace (bf16 element offsets), 32 KiB:
constexpr int kBlockElems = 16384;
constexpr int kOutK = 0;                // K as A fragments [fb][m][lane][8]
constexpr int kOutQt = 4096;            // Qt as B fragments [ib][m][lane][8]
constexpr int kOutH = 8192;             // H as result tiles [cb][fb][lane][4]
constexpr int kOutOt = 12288;           // Ot^T as result tiles [cb][ib][lane][4]
// followed, after all blocks, by e^{g_63} of every chunk (float).

struct Seq {
  const bf16_t* K;
  const bf16_t* Q;
  const bf16_t* V;
  const float* beta;
  const float* lam;
  const bf16_t* k_prev;
  int T;
};

__device__ __forceinline__ Seq make_seq(const bf16_t* phi_k, const bf16_t* phi_q, const bf16_t* v,
                                        const float* beta, const float* lam, const bf16_t* k_prev,
                                        int64_t bh, int T) {
  Seq sq;
  sq.K = phi_k + bh * T * kD;
  sq.Q = phi_q ? phi_q + bh * T * kD : nullptr;
  sq.V = v ? v + bh * T * kD : nullptr;
  sq.beta = beta + bh * T;
  sq.lam = lam + bh * T;
  sq.k_prev = k_prev ? k_prev + bh * kD : nullptr;
  sq.T = T;
  return sq;
}

// Key row r of chunk c (phi(k_{t0+r-1}); the fresh-start row and rows past
// the sequence read a valid row, their step size is 0).
__device__ __forceinline__ const bf16_t* key_row(const Seq& sq, int c, int r) {
  const int kt = c * kC + r - 1;
  if (kt < 0) return sq.k_prev ? sq.k_prev : sq.K;
  return sq.K + int64_t(kt < sq.T ? kt : sq.T - 1) * kD;
}
__device__ __forceinline__ const bf16_t* token_row(const bf16_t* base, const Seq& sq, int c, int r) {
  const int t = c * kC + r;
  return base + int64_t(t < sq.T ? t : sq.T - 1) * kD;
}

// ============================================================================
// Launch 1: chunk matrices, one chunk per workgroup (four waves).
//
// "frag(Z)[b][m]" below is the operand fragment of row block b of a matrix Z
// with k = 32 m + kperm: lane l holds Z[16 b + (l & 15)][32 m + kperm(l >> 4, e)].
// A product of frag(P) and frag(Q) gives the tile P Q^T; two such tiles
// stacked over consecutive row blocks of P are frag(Q P^T).
// ============================================================================

struct WyGates {
  float graw[kC];                 // g_s, token order
  float sxg[kC];                  // eta_s e^{g_{s-1}}
  float sxh[kC];                  // e^{g_63 - g_s}
  float eta[kC];                  // eta_s
  float eta_t[kC];                // eta_i at [c16 * 4 + ib] for i = 16 ib + c16
  float gprev_t[kC];              // g_{i-1}, same order
  float e63;                      // e^{g_63}
};

struct WySmem {
  uint16_t x[kC * kD];            // keys (swizzled rows); then frag(-W^T) [fb][m][lane][8]
  uint16_t xh[kC * kD];           // frag(Xh^T) [fb][m][lane][8]
  uint16_t ut[kC * kD];           // values (swizzled rows); then frag(U^T) [cb][m][lane][8]
  uint16_t tb[kC * kP];           // T, row-major
  float abt[4][16][16];           // diagonal blocks of -A: [b][s][i] = -A[16b+i][16b+s]
  WyGates G;
  int go;                         // the output policy's verdict, shared by the waves
};

// T = (I + A)^{-1} into sm.tb (wave 0): the decayed Gram on MFMA, the four
// 16x16 diagonal blocks by column elimination in registers, then two levels of
// MFMA block products.
__device__ __forceinline__ void build_inverse(WySmem& sm, int l) {
  const int g = l >> 4, c16 = l & 15;
  uint16_t* tb = sm.tb;
  bf16x8 xf[4][2];
#pragma unroll
  for (int ib = 0; ib < 4; ++ib)
#pragma unroll
    for (int m = 0; m < 2; ++m) xf[ib][m] = ring_frag_c(sm.x, 16 * ib + c16, m, g);
  const f32x4 eta_i = ld4(&sm.G.eta_t[c16 * 4]);
  const f32x4 gpv_i = ld4(&sm.G.gprev_t[c16 * 4]);
  f32x4 gs_s[4];                                           // g_s for s = 16 sb + 4 g + r
#pragma unroll
  for (int sb = 0; sb < 4; ++sb) gs_s[sb] = ld4(&sm.G.graw[16 * sb + 4 * g]);
  s16x4 a10, a32;      // A blocks (1,0) and (3,2) as K=16 A fragments
  bf16x8 a2lo, a3lo;   // A rows 32-47 / 48-63, columns 0-31, as K=32 A fragments
  {
    f32x4 a_off[6];
#pragma unroll
    for (int n = 0; n < 10; ++n) {
      int ib, sb;
      lower_tile(n, ib, sb);
      // A^T tile (sb, ib): lane holds A[16ib+c16][16sb+4g+r]
      f32x4 acc = mfma32(xf[sb][0], xf[ib][0], zero4());
      acc = mfma32(xf[sb][1], xf[ib][1], acc);
      const int i = 16 * ib + c16;
      f32x4 a;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int s_ = 16 * sb + 4 * g + r;
        a[r] = s_ < i ? eta_i[ib] * __expf(gpv_i[ib] - gs_s[sb][r]) * acc[r] : 0.0f;
      }
      if (ib == sb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) sm.abt[ib][4 * g + r][c16] = -a[r];
      } else {
        a_off[n - ib] = a;     // n - ib enumerates the off-diagonal tiles in order
      }
    }
    a10 = s16_acc(a_off[0]);
    a32 = s16_acc(a_off[5]);
    a2lo = frag_acc(a_off[1], a_off[2]);
    a3lo = frag_acc(a_off[3], a_off[4]);
  }
  {
    float t[16], ncol[16];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const f32x4 v = ld4(&sm.abt[g][c16][4 * q4]);          // -A[16g+i][16g+c16], all i
      ncol[4 * q4] = v[0]; ncol[4 * q4 + 1] = v[1]; ncol[4 * q4 + 2] = v[2]; ncol[4 * q4 + 3] = v[3];
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) t[i] = (i == c16) ? 1.0f : 0.0f;
    eliminate16(t, ncol);
#pragma unroll
    for (int i = 0; i < 16; ++i) tb[(16 * g + i) * kP + 16 * g + c16] = bf(t[i]);
  }
  // off-diagonal 16x16 blocks: T_hl = -T_hh A_hl T_ll for (1,0), (3,2)
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int lo = 2 * p, hi = 2 * p + 1;
    s16x4 tl;
#pragma unroll
    for (int e = 0; e < 4; ++e) tl[e] = static_cast<short>(tb[(16 * lo + 4 * g + e) * kP + 16 * lo + c16]);
    const f32x4 y = mfma16(p == 0 ? a10 : a32, tl, zero4());
    const s16x4 th = __builtin_bit_cast(
        s16x4, *reinterpret_cast<const uint2*>(&tb[(16 * hi + c16) * kP + 16 * hi + 4 * g]));
    const f32x4 z = mfma16(th, s16_acc(y), zero4());
#pragma unroll
    for (int r = 0; r < 4; ++r) tb[(16 * hi + 4 * g + r) * kP + 16 * lo + c16] = bf(-z[r]);
  }
  // lower-left 32x32 block: T_21 = -T_22 A_21 T_11 (2x2 block sense)
  {
    bf16x8 tlo[2];
#pragma unroll
    for (int cj = 0; cj < 2; ++cj)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        tlo[cj][e] = __builtin_bit_cast(__bf16, tb[kperm(g, e) * kP + 16 * cj + c16]);
    const bf16x8 th2 = frag_lds(&tb[(32 + c16) * kP], 32, g);
    const bf16x8 th3 = frag_lds(&tb[(48 + c16) * kP], 32, g);
#pragma unroll
    for (int cj = 0; cj < 2; ++cj) {
      const bf16x8 yb = frag_acc(mfma32(a2lo, tlo[cj], zero4()), mfma32(a3lo, tlo[cj], zero4()));
      const f32x4 z2 = mfma32(th2, yb, zero4());
      const f32x4 z3 = mfma32(th3, yb, zero4());
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        tb[(32 + 4 * g + r) * kP + 16 * cj + c16] = bf(-z2[r]);
        tb[(48 + 4 * g + r) * kP + 16 * cj + c16] = bf(-z3[r]);
      }
    }
  }
}

// Fragment slot [b][m] of a 64x64 fragment array.
__host__ __device__ inline int fslot(int b, int m, int l) { return ((b * 2 + m) * 64 + l) * 8; }

__device__ __forceinline__ bf16x8 ldg_frag(const bf16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}
__device__ __forceinline__ uint2 ldg_half(const bf16_t* p) { return *reinterpret_cast<const uint2*>(p); }
__device__ __forceinline__ f32x4 unpack_half(uint2 v) {
  return f32x4{__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
               __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u)};
}

// The chunk matrices of chunk c of sequence bh, computed by one workgroup of
// four waves and handed to `out`: out.prefetch() is called at the start,
// out.acquire() by every wave before the first store (it returns the same
// verdict in every wave; false: store nothing); each wave then stores its
// row block of K and H to out.block() (element offsets Out::kK, Out::kH), the
// wave holding the gates stores e^{g_63} to out.decay(), and every wave hands
// its token block of Qt (fragments) and of Ot^T (bf16 tiles) to out.finish().
//
// Every global load is issued at the start, so a workgroup waits for memory
// once.  Keys and values are staged in LDS; each wave's queries and the gate
// inputs go straight into registers.  Wave w owns token block ib = w of the
// read mask M, Qt and Ot, and row block w of K and H.
template <class Out>
__device__ __forceinline__ void wy_chunk(WySmem& sm, const bf16_t* __restrict__ phi_k,
                                         const bf16_t* __restrict__ phi_q, const bf16_t* __restrict__ v,
                                         const float* __restrict__ beta, const float* __restrict__ lam,
                                         const bf16_t* __restrict__ k_prev, int64_t bh, int c, int T,
                                         float eps, float eps_gamma, Out& out) {
  const int tid = threadIdx.x;
  // role index: wave-uniform (so role branches are scalar) and rotated by the
  // workgroup, so the long inverse role is spread over the SIMDs
  const int w = (__builtin_amdgcn_readfirstlane(tid >> 6) + int(blockIdx.x)) & 3, l = tid & 63;
  const int g = l >> 4, c16 = l & 15;
  const Seq sq = make_seq(phi_k, phi_q, v, beta, lam, k_prev, bh, T);
  const bool fresh = (k_prev == nullptr);
  out.prefetch(w);

  // ---- stage keys and values (wave w rows 16w..16w+15); fetch this wave's
  // queries and, for the gates, beta and lam of token c * 64 + l --------------
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = 16 * w + 8 * j + (l >> 3);
    const int off = r * kD + 8 * seg_pos(r, l & 7);
    *reinterpret_cast<bf16x8*>(sm.x + off) = *reinterpret_cast<const bf16x8*>(key_row(sq, c, r) + 8 * (l & 7));
    *reinterpret_cast<bf16x8*>(sm.ut + off) = *reinterpret_cast<const bf16x8*>(token_row(sq.V, sq, c, r) + 8 * (l & 7));
  }
  const int gtok = c * kC + l < T ? c * kC + l : T - 1;
  const float beta_l = sq.beta[gtok], lam_l = sq.lam[gtok];
  // query row i = 16w + c16: contiguous fragments for Q X^T, and Q[i][16fb+4g..+3]
  const bf16_t* qrow = token_row(sq.Q, sq, c, 16 * w + c16);
  const bf16x8 qa0 = ldg_frag(qrow + 8 * g);
  const bf16x8 qa1 = ldg_frag(qrow + 32 + 8 * g);
  uint2 qi[4];
#pragma unroll
  for (int fb = 0; fb < 4; ++fb) qi[fb] = ldg_half(qrow + 16 * fb + 4 * g);
  // T's upper blocks are never written
  for (int e = tid; e < kC * kP / 2; e += 256) reinterpret_cast<uint32_t*>(sm.tb)[e] = 0u;
  __syncthreads();
  // ---- a1: gates (wave 0) ----------------------------------------------------
  if (w == 0) {
    float eta, gi, gprev, glast;
    chunk_gates(sm.x, beta_l, lam_l, c * kC + l, T, eps, eps_gamma, fresh, l, eta, gi, gprev, glast);
    sm.G.graw[l] = gi;
    sm.G.sxg[l] = eta * __expf(gprev);
    sm.G.sxh[l] = __expf(glast - gi);
    sm.G.eta[l] = eta;
    sm.G.eta_t[c16 * 4 + g] = eta;
    sm.G.gprev_t[c16 * 4 + g] = gprev;
    if (l == 0) sm.G.e63 = __expf(glast);
  }
  __syncthreads();
  // ---- T; scaled key and value transposes; this wave's rows of M -------------
  bf16x8 xg[2][2];              // waves 1, 2: frag((Diag(eta e^{g_{s-1}}) X)^T) for fb = 2(w-1) + h
  bf16x8 vt[4][2];              // wave 3: frag((Diag(eta) V)^T) for all cb
  if (w == 0) {
    build_inverse(sm, l);
  } else if (w <= 2) {
    const int mk = w - 1;       // feature half
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // tile sb: lane holds X[16sb+4g+r][32mk+16h+c16]
      const bf16x8 sel = select_frag(h, g, c16);
      f32x4 d[4];
#pragma unroll
      for (int sb = 0; sb < 4; ++sb) d[sb] = mfma32(ring_frag_c(sm.x, 16 * sb + c16, mk, g), sel, zero4());
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        xg[h][m] = frag_acc(d[2 * m] * ld4(&sm.G.sxg[32 * m + 4 * g]), d[2 * m + 1] * ld4(&sm.G.sxg[32 * m + 16 + 4 * g]));
        store_frag(&sm.xh[fslot(2 * mk + h, m, l)],
                   frag_acc(d[2 * m] * ld4(&sm.G.sxh[32 * m + 4 * g]), d[2 * m + 1] * ld4(&sm.G.sxh[32 * m + 16 + 4 * g])));
      }
    }
  } else {
#pragma unroll
    for (int hv = 0; hv < 2; ++hv) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int cb = 2 * hv + h;
        const bf16x8 sel = select_frag(h, g, c16);
        f32x4 d[4];
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) d[sb] = mfma32(ring_frag_c(sm.ut, 16 * sb + c16, hv, g), sel, zero4());
#pragma unroll
        for (int m = 0; m < 2; ++m)
          vt[cb][m] = frag_acc(d[2 * m] * ld4(&sm.G.eta[32 * m + 4 * g]), d[2 * m + 1] * ld4(&sm.G.eta[32 * m + 16 + 4 * g]));
      }
    }
  }
  // M rows of token block ib = w: tile sb of X Q^T holds M[16w+c16][16sb+4g+r]
  // after the decay and the causal mask (s <= i); tiles 2m, 2m+1 stack into frag(M)[w][m]
  bf16x8 mf[2];
  {
    const int i = 16 * w + c16;
    const float gi = sm.G.graw[i];
    f32x4 mt[4];
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) {
      mt[sb] = zero4();
      if (sb <= w) {
        f32x4 acc = mfma32(ring_frag_c(sm.x, 16 * sb + c16, 0, g), qa0, zero4());
        acc = mfma32(ring_frag_c(sm.x, 16 * sb + c16, 1, g), qa1, acc);
        const f32x4 gs = ld4(&sm.G.graw[16 * sb + 4 * g]);
#pragma unroll
        for (int r = 0; r < 4; ++r) mt[sb][r] = 16 * sb + 4 * g + r <= i ? __expf(gi - gs[r]) * acc[r] : 0.0f;
      }
    }
    mf[0] = frag_acc(mt[0], mt[1]);
    mf[1] = frag_acc(mt[2], mt[3]);
  }
  __syncthreads();                                           // T, Xh complete; the key and value rows are free
  // ---- W and U as fragments over tokens --------------------------------------
  if (w >= 1) {
    bf16x8 tf[4][2];
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) {
      tf[ib][0] = frag_lds(&sm.tb[(16 * ib + c16) * kP], 0, g);
      tf[ib][1] = frag_lds(&sm.tb[(16 * ib + c16) * kP], 32, g);
    }
    if (w <= 2) {
      // tile (ib, fb) = T (Diag(eta e^{g_{s-1}}) X): lane holds W[16ib+4g+r][16fb+c16];
      // tiles ib = 2m, 2m+1 stack into frag(W^T)[fb][m] (stored negated)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int fb = 2 * (w - 1) + h;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          f32x4 d0 = mfma32(tf[2 * m][0], xg[h][0], zero4());
          f32x4 d1 = mfma32(tf[2 * m + 1][0], xg[h][0], zero4());
          if (m == 1) {                                       // T is lower triangular
            d0 = mfma32(tf[2 * m][1], xg[h][1], d0);
            d1 = mfma32(tf[2 * m + 1][1], xg[h][1], d1);
          }
          store_frag(&sm.x[fslot(fb, m, l)], frag_acc(-d0, -d1));
        }
      }
    } else {
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          f32x4 d0 = mfma32(tf[2 * m][0], vt[cb][0], zero4());
          f32x4 d1 = mfma32(tf[2 * m + 1][0], vt[cb][0], zero4());
          if (m == 1) {
            d0 = mfma32(tf[2 * m][1], vt[cb][1], d0);
            d1 = mfma32(tf[2 * m + 1][1], vt[cb][1], d1);
          }
          store_frag(&sm.ut[fslot(cb, m, l)], frag_acc(d0, d1));
        }
    }
  }
  __syncthreads();                                           // frag(-W^T), frag(U^T) complete
  // ---- chunk matrices ---------------------------------------------------------
  if (!out.acquire(sm, w, l)) return;
  uint16_t* dst = out.block();
  if (w == 0 && l == 0) *out.decay() = sm.G.e63;
  {
    bf16x8 wt[4][2], ut[4][2];
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        wt[b][m] = load_frag(&sm.x[fslot(b, m, l)]);
        ut[b][m] = load_frag(&sm.ut[fslot(b, m, l)]);
      }
    const bf16x8 xh0 = load_frag(&sm.xh[fslot(w, 0, l)]);
    const bf16x8 xh1 = load_frag(&sm.xh[fslot(w, 1, l)]);
    // K: tile (fb', fb = w) of (-W^T) Xh = K^T; fb' = 2m, 2m+1 stack into frag(K)[w][m]
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      f32x4 t0 = mfma32(wt[2 * m][0], xh0, zero4());
      t0 = mfma32(wt[2 * m][1], xh1, t0);
      f32x4 t1 = mfma32(wt[2 * m + 1][0], xh0, zero4());
      t1 = mfma32(wt[2 * m + 1][1], xh1, t1);
      store_frag(dst + Out::kK + fslot(w, m, l), frag_acc(t0, t1));
    }
    // H: tile (fb = w, cb) of Xh^T U, lane holds H[16w+4g+r][16cb+c16]
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      f32x4 hacc = mfma32(xh0, ut[cb][0], zero4());
      hacc = mfma32(xh1, ut[cb][1], hacc);
      store_half(dst + Out::kH + ((cb * 4 + w) * 64 + l) * 4, hacc);
    }
    // Qt: tile (fb, ib = w) of e^{g_i} Q^T - W^T M^T = Qt^T; fb = 2m, 2m+1 stack into frag(Qt)[w][m]
    bf16x8 qt[2];
    {
      const float egi = __expf(sm.G.graw[16 * w + c16]);
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        f32x4 t[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int fb = 2 * m + h;
          f32x4 acc = unpack_half(qi[fb]) * egi;
          acc = mfma32(wt[fb][0], mf[0], acc);
          if (w >= 2) acc = mfma32(wt[fb][1], mf[1], acc);
          t[h] = acc;
        }
        qt[m] = frag_acc(t[0], t[1]);
      }
    }
    // Ot^T: tile (cb, ib = w) of U^T M^T, lane holds Ot[16w+c16][16cb+4g+r] (bf16)
    uint2 ot[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      f32x4 oacc = mfma32(ut[cb][0], mf[0], zero4());
      if (w >= 2) oacc = mfma32(ut[cb][1], mf[1], oacc);
      ot[cb] = make_uint2(pack_bf16x2(oacc[0], oacc[1]), pack_bf16x2(oacc[2], oacc[3]));
    }
    out.finish(sm, w, l, qt, ot);
  }
}

// Output policy of the two-launch form: every chunk has its own block of the
// workspace holding K, Qt, H and Ot; nothing to wait for or announce.
struct BlockOut {
  static constexpr int kK = kOutK, kH = kOutH;
  uint16_t* blk;
  float* e63;
  __device__ void prefetch(int) {}
  __device__ bool acquire(WySmem&, int, int) { return true; }
  __device__ uint16_t* block() { return blk; }
  __device__ float* decay() { return e63; }
  __device__ void finish(WySmem&, int w, int l, const bf16x8 (&qt)[2], const uint2 (&ot)[4]) {
#pragma unroll
    for (int m = 0; m < 2; ++m) store_frag(blk + kOutQt + fslot(w, m, l), qt[m]);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) *reinterpret_cast<uint2*>(blk + kOutOt + ((cb * 4 + w) * 64 + l) * 4) = ot[cb];
  }
};

__global__ void __launch_bounds__(256, 4)
falcon1_wy_kernel(const bf16_t* __restrict__ phi_k, const bf16_t* __restrict__ phi_q,
                  const bf16_t* __restrict__ v, const float* __restrict__ beta, const float* __restrict__ lam,
                  const bf16_t* __restrict__ k_prev, uint16_t* __restrict__ blocks, float* __restrict__ decay63,
                  int T, int nchunks, float eps, float eps_gamma) {
  __shared__ WySmem sm;
  BlockOut out{blocks + int64_t(blockIdx.x) * kBlockElems, decay63 + blockIdx.x};
  wy_chunk(sm, phi_k, phi_q, v, beta, lam, k_prev, blockIdx.x / nchunks, blockIdx.x % nchunks, T, eps, eps_gamma,
           out);
}

// ============================================================================
// Launch 2: state passing and outputs.
//
// kSplit workgroups per sequence, each owning 64 / kSplit value columns (the
// columns of S evolve independently).  kStagers staging waves each fetch every
// kStagers-th chunk's K, Qt and this workgroup's columns of H and Ot into
// registers, then into a kRing-entry LDS ring, so that several chunks are in
// flight from memory at once; the chain waves (16 value columns each, fp32
// state in MFMA result registers) run S' = e^{g_63} S + K S + H and
// O = Qt S + Ot.  Hand-over is through LDS counters with bounded waits.
// ============================================================================

constexpr int kSplit = 2;
constexpr int kColWaves = 4 / kSplit;
constexpr int kStagers = 4;
constexpr int kRing = 4;
constexpr int kChainThreads = 64 * (kColWaves + kStagers);
constexpr int kEntryElems = 8192 + kColWaves * 2048;     // K, Qt, then per chain wave H and Ot
constexpr int kEntryFrags = kEntryElems / 512;           // 16-byte fragments per lane

struct ChainSmem {
  uint16_t d[kRing][kEntryElems];
  float e63[kRing];
  int in_ready[kRing];            // chunks stored into the entry so far
  int in_free[kRing];             // +1 per chain wave done with an entry
  int abort_flag;
};

// Polls `flag` until it reaches `target`, at most `limit` times.  A wait
// that runs out sets the workgroup's abort flag and returns false; once the
// flag is set every later wait returns false at once.
__device__ __forceinline__ bool wait_at_least(int* flag, int target, int* abort_flag, int limit) {
  for (int it = 0; it < limit; ++it) {
    const int val = __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (__builtin_amdgcn_readfirstlane(val) >= target) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
      return true;
    }
    if (__hip_atomic_load(abort_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) return false;
    __builtin_amdgcn_s_sleep(1);
  }
  __hip_atomic_store(abort_flag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  return false;
}
__device__ __forceinline__ void signal_add(int* flag, int l) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  if (l == 0) __hip_atomic_fetch_add(flag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Workspace element offset of ring-entry fragment j for column part `part`.
__device__ __forceinline__ int entry_src(int j, int part) {
  constexpr int kParts = 2 * kColWaves;                  // fragments of H (and of Ot) per part
  if (j < 16) return j * 512;
  if (j < 16 + kParts) return kOutH + part * kParts * 512 + (j - 16) * 512;
  return kOutOt + part * kParts * 512 + (j - 16 - kParts) * 512;
}

// The two chain waves of a workgroup: the state of value columns
// 16 cb .. 16 cb + 15 in MFMA result registers, one step per chunk.
__device__ __forceinline__ void chain_waves(ChainSmem& sm, const float* S0, bf16_t* __restrict__ o, float* S_T,
                                            int64_t bh, int part, int wave, int l, int T, int nchunks,
                                            int spin_limit) {
  // ---- chain waves ------------------------------------------------------------
  // Per chunk c: the reads of Qt and Ot are issued before the state update and
  // the reads of chunk c + 1's K and H before the outputs, so LDS latency hides
  // behind the matrix products.  A wait that runs out sets the abort flag; the
  // loop still runs to its end (every later wait returns at once).
  const int cw = wave;
  const int g = l >> 4, c16 = l & 15;
  const int cb = part * kColWaves + cw;                      // value columns 16 cb .. 16 cb + 15
  const int hoff = 8192 + cw * 1024 + l * 4;                 // this wave's H tiles in an entry
  const int ooff = 8192 + kColWaves * 1024 + cw * 1024 + l * 4;
  f32x4 S[4];                                                // S[fb]: lane holds S[16fb+4g+r][16cb+c16]
#pragma unroll
  for (int fb = 0; fb < 4; ++fb)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      S[fb][r] = S0 ? S0[(bh * kD + 16 * fb + 4 * g + r) * kD + 16 * cb + c16] : 0.0f;
  bf16_t* o_bh = o + bh * T * kD;
  bf16x8 kf[4][2];                                           // frag(K)[fb][m] of the current chunk
  uint2 hf[4];                                               // its H tiles
  float e63;
  wait_at_least(&sm.in_ready[0], 1, &sm.abort_flag, spin_limit);
#pragma unroll
  for (int fb = 0; fb < 4; ++fb) {
    kf[fb][0] = load_frag(&sm.d[0][kOutK + fslot(fb, 0, l)]);
    kf[fb][1] = load_frag(&sm.d[0][kOutK + fslot(fb, 1, l)]);
    hf[fb] = *reinterpret_cast<const uint2*>(&sm.d[0][hoff + fb * 256]);
  }
  e63 = sm.e63[0];
  // the state as a bf16 operand, carried around the loop (forming it here also
  // retires the S0 loads before the loop, so no wait in the loop covers the
  // output stores)
  bf16x8 sb0 = frag_acc(S[0], S[1]);
  bf16x8 sb1 = frag_acc(S[2], S[3]);
  for (int c = 0; c < nchunks; ++c) {
    const uint16_t* D = sm.d[c % kRing];
    const int e1 = (c + 1) % kRing;
    // chunk c + 1 must be in its entry before its reads below; after the last
    // chunk those reads only see a stale entry and are not used
    if (c + 1 < nchunks) wait_at_least(&sm.in_ready[e1], (c + 1) / kRing + 1, &sm.abort_flag, spin_limit);
    bf16x8 qf[4][2];
    uint2 of[4];
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) {
      qf[ib][0] = load_frag(&D[kOutQt + fslot(ib, 0, l)]);
      qf[ib][1] = load_frag(&D[kOutQt + fslot(ib, 1, l)]);
      of[ib] = *reinterpret_cast<const uint2*>(&D[ooff + ib * 256]);
    }
    // S <- e^{g_63} S + K S + H
#pragma unroll
    for (int fb = 0; fb < 4; ++fb) {
      f32x4 acc = S[fb] * e63 + unpack_half(hf[fb]);
      acc = mfma32(kf[fb][0], sb0, acc);
      S[fb] = mfma32(kf[fb][1], sb1, acc);
    }
    {
      const uint16_t* D1 = sm.d[e1];
#pragma unroll
      for (int fb = 0; fb < 4; ++fb) {
        kf[fb][0] = load_frag(&D1[kOutK + fslot(fb, 0, l)]);
        kf[fb][1] = load_frag(&D1[kOutK + fslot(fb, 1, l)]);
        hf[fb] = *reinterpret_cast<const uint2*>(&D1[hoff + fb * 256]);
      }
      e63 = sm.e63[e1];
    }
    // O^T tiles: S^T Qt^T + Ot^T; lane holds o[t0+16ib+c16][16cb+4g+r]
    const int t0 = c * kC;
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) {
      f32x4 acc = mfma32(sb0, qf[ib][0], unpack_half(of[ib]));
      acc = mfma32(sb1, qf[ib][1], acc);
      const int tok = t0 + 16 * ib + c16;
      if (tok < T)
        *reinterpret_cast<uint2*>(o_bh + int64_t(tok) * kD + 16 * cb + 4 * g) =
            make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
    }
    sb0 = frag_acc(S[0], S[1]);
    sb1 = frag_acc(S[2], S[3]);
    signal_add(&sm.in_free[c % kRing], l);
  }
  // the final state (overwritten with NaN after the loop if any wait ran out)
  if (S_T) {
#pragma unroll
    for (int fb = 0; fb < 4; ++fb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        S_T[(bh * kD + 16 * fb + 4 * g + r) * kD + 16 * cb + c16] = S[fb][r];
  }
}

__global__ void __launch_bounds__(kChainThreads)
falcon1_chain_kernel(const float* S0, const uint16_t* __restrict__ blocks, const float* __restrict__ decay63,
                     bf16_t* __restrict__ o, float* S_T, int T, int nchunks, int64_t BH, int spin_limit) {
  __shared__ ChainSmem sm;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;
  const int g = l >> 4, c16 = l & 15;
  // workgroups b and b + 8 (and so on) take the parts of one sequence, so they
  // share an XCD and its L2
  const int64_t bh = (int64_t(blockIdx.x) / (8 * kSplit)) * 8 + blockIdx.x % 8;
  const int part = (blockIdx.x / 8) % kSplit;
  if (bh >= BH) return;
  const uint16_t* blk_bh = blocks + bh * nchunks * kBlockElems;
  const float* e63_bh = decay63 + bh * nchunks;

  if (tid < kRing) { sm.in_ready[tid] = 0; sm.in_free[tid] = 0; }
  if (tid == 0) sm.abort_flag = 0;
  __syncthreads();

  if (wave >= kColWaves) {
    // ---- staging: chunks c = s, s + kStagers, ... -----------------------------
    const int s = wave - kColWaves;
    int src[kEntryFrags];
#pragma unroll
    for (int j = 0; j < kEntryFrags; ++j) src[j] = entry_src(j, part) + l * 8;
    for (int c = s; c < nchunks; c += kStagers) {
      bf16x8 R[kEntryFrags];
      const uint16_t* blk = blk_bh + int64_t(c) * kBlockElems;
#pragma unroll
      for (int j = 0; j < kEntryFrags; ++j) R[j] = load_frag(blk + src[j]);
      const float e63 = e63_bh[c];
      const int e = c % kRing;
      if (!wait_at_least(&sm.in_free[e], kColWaves * (c / kRing), &sm.abort_flag, spin_limit)) break;
#pragma unroll
      for (int j = 0; j < kEntryFrags; ++j) store_frag(&sm.d[e][j * 512 + l * 8], R[j]);
      if (l == 0) sm.e63[e] = e63;
      signal_add(&sm.in_ready[e], l);
    }
  } else {
    chain_waves(sm, S0, o, S_T, bh, part, wave, l, T, nchunks, spin_limit);
  }
  // Every wave gets here.  A wait that ran out anywhere in the workgroup (a
  // hand-over that never came) poisons this part of the sequence: its outputs
  // and its final state become NaN, so an abort can never pass for a result.
  __syncthreads();
  if (wave < kColWaves &&
      __hip_atomic_load(&sm.abort_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) != 0) {
    const int cb = part * kColWaves + wave;
    const uint16_t nan_bits = 0x7fc0;
    const uint32_t nan2 = uint32_t(nan_bits) | (uint32_t(nan_bits) << 16);
    bf16_t* o_bh = o + bh * T * kD;
    // the wave's own columns, after its own stores to them (program order)
    for (int tok = l >> 1; tok < T; tok += 32)
      *reinterpret_cast<uint4*>(o_bh + int64_t(tok) * kD + 16 * cb + 8 * (l & 1)) = make_uint4(nan2, nan2, nan2, nan2);
    if (S_T) {
      const int g = l >> 4, c16 = l & 15;
#pragma unroll
      for (int fb = 0; fb < 4; ++fb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          S_T[(bh * kD + 16 * fb + 4 * g + r) * kD + 16 * cb + c16] = __builtin_nanf("");
    }
  }
}

// ============================================================================
// One launch: chunk workgroups and per-sequence chains side by side.
//
// Chunk workgroups build and store the chunk matrices exactly as in the
// two-launch form and announce each block with a flag; the chain of a
// sequence starts on a chunk as soon as it is announced, so the sequential
// part overlaps the chunk-parallel part and reads the blocks from L2 rather
// than HBM.
//
// Placement: workgroup b runs on XCD b mod 8 (workgroups are dealt to the
// XCDs in turn).  The chain of sequence s runs in workgroups s and BHpad + s
// (value-column halves) and chunk c of s in workgroup BHpad (c + 2) + s, so
// all of a sequence's work sits on XCD s mod 8 and shares its L2.  Chains come
// first in the grid, so they are resident before any chunk workgroup is
// dispatched, and chunk workgroups never wait, so every wait of a chain ends.
// The waits are nevertheless bounded: a wait that gives up poisons the
// sequence's outputs and final state with NaN.
//
// Hand-over without device-wide fences: a chunk workgroup's stores reach the
// L2 of its XCD before it announces them (s_waitcnt vmcnt(0) in every wave,
// then a barrier, then the flag store); the chain, on the same XCD, reads the
// flag with a device-scope load and only then the block, from that L2.  No
// block address is read before its announcement or twice by one CU in a
// launch, and the vector L1 starts every launch empty, so no L1 line is ever
// stale; the decays, several to a line, are read with device-scope loads.
// Flags carry the writer's XCD, and a chain that sees another XCD gives up
// (NaN) rather than read an incoherent L2.
// ============================================================================

constexpr int kTagMask = 0xffffff;

// Role of workgroup b of the one-launch grid: the two chain workgroups of
// sequence s (value-column half `part`) come first, then chunk c of sequence
// s.  Shared by the kernel and the host-side bounds model.
struct FusedRole {
  bool chain;
  int s, part, c;
};
__host__ __device__ inline FusedRole fused_role(int b, int BHpad) {
  FusedRole r;
  r.chain = b < 2 * BHpad;
  const int j = r.chain ? b : b - 2 * BHpad;
  r.s = j % BHpad;
  r.part = r.chain ? j / BHpad : 0;
  r.c = r.chain ? 0 : j / BHpad;
  return r;
}
// A chain wave's per-lane byte offsets: its first K fragment in a block, its
// first H (and Ot) tile in a block, its output row within a chunk.
__host__ __device__ inline uint32_t chain_lf(int w, int l) { return uint32_t(2 * fslot(w, 0, l)); }
__host__ __device__ inline uint32_t chain_lh(int p, int w, int l) { return uint32_t(8 * ((8 * p + w) * 64 + l)); }
__host__ __device__ inline uint32_t chain_lo(int p, int w, int l) {
  return uint32_t(2 * ((16 * w + (l & 15)) * 64 + 32 * p + 4 * (l >> 4)));
}

struct FusedArgs {
  const bf16_t* phi_k;
  const bf16_t* phi_q;
  const bf16_t* v;
  const float* beta;
  const float* lam;
  const bf16_t* k_prev;
  const float* S0;
  bf16_t* o;
  float* S_T;
  uint16_t* blocks;                    // [BH][nchunks][kBlockElems]
  float* decay63;                      // [BH][nchunks]
  int* flags;                          // [BHpad][nflag], zero at launch
  int T, nchunks, nflag, BH, BHpad, spin_limit;
  float eps, eps_gamma;
};

__device__ __forceinline__ int xcc_id() {
  return __builtin_amdgcn_s_getreg((3 << 11) | 20) & 15;      // HW_REG_XCC_ID, bits 3:0
}
__device__ __forceinline__ int load_flag(const int* f) {
  return __builtin_amdgcn_readfirstlane(__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
// 1: the flag announces chunk c from this XCD; 0: not yet; -1: from another XCD
__device__ __forceinline__ int tag_state(int v, int c, int xcc) {
  if ((v & kTagMask) != ((c + 1) & kTagMask)) return 0;
  return (v >> 24) == xcc ? 1 : -1;
}

// Output policy of a chunk workgroup of the one-launch form: the block of the
// two-launch form, then its announcement.
struct FlagOut {
  static constexpr int kK = kOutK, kH = kOutH;
  uint16_t* blk;
  float* e63;
  int* ready;                          // this chunk's flag
  int tag;                             // (XCD << 24) | (c + 1)
  __device__ void prefetch(int) {}
  __device__ bool acquire(WySmem&, int, int) { return true; }
  __device__ uint16_t* block() { return blk; }
  __device__ float* decay() { return e63; }
  __device__ void finish(WySmem&, int w, int l, const bf16x8 (&qt)[2], const uint2 (&ot)[4]) {
#pragma unroll
    for (int m = 0; m < 2; ++m) store_frag(blk + kOutQt + fslot(w, m, l), qt[m]);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) *reinterpret_cast<uint2*>(blk + kOutOt + ((cb * 4 + w) * 64 + l) * 4) = ot[cb];
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");       // this wave's stores are in L2
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_store(ready, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
};

// Waits until chunk c is announced by a chunk workgroup on this XCD; `seen`
// is its flag as read earlier (0 if never), so that a chunk announced in time
// costs no load.  A wait that gives up (any wait, with a limit of 0), or a
// writer on another XCD, sets the workgroup's abort flag; once it is set,
// every later wait returns at once.
__device__ __forceinline__ void wait_chunk(const int* flag, int c, int xcc, int limit, int seen, int* abort_flag) {
  if (__hip_atomic_load(abort_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) return;
  int v = __builtin_amdgcn_readfirstlane(seen);
  for (int it = 0; limit > 0; ++it) {
    const int st = tag_state(v, c, xcc);
    if (st == 1) return;
    if (st < 0 || it >= limit) break;
    if (it > 0) __builtin_amdgcn_s_sleep(1);
    v = load_flag(flag);
  }
  __hip_atomic_store(abort_flag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// A workgroup barrier that orders LDS only: outstanding global loads and
// stores stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Chain workgroups of a sequence: value columns evolve independently, so
// the sequence's state is split into column halves, one workgroup each.  In
// half p, wave w holds rows 16 w .. 16 w + 15 of columns 32 p .. 32 p + 31 in
// MFMA result registers (S[i]: lane holds S[16w+4g+r][16(2p+i)+c16]).  Per
// chunk it needs only its share of the block (K and Qt fragments of row block
// w, H and Ot tiles of row or token block w in its columns), read straight
// from L2 one chunk ahead.  The bf16 state that every row block multiplies is
// exchanged through LDS, double-buffered, one barrier a chunk: column j of the
// half is a row of kSRow bf16 with key 32 m + 16 h + 4 g + r at position
// 32 m + 8 g + 4 h + r, so that one 16-byte read is a result-compatible
// fragment (the order frag_acc gives).
constexpr int kSRow = 72;              // 64 keys + 8 of padding (16-byte reads conflict-free)
constexpr int kHalfCols = 32;

struct ChainSmemRow {
  uint16_t s[2][kHalfCols * kSRow];
  int abort_flag;
};

union FusedSmem {
  WySmem p;
  ChainSmemRow c;
};

// A wave's share of one chunk's block, and the chunk's decay.
struct RowTiles {
  bf16x8 k0, k1, q0, q1;               // K and Qt fragments (row block w, m = 0, 1)
  uint2 h0, h1;                        // H tiles (column blocks 2p, 2p + 1; row block w)
  uint2 o0, o1;                        // Ot tiles (column blocks 2p, 2p + 1; token block w)
  float e63;
};
// Loads at a uniform base plus a 32-bit per-lane byte offset (one address
// register per lane, the base in scalar registers).
template <class V>
__device__ __forceinline__ V load_at(const char* base, uint32_t off) {
  return *reinterpret_cast<const V*>(base + off);
}
// blk: the chunk's block; lf = 2 fslot(w, 0, l) and lh = 8 ((8p + w) 64 + l),
// the lane's byte offsets of its first K fragment and first H tile (tile
// (cb, w) of H and of Ot sits at element ((cb * 4 + w) * 64 + l) * 4).
__device__ __forceinline__ RowTiles load_row_tiles(const uint16_t* blk, const float* e63, uint32_t lf, uint32_t lh) {
  const char* b = reinterpret_cast<const char*>(blk);
  RowTiles r;
  r.k0 = load_at<bf16x8>(b + 2 * kOutK, lf);
  r.k1 = load_at<bf16x8>(b + 2 * kOutK + 1024, lf);
  r.q0 = load_at<bf16x8>(b + 2 * kOutQt, lf);
  r.q1 = load_at<bf16x8>(b + 2 * kOutQt + 1024, lf);
  r.h0 = load_at<uint2>(b + 2 * kOutH, lh);
  r.h1 = load_at<uint2>(b + 2 * kOutH + 2048, lh);
  r.o0 = load_at<uint2>(b + 2 * kOutOt, lh);
  r.o1 = load_at<uint2>(b + 2 * kOutOt + 2048, lh);
  r.e63 = __hip_atomic_load(e63, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return r;
}

// What a chain wave carries from chunk to chunk besides its state and tiles.
struct RowCtx {
  const int* fl;                       // the sequence's flags
  const uint16_t* blocks;              // the sequence's blocks
  const float* e63;                    // the sequence's decays
  bf16_t* o;                           // the sequence's outputs
  uint32_t lf, lh, lo;                 // lane byte offsets: K fragment, H tile, output row
  int p, w, l, xcc, ahead;             // ahead: flag of the next chunk, as read one step earlier
};

// One chunk of a chain wave: O = Qt S + Ot for token block w and
// S <- e^{g_63} S + K S + H for row block w, with the operand roundings of the
// two-launch chain, then the new state's bf16 rows into the other LDS buffer.
// `cur` holds this chunk's tiles.  A read of a just-written block takes about
// a microsecond, several chunks' worth of chain work, so tiles are read two
// chunks ahead, into `dst` (the set of the chunk before this one), once that
// chunk is announced; near the end the last chunk is read again instead (it
// is announced, so the read is harmless).  Output rows go through a buffer
// descriptor that ends at row T, so rows past T are dropped by the hardware.
// Every step thus issues the same loads and stores, and the caller rotates
// three tile sets rather than copying them: the compiler then waits for
// exactly the loads a step uses, never for earlier output stores.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void chain_row_step(ChainSmemRow& sm, const FusedArgs& a, RowCtx& x, int c,
                                               const RowTiles& cur, RowTiles& dst, f32x4 (&S)[2]) {
  const int n = a.nchunks, l = x.l, w = x.w;
  const int g = l >> 4, c16 = l & 15;
  const int ca = c + 2 < n ? c + 2 : n - 1;
  wait_chunk(&x.fl[ca], ca, x.xcc, a.spin_limit, x.ahead, &sm.abort_flag);
  // the next flag before the tiles: loads complete in order, so the next
  // step's look at the flag then waits for nothing issued after it
  x.ahead = __hip_atomic_load(&x.fl[c + 3 < n ? c + 3 : n - 1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  dst = load_row_tiles(x.blocks + int64_t(ca) * kBlockElems, x.e63 + ca, x.lf, x.lh);
  const uint16_t* Sb = sm.s[c & 1];
  uint16_t* Sn = sm.s[(c + 1) & 1];
  const float ec = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(cur.e63)));
  const uint2 hc[2] = {cur.h0, cur.h1};
  const uint2 oc[2] = {cur.o0, cur.o1};
  const int rows = a.T - c * kC < kC ? a.T - c * kC : kC;
  const __amdgpu_buffer_rsrc_t orow =
      __builtin_amdgcn_make_buffer_rsrc(x.o + int64_t(c) * kC * kD, 0, rows * kD * 2, 0x00020000);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint16_t* col = Sb + (16 * i + c16) * kSRow + 8 * g;
    const bf16x8 f0 = load_frag(col);                      // keys 0..31 of column 16cb+c16
    const bf16x8 f1 = load_frag(col + 32);                 // keys 32..63
    // O^T tile: S^T Qt^T + Ot^T; lane holds o[c*64+16w+c16][16cb+4g+r]
    f32x4 ov = mfma32(f0, cur.q0, unpack_half(oc[i]));
    ov = mfma32(f1, cur.q1, ov);
    const u32x2 ob = {pack_bf16x2(ov[0], ov[1]), pack_bf16x2(ov[2], ov[3])};
    __builtin_amdgcn_raw_buffer_store_b64(ob, orow, x.lo + 32 * i, 0, 0);
    // S <- e^{g_63} S + K S + H
    f32x4 acc = S[i] * ec + unpack_half(hc[i]);
    acc = mfma32(cur.k0, f0, acc);
    S[i] = mfma32(cur.k1, f1, acc);
    *reinterpret_cast<uint2*>(Sn + (16 * i + c16) * kSRow + 32 * (w >> 1) + 8 * g + 4 * (w & 1)) =
        make_uint2(pack_bf16x2(S[i][0], S[i][1]), pack_bf16x2(S[i][2], S[i][3]));
  }
  lds_barrier();
}

__device__ __forceinline__ void chain_workgroup(ChainSmemRow& sm, const FusedArgs& a, int s, int p) {
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;
  const int g = l >> 4, c16 = l & 15;
  const int n = a.nchunks;
  if (tid == 0) sm.abort_flag = 0;
  RowCtx x;
  x.fl = a.flags + int64_t(s) * a.nflag;
  x.blocks = a.blocks + int64_t(s) * n * kBlockElems;
  x.e63 = a.decay63 + int64_t(s) * n;
  x.o = a.o + int64_t(s) * a.T * kD;
  x.p = p;
  x.w = w;
  x.l = l;
  x.xcc = xcc_id();
  x.lf = chain_lf(w, l);
  x.lh = chain_lh(p, w, l);
  x.lo = chain_lo(p, w, l);                                // o[16w+c16][32p+4g], within a chunk
  f32x4 S[2];
  const float* S0 = a.S0 ? a.S0 + int64_t(s) * kD * kD + (16 * w + 4 * g) * kD + 32 * p + c16 : nullptr;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    S[i] = zero4();
    if (S0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) S[i][r] = S0[r * kD + 16 * i];
    }
    *reinterpret_cast<uint2*>(sm.s[0] + (16 * i + c16) * kSRow + 32 * (w >> 1) + 8 * g + 4 * (w & 1)) =
        make_uint2(pack_bf16x2(S[i][0], S[i][1]), pack_bf16x2(S[i][2], S[i][3]));
  }
  __syncthreads();
  // Tiles of chunks 0 and 1 with the flag of chunk 2 between them, then two
  // flag loads (values unused): the loop is entered with the loads in flight
  // after that flag that its back edge has (a set of tiles and two output
  // stores), so the compiler's wait for the flag at the loop head leaves
  // them in flight.
  const int c1 = n > 1 ? 1 : 0;
  wait_chunk(&x.fl[0], 0, x.xcc, a.spin_limit, 0, &sm.abort_flag);
  RowTiles t0 = load_row_tiles(x.blocks, x.e63, x.lf, x.lh);
  wait_chunk(&x.fl[c1], c1, x.xcc, a.spin_limit, 0, &sm.abort_flag);
  x.ahead = __hip_atomic_load(&x.fl[n > 2 ? 2 : n - 1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  RowTiles t1 = load_row_tiles(x.blocks + int64_t(c1) * kBlockElems, x.e63 + c1, x.lf, x.lh);
  RowTiles t2;
  int pad = __hip_atomic_load(&x.fl[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  pad |= __hip_atomic_load(&x.fl[c1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // tile set of chunk c is t(c mod 3)
  int c = 0;
  for (; c + 3 <= n; c += 3) {
    chain_row_step(sm, a, x, c, t0, t2, S);
    chain_row_step(sm, a, x, c + 1, t1, t0, S);
    chain_row_step(sm, a, x, c + 2, t2, t1, S);
  }
  if (c < n) chain_row_step(sm, a, x, c, t0, t2, S);
  if (c + 1 < n) chain_row_step(sm, a, x, c + 1, t1, t0, S);
  if (pad == -1) sm.abort_flag = 2;                        // never: flags are never -1; keeps the loads
  // A wait that gave up anywhere in the workgroup poisons the sequence: its
  // outputs and final state are NaN.
  __syncthreads();
  const bool bad = __hip_atomic_load(&sm.abort_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) != 0;
  if (bad) {
    const uint32_t nan2 = 0x7fc07fc0u;                     // two bf16 NaNs
    uint4* o4 = reinterpret_cast<uint4*>(x.o);
    for (int64_t i = tid; i < int64_t(a.T) * 4; i += 256) o4[(i >> 2) * 8 + 4 * p + (i & 3)] = make_uint4(nan2, nan2, nan2, nan2);
  }
  if (a.S_T) {
    float* st = a.S_T + int64_t(s) * kD * kD + (16 * w + 4 * g) * kD + 32 * p + c16;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) st[r * kD + 16 * i] = bad ? __builtin_nanf("") : S[i][r];
  }
}

__global__ void __launch_bounds__(256, 4) falcon1_fused_kernel(FusedArgs a) {
  __shared__ FusedSmem sm;
  const FusedRole r = fused_role(blockIdx.x, a.BHpad);
  if (r.s >= a.BH) return;
  if (r.chain) {
    chain_workgroup(sm.c, a, r.s, r.part);
    return;
  }
  const int s = r.s, c = r.c;
  const int64_t q = int64_t(s) * a.nchunks + c;
  FlagOut out{a.blocks + q * kBlockElems, a.decay63 + q, a.flags + int64_t(s) * a.nflag + c,
              (xcc_id() << 24) | ((c + 1) & kTagMask)};
  wy_chunk(sm.p, a.phi_k, a.phi_q, a.v, a.beta, a.lam, a.k_prev, s, c, a.T, a.eps, a.eps_gamma, out);
}

__global__ void zero_ints_kernel(int* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

}  // namespace

bool chunked_wy_applies(const ProblemArgs& a) {
  return a.bf16 && a.variant == kF1 && a.dk == kD && a.dv == kD && a.C == kC && a.T > 0;
}

// Workspace: a 32 KiB block of chunk matrices per chunk, then the decays
// e^{g_63}; the one-launch form adds a line of flags per sequence in front.
struct WyLayout {
  int64_t BHpad, nflag, flags_bytes, e63_bytes, blocks_bytes, total;
  WyLayout(int64_t BH, int64_t nchunks) {
    BHpad = (BH + 7) / 8 * 8;
    nflag = (nchunks + 63) / 64 * 64;
    flags_bytes = BHpad * nflag * 4;
    e63_bytes = (BH * nchunks * 4 + 255) / 256 * 256;
    blocks_bytes = BH * nchunks * int64_t(kBlockElems) * 2;
    total = flags_bytes + e63_bytes + blocks_bytes;
  }
};

size_t chunked_wy_workspace_bytes(const ProblemArgs& a) {
  return size_t(WyLayout(int64_t(a.B) * a.H, (int64_t(a.T) + kC - 1) / kC).total);
}

// The one-launch grid against the workspace layout and the buffers, on the
// host (bounds-check builds): every workgroup's role and XCD, the block,
// decay and flag each chunk workgroup writes (each exactly once), the chunks
// and output rows each chain reads and writes, and a chain lane's reads within
// a block.
void check_fused_grid(const ProblemArgs& a, const WyLayout& L, int nchunks) {
  const int64_t BH = int64_t(a.B) * a.H;
  const int64_t grid = L.BHpad * (int64_t(nchunks) + 2);
  FALCON_HOST_CHECK(grid <= INT32_MAX);
  FALCON_HOST_CHECK(L.BHpad % 8 == 0 && L.BHpad >= BH && L.BHpad < BH + 8);
  FALCON_HOST_CHECK(L.nflag >= nchunks && L.nflag % 64 == 0);
  FALCON_HOST_CHECK(int64_t(a.workspace_bytes) >= L.total);
  FALCON_HOST_CHECK(L.flags_bytes % 256 == 0 && L.e63_bytes % 256 == 0);
  std::vector<int> chains(size_t(BH) * 2, 0), chunks(size_t(BH) * nchunks, 0);
  for (int64_t b = 0; b < grid; ++b) {
    const FusedRole r = fused_role(int(b), int(L.BHpad));
    FALCON_HOST_CHECK(r.s >= 0 && r.s < L.BHpad);
    FALCON_HOST_CHECK(b % 8 == r.s % 8);                   // on its sequence's XCD
    if (r.s >= BH) continue;
    if (r.chain) {
      FALCON_HOST_CHECK(r.part == 0 || r.part == 1);
      ++chains[size_t(r.s) * 2 + r.part];
      continue;
    }
    FALCON_HOST_CHECK(r.c >= 0 && r.c < nchunks);
    ++chunks[size_t(r.s) * nchunks + r.c];
    const int64_t q = int64_t(r.s) * nchunks + r.c;
    FALCON_HOST_CHECK((q + 1) * kBlockElems * 2 <= L.blocks_bytes);
    FALCON_HOST_CHECK((q + 1) * 4 <= L.e63_bytes);
    FALCON_HOST_CHECK((int64_t(r.s) * L.nflag + r.c + 1) * 4 <= L.flags_bytes);
  }
  for (int v : chains) FALCON_HOST_CHECK(v == 1);
  for (int v : chunks) FALCON_HOST_CHECK(v == 1);
  for (int c = 0; c < nchunks; ++c) {
    const int ca = c + 2 < nchunks ? c + 2 : nchunks - 1;  // chunk read ahead
    const int cf = c + 3 < nchunks ? c + 3 : nchunks - 1;  // flag read ahead
    FALCON_HOST_CHECK(ca >= 0 && ca < nchunks && cf >= 0 && cf < nchunks);
    const int rows = a.T - c * kC < kC ? a.T - c * kC : kC;
    FALCON_HOST_CHECK(rows > 0 && int64_t(c) * kC + rows <= a.T);
  }
  for (int p = 0; p < 2; ++p)
    for (int w = 0; w < 4; ++w)
      for (int l = 0; l < 64; ++l) {
        FALCON_HOST_CHECK(2 * kOutK + chain_lf(w, l) + 1024 + 16 <= 2 * kOutQt);
        FALCON_HOST_CHECK(2 * kOutQt + chain_lf(w, l) + 1024 + 16 <= 2 * kOutH);
        FALCON_HOST_CHECK(2 * kOutH + chain_lh(p, w, l) + 2048 + 8 <= 2 * kOutOt);
        FALCON_HOST_CHECK(2 * kOutOt + chain_lh(p, w, l) + 2048 + 8 <= 2 * kBlockElems);
        FALCON_HOST_CHECK(chain_lo(p, w, l) + 32 + 8 <= uint32_t(2 * kC * kD));
      }
}

// The one-launch form holds two workgroup slots per sequence for its chains
// for the whole launch (four slots per CU, 128 per XCD), and a chunk
// workgroup can only run on its sequence's XCD: with more than 64 chains per
// XCD the chunk workgroups would crowd into too few slots (none at 128, where
// every chain's wait would give up), so larger batches take two launches.
constexpr int64_t kMaxOneLaunchSeqs = 256;

hipError_t launch_chunked_wy(const ProblemArgs& a, hipStream_t st) {
  const int64_t BH = int64_t(a.B) * a.H;
  const int nchunks = (a.T + kC - 1) / kC;
  if (BH == 0 || nchunks == 0) return hipSuccess;
  const WyLayout L(BH, nchunks);
  char* ws = static_cast<char*>(a.workspace);
  int* flags = reinterpret_cast<int*>(ws);
  float* decay63 = reinterpret_cast<float*>(ws + L.flags_bytes);
  uint16_t* blocks = reinterpret_cast<uint16_t*>(ws + L.flags_bytes + L.e63_bytes);
  if (a.f1_form == 1 || L.BHpad > kMaxOneLaunchSeqs) {
    FALCON_HOST_CHECK(int64_t(a.workspace_bytes) >= L.total && BH * nchunks <= INT32_MAX);
    hipLaunchKernelGGL(falcon1_wy_kernel, dim3(unsigned(BH * nchunks)), dim3(256), 0, st,
                       static_cast<const bf16_t*>(a.phi_k), static_cast<const bf16_t*>(a.phi_q),
                       static_cast<const bf16_t*>(a.v), a.beta, a.lam, static_cast<const bf16_t*>(a.k_prev),
                       blocks, decay63, a.T, nchunks, a.eps, a.eps_gamma);
    const int64_t groups = (BH + 7) / 8;
    hipLaunchKernelGGL(falcon1_chain_kernel, dim3(unsigned(groups * 8 * kSplit)), dim3(kChainThreads), 0, st,
                       a.S0, blocks, decay63, static_cast<bf16_t*>(a.o), a.S_T, a.T, nchunks, BH, a.spin_limit);
    return hipGetLastError();
  }
  FusedArgs f;
  f.phi_k = static_cast<const bf16_t*>(a.phi_k);
  f.phi_q = static_cast<const bf16_t*>(a.phi_q);
  f.v = static_cast<const bf16_t*>(a.v);
  f.beta = a.beta;
  f.lam = a.lam;
  f.k_prev = static_cast<const bf16_t*>(a.k_prev);
  f.S0 = a.S0;
  f.o = static_cast<bf16_t*>(a.o);
  f.S_T = a.S_T;
  f.blocks = blocks;
  f.decay63 = decay63;
  f.flags = flags;
  f.T = a.T;
  f.nchunks = nchunks;
  f.nflag = int(L.nflag);
  f.BH = int(BH);
  f.BHpad = int(L.BHpad);
  f.spin_limit = a.spin_limit;
  f.eps = a.eps;
  f.eps_gamma = a.eps_gamma;
  const int64_t nflags = L.flags_bytes / 4;
  FALCON_HOST_CHECK(L.BHpad <= kMaxOneLaunchSeqs);
  if (kBoundsCheck) check_fused_grid(a, L, nchunks);
  hipLaunchKernelGGL(zero_ints_kernel, dim3(unsigned((nflags + 255) / 256)), dim3(256), 0, st, flags, int(nflags));
  hipLaunchKernelGGL(falcon1_fused_kernel, dim3(unsigned(L.BHpad * (int64_t(nchunks) + 2))), dim3(256), 0, st, f);
  return hipGetLastError();
}

}  // namespace falcon
