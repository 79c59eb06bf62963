// Fused chunk-parallel Falcon-1 forward on MFMA (gfx950), bf16 I/O,
// dk = dv = 64, chunk C = 64.
//
// One workgroup (4 waves) owns one (batch, head) sequence and walks its
// chunks in order; the float32 state never leaves registers.  Per chunk the
// four stages of the chunk-parallel form run back to back on data staged in
// LDS, so every input byte is read from HBM once and every output byte is
// written once:
//
//   a1  shift and normalise: x_i = phi(k_{t0+i-1}), E_i = ||x_i||^2,
//       eta_i (Eq. 3.4 with the fresh-start sentinel), the clamped decay
//       log gamma_i = log1p(-min(eta_i lam_i, 1 - eps_gamma)) (Section 4.3)
//       and its chunk-local inclusive prefix g_i (log-space renormalisation,
//       Section 4.4, applied chunk-locally as for Eq. 4.16).
//   a2  WY/UT factors: the decayed strictly-lower Gram matrix
//       A_{i,s} = eta_i e^{g_{i-1}-g_s} (x_i . x_s) on MFMA, T = (I + A)^{-1}
//       by blocked forward substitution (16x16 diagonal blocks by row
//       elimination in registers, off-diagonal blocks on MFMA), then
//       W = T Diag(eta e^{g_{-1}}) X and U = T Diag(eta) V ("one multi-RHS
//       TriSolve per chunk" of the WY form).
//   a3  state passing: R = U - W S (rows eta_i r_i), then
//       S <- e^{g_63} S + (Diag(e^{g_63-g}) X)^T R.
//   a4  read after write: O = Diag(e^g) Q S + (tril(Q X^T) o e^{g_i-g_s}) R.
//
// MFMA operand convention.  v_mfma_f32_16x16x32_bf16 takes, in lane l, row
// (l & 15) of A and column (l & 15) of B with eight k-values each; the
// result holds column (l & 15), rows 4 (l >> 4) .. +3.  Every product here
// feeds lane group g = l >> 4 the k-values {4g..4g+3, 16+4g..16+4g+3} of
// each 32-wide k block (the same permutation for A and B, so the sum is
// unchanged).  With that choice two stacked result tiles ARE the operand
// fragment of the next product, which keeps S and R in registers.

#include "falcon_device.h"
#include "falcon_launch.h"

namespace falcon {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kC = 64;        // chunk length
constexpr int kD = 64;        // dk = dv
constexpr int kP = 72;        // bf16 row pitch of the staged tiles (elements)
constexpr int kPA = 68;       // float row pitch of the decayed Gram matrix

struct Smem {
  uint16_t xr[kC * kP];       // X rows (token-major), natural layout
  uint16_t qr[kC * kP];       // Q rows
  uint16_t xg[kD * kP];       // (Diag(eta e^{g_{s-1}}) X)^T : feature-major
  uint16_t xh[kD * kP];       // (Diag(e^{g_63 - g_s}) X)^T
  uint16_t vt[kD * kP];       // (Diag(eta) V)^T
  uint16_t tb[kC * kP];       // T = (I + A)^{-1}, row-major
  float at[kC * kPA];         // A^T (A_{i,s} stored at at[s][i])
  uint16_t wf[4 * 2 * 64 * 8];  // -W as A fragments [ib][m][lane][8]
  uint16_t mf[4 * 2 * 64 * 8];  // decayed Q X^T as B fragments of M^T
  float energy[kC];
  float eta[kC];
  float gexp[kC];             // e^{g_i}
  float gtail[kC];            // e^{g_63 - g_i}
  float graw[kC];             // g_i
};

__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(s16x4 a, s16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint16_t bf(float f) { return f32_to_bf16(f); }
__device__ __forceinline__ float fl(uint16_t b) { return bf16_to_f32(b); }

// Fragment (k block starting at kbase) from a bf16 row: k = kbase + {4g..4g+3,
// 16+4g..16+4g+3}.
__device__ __forceinline__ bf16x8 frag_row(const uint16_t* row, int kbase, int g) {
  const uint2 a = *reinterpret_cast<const uint2*>(row + kbase + 4 * g);
  const uint2 b = *reinterpret_cast<const uint2*>(row + kbase + 16 + 4 * g);
  return __builtin_bit_cast(bf16x8, make_uint4(a.x, a.y, b.x, b.y));
}
// Fragment from two stacked result tiles (rows 0-15 and 16-31 of a k block).
__device__ __forceinline__ bf16x8 frag_from_acc(f32x4 lo, f32x4 hi) {
  bf16x8 r;
  r[0] = static_cast<__bf16>(lo[0]); r[1] = static_cast<__bf16>(lo[1]);
  r[2] = static_cast<__bf16>(lo[2]); r[3] = static_cast<__bf16>(lo[3]);
  r[4] = static_cast<__bf16>(hi[0]); r[5] = static_cast<__bf16>(hi[1]);
  r[6] = static_cast<__bf16>(hi[2]); r[7] = static_cast<__bf16>(hi[3]);
  return r;
}
__device__ __forceinline__ bf16x8 load_frag(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}
__device__ __forceinline__ void store_half_frag(uint16_t* p, f32x4 v, float scale) {
  const uint32_t a = uint32_t(bf(v[0] * scale)) | (uint32_t(bf(v[1] * scale)) << 16);
  const uint32_t b = uint32_t(bf(v[2] * scale)) | (uint32_t(bf(v[3] * scale)) << 16);
  *reinterpret_cast<uint2*>(p) = make_uint2(a, b);
}
__device__ __forceinline__ s16x4 s16_from_acc(f32x4 v) {
  s16x4 r;
  r[0] = static_cast<short>(bf(v[0])); r[1] = static_cast<short>(bf(v[1]));
  r[2] = static_cast<short>(bf(v[2])); r[3] = static_cast<short>(bf(v[3]));
  return r;
}

// Lower 16x16 tiles (ib >= sb) of a 64x64 matrix, in a fixed order.
__constant__ int8_t kLowerTiles[10][2] = {{0, 0}, {1, 0}, {1, 1}, {2, 0}, {2, 1},
                                          {2, 2}, {3, 0}, {3, 1}, {3, 2}, {3, 3}};

// Global loads of one chunk into registers (prefetched one chunk ahead).
struct ChunkRegs {
  uint4 x[2], q[2], v[2];
  float beta, lam;
};

__device__ __forceinline__ void load_chunk(ChunkRegs& r, const bf16_t* K, const bf16_t* Q,
                                           const bf16_t* V, const float* beta,
                                           const float* lam, const bf16_t* k_prev, int T,
                                           int t0, int tid) {
  const int seg = tid & 7;
  const uint4 zero = make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int row = (tid >> 3) + 32 * h;
    const int tok = t0 + row;
    const int kt = tok - 1;                        // x_i = phi(k_{t-1})
    uint4 xv = zero;
    if (kt >= 0 && kt < T) xv = *reinterpret_cast<const uint4*>(K + int64_t(kt) * kD + 8 * seg);
    else if (kt == -1 && k_prev) xv = *reinterpret_cast<const uint4*>(k_prev + 8 * seg);
    r.x[h] = xv;
    r.q[h] = tok < T ? *reinterpret_cast<const uint4*>(Q + int64_t(tok) * kD + 8 * seg) : zero;
    r.v[h] = tok < T ? *reinterpret_cast<const uint4*>(V + int64_t(tok) * kD + 8 * seg) : zero;
  }
  const int tok = t0 + tid;
  r.beta = (tid < kC && tok < T) ? beta[tok] : 0.0f;
  r.lam = (tid < kC && tok < T) ? lam[tok] : 0.0f;
}

__device__ __forceinline__ void unpack8(uint4 w, float out[8]) {
  const uint32_t a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(a[i] << 16);
    out[2 * i + 1] = __uint_as_float(a[i] & 0xffff0000u);
  }
}

__global__ void __launch_bounds__(256)
falcon1_chunked_mfma_kernel(const bf16_t* __restrict__ phi_k, const bf16_t* __restrict__ phi_q,
                            const bf16_t* __restrict__ v, const float* __restrict__ beta,
                            const float* __restrict__ lam, const float* S0,
                            const bf16_t* __restrict__ k_prev, bf16_t* __restrict__ o,
                            float* S_T, int T, float eps, float eps_gamma) {
  __shared__ Smem sm;
  const int tid = threadIdx.x;
  const int w = tid >> 6;          // wave index = owned value-column block
  const int l = tid & 63;
  const int g = l >> 4, c16 = l & 15;
  const int64_t bh = blockIdx.x;
  const bf16_t* K = phi_k + bh * T * kD;
  const bf16_t* Q = phi_q + bh * T * kD;
  const bf16_t* V = v + bh * T * kD;
  const float* Bt = beta + bh * T;
  const float* Lm = lam + bh * T;
  const bf16_t* KP = k_prev ? k_prev + bh * kD : nullptr;
  const bool fresh = (k_prev == nullptr);

  // T's upper blocks and the structurally-zero halves of the M fragments
  // stay zero for the whole run.
  for (int e = tid; e < kC * kP; e += 256) sm.tb[e] = 0;
  for (int e = tid; e < 64 * 4; e += 256) {
    const int ln = e >> 2, k = e & 3;
    sm.mf[((0 * 2 + 0) * 64 + ln) * 8 + 4 + k] = 0;   // M tile (i-block 0, s-block 1)
    sm.mf[((2 * 2 + 1) * 64 + ln) * 8 + 4 + k] = 0;   // M tile (i-block 2, s-block 3)
  }

  // State: wave w owns columns 16w..16w+15, as four 16x16 result tiles
  // (feature blocks fb = 0..3); lane holds rows 16fb + 4g + r of column c16.
  f32x4 S[4];
#pragma unroll
  for (int fb = 0; fb < 4; ++fb)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      S[fb][r] = S0 ? S0[(bh * kD + 16 * fb + 4 * g + r) * kD + 16 * w + c16] : 0.0f;

  ChunkRegs cr;
  load_chunk(cr, K, Q, V, Bt, Lm, KP, T, 0, tid);

  const int nchunks = (T + kC - 1) / kC;
  for (int c = 0; c < nchunks; ++c) {
    const int t0 = c * kC;
    __syncthreads();   // the previous chunk is done with every LDS buffer

    // ---------------- a1: energies, step sizes, decays -----------------
    const int seg = tid & 7;
    float xs[2][8];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      unpack8(cr.x[h], xs[h]);
      float e = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) e = fmaf(xs[h][k], xs[h][k], e);
      e += __shfl_xor(e, 1);
      e += __shfl_xor(e, 2);
      e += __shfl_xor(e, 4);
      if (seg == 0) sm.energy[(tid >> 3) + 32 * h] = e;
    }
    __syncthreads();
    if (w == 0) {
      const int i = l;
      const int tok = t0 + i;
      float eta = 0.f, lg = 0.f;
      if (tok < T) {
        eta = nlms_eta(cr.beta, sm.energy[i], cr.lam, eps, fresh && tok == 0);
        lg = clamped_log_gamma(eta, cr.lam, eps_gamma);
      }
      float gi = lg;                                   // inclusive prefix over the chunk
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const float up = __shfl_up(gi, d);
        if (i >= d) gi += up;
      }
      const float gprev = __shfl_up(gi, 1);
      const float glast = __shfl(gi, 63);
      sm.eta[i] = eta;
      sm.graw[i] = gi;
      sm.gexp[i] = __expf(gi);
      sm.gtail[i] = __expf(glast - gi);
      sm.energy[i] = eta * (i == 0 ? 1.0f : __expf(gprev));   // eta_i e^{g_{i-1}}
    }
    __syncthreads();
    // Stage X, Q (natural) and the scaled transposes of X and V.
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = (tid >> 3) + 32 * h;
      *reinterpret_cast<uint4*>(&sm.xr[row * kP + 8 * seg]) = cr.x[h];
      *reinterpret_cast<uint4*>(&sm.qr[row * kP + 8 * seg]) = cr.q[h];
      const float sg = sm.energy[row], st = sm.gtail[row], se = sm.eta[row];
      float vs[8];
      unpack8(cr.v[h], vs);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int f = 8 * seg + k;
        sm.xg[f * kP + row] = bf(xs[h][k] * sg);
        sm.xh[f * kP + row] = bf(xs[h][k] * st);
        sm.vt[f * kP + row] = bf(vs[k] * se);
      }
    }
    // Prefetch the next chunk while this one is processed.
    if (c + 1 < nchunks) load_chunk(cr, K, Q, V, Bt, Lm, KP, T, t0 + kC, tid);
    __syncthreads();

    // ---------------- a2: decayed Gram (A^T) and decayed Q X^T ----------
    for (int item = w; item < 20; item += 4) {
      const int li = item % 10;
      const int ib = kLowerTiles[li][0], sb = kLowerTiles[li][1];
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      if (item < 10) {
        // G tile (ib, sb) = X_ib X_sb^T; lane gets rows i = 16ib+4g+r, column s.
#pragma unroll
        for (int m = 0; m < 2; ++m)
          acc = mfma32(frag_row(&sm.xr[(16 * ib + c16) * kP], 32 * m, g),
                       frag_row(&sm.xr[(16 * sb + c16) * kP], 32 * m, g), acc);
        const int s = 16 * sb + c16;
        const float gs = sm.graw[s];
        float a4[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * ib + 4 * g + r;
          a4[r] = (s < i) ? sm.eta[i] * __expf(sm.graw[i - 1] - gs) * acc[r] : 0.0f;
        }
        *reinterpret_cast<float4*>(&sm.at[s * kPA + 16 * ib + 4 * g]) =
            make_float4(a4[0], a4[1], a4[2], a4[3]);
      } else {
        // P^T tile (sb, ib) = X_sb Q_ib^T; lane gets rows s = 16sb+4g+r, column i.
#pragma unroll
        for (int m = 0; m < 2; ++m)
          acc = mfma32(frag_row(&sm.xr[(16 * sb + c16) * kP], 32 * m, g),
                       frag_row(&sm.qr[(16 * ib + c16) * kP], 32 * m, g), acc);
        const int i = 16 * ib + c16;
        const float gi = sm.graw[i];
        f32x4 mv;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int s = 16 * sb + 4 * g + r;
          mv[r] = (s <= i) ? __expf(gi - sm.graw[s]) * acc[r] : 0.0f;
        }
        store_half_frag(&sm.mf[((ib * 2 + (sb >> 1)) * 64 + l) * 8 + 4 * (sb & 1)], mv, 1.0f);
      }
    }
    __syncthreads();

    // ---------------- a2: T = (I + A)^{-1} -------------------------------
    if (w == 0) {
      // Diagonal blocks: lane (block b = g, column j = c16) eliminates rows.
      const int b = g, j = c16;
      float t[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) t[i] = (i == j) ? 1.0f : 0.0f;
#pragma unroll
      for (int s = 0; s < 15; ++s) {
        const float* arow = &sm.at[(16 * b + s) * kPA + 16 * b];   // A[16b+i][16b+s], all i
        float a[16];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float4 v4 = *reinterpret_cast<const float4*>(arow + 4 * q4);
          a[4 * q4] = v4.x; a[4 * q4 + 1] = v4.y; a[4 * q4 + 2] = v4.z; a[4 * q4 + 3] = v4.w;
        }
#pragma unroll
        for (int i = s + 1; i < 16; ++i) t[i] = fmaf(-a[i], t[s], t[i]);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) sm.tb[(16 * b + i) * kP + 16 * b + j] = bf(t[i]);
    }
    __syncthreads();
    if (w < 2) {
      // T_{hi,lo} = -T_hi,hi A_hi,lo T_lo,lo for the pairs (1,0) and (3,2).
      const int lo = 2 * w, hi = 2 * w + 1;
      s16x4 af, bfr;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        af[e] = static_cast<short>(bf(sm.at[(16 * lo + 4 * g + e) * kPA + 16 * hi + c16]));
        bfr[e] = static_cast<short>(sm.tb[(16 * lo + 4 * g + e) * kP + 16 * lo + c16]);
      }
      f32x4 y = {0.f, 0.f, 0.f, 0.f};
      y = mfma16(af, bfr, y);                                   // A_hi,lo T_lo,lo
      const uint2 th = *reinterpret_cast<const uint2*>(&sm.tb[(16 * hi + c16) * kP + 16 * hi + 4 * g]);
      s16x4 ta = __builtin_bit_cast(s16x4, th);
      f32x4 z = {0.f, 0.f, 0.f, 0.f};
      z = mfma16(ta, s16_from_acc(y), z);
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.tb[(16 * hi + 4 * g + r) * kP + 16 * lo + c16] = bf(-z[r]);
    }
    __syncthreads();
    if (w < 2) {
      // Lower-left 32x32 block: T_21 = -T_22 A_21 T_11 (2x2 block sense).
      const int cj = w;
      f32x4 y2[2];
#pragma unroll
      for (int ri = 0; ri < 2; ++ri) {
        bf16x8 af, bfr;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int s = (e < 4) ? 4 * g + e : 16 + 4 * g + (e - 4);
          af[e] = static_cast<__bf16>(sm.at[s * kPA + 32 + 16 * ri + c16]);
          bfr[e] = __builtin_bit_cast(__bf16, sm.tb[s * kP + 16 * cj + c16]);
        }
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        y2[ri] = mfma32(af, bfr, acc);
      }
      const bf16x8 yb = frag_from_acc(y2[0], y2[1]);
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = mfma32(frag_row(&sm.tb[(32 + 16 * rr + c16) * kP], 32, g), yb, acc);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          sm.tb[(32 + 16 * rr + 4 * g + r) * kP + 16 * cj + c16] = bf(-acc[r]);
      }
    }
    __syncthreads();

    // ---------------- a2: W^T tiles (fb = w) and U tiles (column block w)
    f32x4 U[4];
    {
      const int fb = w;
#pragma unroll
      for (int ib = 0; ib < 4; ++ib) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        f32x4 uacc = {0.f, 0.f, 0.f, 0.f};
        const int msteps = ib < 2 ? 1 : 2;             // T is lower triangular
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          if (m < msteps) {
            const bf16x8 trow = frag_row(&sm.tb[(16 * ib + c16) * kP], 32 * m, g);
            acc = mfma32(frag_row(&sm.xg[(16 * fb + c16) * kP], 32 * m, g), trow, acc);
            uacc = mfma32(trow, frag_row(&sm.vt[(16 * w + c16) * kP], 32 * m, g), uacc);
          }
        }
        U[ib] = uacc;
        // W^T tile (fb, ib): lane has W[16ib+c16][16fb+4g+r]; store -W as the
        // A fragment (ib, m = fb/2) of R = U - W S.
        store_half_frag(&sm.wf[((ib * 2 + (fb >> 1)) * 64 + l) * 8 + 4 * (fb & 1)], acc, -1.0f);
      }
    }
    __syncthreads();

    // ---------------- a3 + a4: residuals, outputs, state ----------------
    {
      const bf16x8 sb0 = frag_from_acc(S[0], S[1]);
      const bf16x8 sb1 = frag_from_acc(S[2], S[3]);
      f32x4 R[4];
#pragma unroll
      for (int ib = 0; ib < 4; ++ib) {
        f32x4 acc = U[ib];
        acc = mfma32(load_frag(&sm.wf[((ib * 2 + 0) * 64 + l) * 8]), sb0, acc);
        acc = mfma32(load_frag(&sm.wf[((ib * 2 + 1) * 64 + l) * 8]), sb1, acc);
        R[ib] = acc;                                  // rows eta_i r_i of column block w
      }
      const bf16x8 rb0 = frag_from_acc(R[0], R[1]);
      const bf16x8 rb1 = frag_from_acc(R[2], R[3]);
#pragma unroll
      for (int ib = 0; ib < 4; ++ib) {
        const int i = 16 * ib + c16;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = mfma32(sb0, frag_row(&sm.qr[i * kP], 0, g), acc);
        acc = mfma32(sb1, frag_row(&sm.qr[i * kP], 32, g), acc);
        const float ge = sm.gexp[i];
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] *= ge;
        acc = mfma32(rb0, load_frag(&sm.mf[((ib * 2 + 0) * 64 + l) * 8]), acc);
        if (ib >= 2) acc = mfma32(rb1, load_frag(&sm.mf[((ib * 2 + 1) * 64 + l) * 8]), acc);
        const int tok = t0 + i;
        if (tok < T) {
          const uint32_t p0 = uint32_t(bf(acc[0])) | (uint32_t(bf(acc[1])) << 16);
          const uint32_t p1 = uint32_t(bf(acc[2])) | (uint32_t(bf(acc[3])) << 16);
          *reinterpret_cast<uint2*>(o + (bh * T + tok) * kD + 16 * w + 4 * g) = make_uint2(p0, p1);
        }
      }
      const float glast = sm.gexp[kC - 1];
#pragma unroll
      for (int fb = 0; fb < 4; ++fb) {
        f32x4 acc = S[fb];
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] *= glast;
        acc = mfma32(frag_row(&sm.xh[(16 * fb + c16) * kP], 0, g), rb0, acc);
        acc = mfma32(frag_row(&sm.xh[(16 * fb + c16) * kP], 32, g), rb1, acc);
        S[fb] = acc;
      }
    }
  }
  if (S_T) {
#pragma unroll
    for (int fb = 0; fb < 4; ++fb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        S_T[(bh * kD + 16 * fb + 4 * g + r) * kD + 16 * w + c16] = S[fb][r];
  }
}

}  // namespace

bool chunked_mfma_applies(const ProblemArgs& a) {
  return a.bf16 && a.variant == kF1 && a.dk == kD && a.dv == kD && a.C == kC;
}

hipError_t launch_chunked_mfma(const ProblemArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(falcon1_chunked_mfma_kernel, dim3(a.B * a.H), dim3(256), 0, st,
                     static_cast<const bf16_t*>(a.phi_k), static_cast<const bf16_t*>(a.phi_q),
                     static_cast<const bf16_t*>(a.v), a.beta, a.lam, a.S0,
                     static_cast<const bf16_t*>(a.k_prev), static_cast<bf16_t*>(a.o), a.S_T, a.T,
                     a.eps, a.eps_gamma);
  return hipGetLastError();
}

}  // namespace falcon
