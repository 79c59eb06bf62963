// Backward of the chunked Falcon-1 forward (gfx950), float32 gradients.
//
// Forward, per 32-token chunk with incoming state S (g_i the chunk-local
// prefix of log gamma, gp_i = g_{i-1}, G = g_31; x_i, q_i, v_i the chunk's
// shifted keys, queries and values):
//   A_{is} = eta_i e^{gp_i-g_s} (x_i.x_s) (s < i),  T = (I + A)^{-1},
//   W = T Diag(eta e^{gp}) X,  U = T Diag(eta) V,  Xh = Diag(e^{G-g}) X,
//   M_{is} = (q_i.x_s) e^{g_i-g_s} (s <= i),
//   S' = P S + H,  O = Qt S + Ot   with
//   P = e^G I - Xh^T W,  H = Xh^T U,  Qt = Diag(e^g) Q - M W,  Ot = M U
// (the chunk-parallel form of Section 4.2 with the log-space renormalisation
// of Section 4.4 applied per chunk; exact up to rounding).  Training
// differentiates through the update (Section 3), so for L = <dO, O> +
// <dS_T, S_T> the backward is:
//   1. chunk maps P, H and G = Qt^T dO for every chunk (chunk-parallel);
//   2. in one launch, the forward state chain, saving the state S_c entering
//      each chunk, and the reverse adjoint chain: with Lam_c = dL/dS at the
//      end of chunk c, Lam_{c-1} = P_c^T Lam_c + G_c, and dS0 = the last Lam
//      (the two chains need only the maps);
//   3. per chunk (chunk-parallel), reverse mode through the chunk maps from
//      dP = Lam S_c^T, dH = Lam, dQt = dO S_c^T, dOt = dO (dP is never formed:
//      Xh dP = (Xh Lam) S_c^T and W dP^T = (W S_c) Lam^T):
//        dW = -(Xh Lam) S_c^T - M^T dQt,  dU = Xh Lam + M^T dO,  dXh = (U - W S_c) Lam^T,
//        dM = -dQt W^T + dO U^T,  dQ = Diag(e^g) dQt + (dM o D) X,
//        dY = T^T dW,  dZ = T^T dU,  dA = -dY W^T - dZ U^T,
//      then the Gram, the decays and the gates (eta, the clamped log decay,
//      the prefix sums) by the chain rule, and the key shift x_t = phi(k_{t-1}).
// Every product runs on the matrix cores with operands in LDS: in float32
// (v_mfma_f32_16x16x4f32), or, where both operands are bf16 inputs, on the
// bf16 matrix cores, whose products of bf16 numbers are exact and whose
// sums are float32.  T comes from a blocked inverse: the two 16 x 16
// diagonal blocks by substitution (a column per lane), the off-diagonal
// block as -T22 A21 T11.

#include <stddef.h>

#include "falcon_device.h"
#include "falcon_launch.h"
#include "falcon_mfma_frag.h"

namespace falcon {

namespace {

constexpr int kBC = 32;        // chunk length of the backward
constexpr int kD = 64;         // dk = dv
constexpr int kPW = 68;        // float pitch of 64-wide LDS matrices
constexpr int kPN = 36;        // float pitch of 32-wide LDS matrices
constexpr int kThreads = 256;  // four waves
// Per-chunk maps, stored in the operand order of the chain kernel's MFMAs
// (a 16x16 tile per wave and column group, four floats per lane; the chain's
// contraction index k runs over 16m + 4(l>>4) + e at step e of block m, so
// every map is exactly a 16x16 accumulator tile of a product the maps
// kernel forms, stored as it sits in the lanes):
//   PA  P as the A operand of P S:      ((w*4 + m)*64 + l)*4 + e <-> P[16w + (l&15)][16m + 4(l>>4) + e]
//   HD  H in accumulator order:         ((w*4 + cg)*64 + l)*4 + r <-> H[16w + 4(l>>4) + r][16cg + (l&15)]
//   GD  G^T in accumulator order:       ((w*4 + cg)*64 + l)*4 + r <-> G[16w + (l&15)][16cg + 4(l>>4) + r]
// The adjoint chain needs P's column blocks; it reads PA too and regroups it
// through LDS, so P is stored once.
constexpr int kOffPA = 0, kOffHD = 4096, kOffGD = 8192;
constexpr int kMapFloats = 12288;
// Per-chunk forward factors the maps kernel hands to the chunk kernel, row-major:
// W [32][64], U [32][64], T [32][32], then the gates eta, g, gp, den, lam,
// flags (int bits), glo, gplo [32] each (G is g_31).
constexpr int kFacW = 0, kFacU = 2048, kFacT = 4096, kFacGates = 5120;
constexpr int kFacFloats = 5408;   // the gates, then gamma [32]

typedef float f32x4 __attribute__((ext_vector_type(4)));

// D (M x N) = op(A) op(B) on the matrix cores in float32; A is M x K (stored
// K x M when TA), B is K x N (stored N x K when TB), both in LDS with float
// pitches pa, pb (multiples of 4, 16-byte aligned rows).  The 16x16 output
// tiles go round-robin to NW waves (tile w + NW it for wave w < NW; the same
// lane always holds the same output element for given M, N, NW, so such
// products can be summed in registers).  With N / 16 dividing NW, all of a
// wave's tiles share one column block, so the wave reads its B fragments once.  Within
// each 16-wide slice of K, lane group g supplies k = 16m + 4g + e at step e,
// so an operand stored with K contiguous is read 16 bytes at a time.
//
// load() reads the operands into registers, run() issues the MFMAs, store()
// hands each result to epi(row, col, value).  Several products of a phase
// load first, run next and store last, so that their LDS reads overlap and
// no product waits behind another's stores.
template <int M, int N, int K, bool TA, bool TB, int NW = 4>
struct Mm {
  static constexpr int TN = N / 16, TM = M / 16, IT = TM * TN / NW, KS = K / 4;
  static_assert(K % 16 == 0, "K must be a multiple of 16");
  static_assert(TM * TN % NW == 0 && NW % TN == 0, "tiles must split evenly over the waves");
  float bv[KS];
  float av[IT][KS];
  f32x4 acc[IT];

  // ra(row) scales row `row` of op(A); kb(k) scales row k of op(B).
  template <typename RowScale, typename KScale>
  __device__ __forceinline__ void load(const float* A, int pa, const float* B, int pb, int w, int l, RowScale ra,
                                       KScale kb) {
    const int g = l >> 4, c16 = l & 15;
    const int tn = w % TN;
#pragma unroll
    for (int m = 0; m < K / 16; ++m) {
      const int k0 = 16 * m + 4 * g;
      if (TB) {
        const float4 v = *reinterpret_cast<const float4*>(B + (16 * tn + c16) * pb + k0);
        bv[4 * m] = v.x; bv[4 * m + 1] = v.y; bv[4 * m + 2] = v.z; bv[4 * m + 3] = v.w;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) bv[4 * m + e] = B[(k0 + e) * pb + 16 * tn + c16];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) bv[4 * m + e] *= kb(k0 + e);
#pragma unroll
      for (int it = 0; it < IT; ++it) {
        const int tm = (w + NW * it) / TN;
        if (TA) {
#pragma unroll
          for (int e = 0; e < 4; ++e) av[it][4 * m + e] = A[(k0 + e) * pa + 16 * tm + c16];
        } else {
          const float4 v = *reinterpret_cast<const float4*>(A + (16 * tm + c16) * pa + k0);
          av[it][4 * m] = v.x; av[it][4 * m + 1] = v.y; av[it][4 * m + 2] = v.z; av[it][4 * m + 3] = v.w;
        }
      }
    }
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const float sc = ra(16 * ((w + NW * it) / TN) + c16);
#pragma unroll
      for (int k = 0; k < KS; ++k) av[it][k] *= sc;
    }
  }
  template <typename RowScale>
  __device__ __forceinline__ void load(const float* A, int pa, const float* B, int pb, int w, int l, RowScale ra) {
    load(A, pa, B, pb, w, l, ra, [](int) { return 1.f; });
  }
  __device__ __forceinline__ void load(const float* A, int pa, const float* B, int pb, int w, int l) {
    load(A, pa, B, pb, w, l, [](int) { return 1.f; }, [](int) { return 1.f; });
  }
  // with a scale ks(k) along the contraction index (applied to B's rows)
  template <typename KScale>
  __device__ __forceinline__ void load_k(const float* A, int pa, const float* B, int pb, int w, int l, KScale ks) {
    load(A, pa, B, pb, w, l, [](int) { return 1.f; }, ks);
  }
  // acc = op(A) op(B), or init + op(A) op(B)
  __device__ __forceinline__ void run() {
#pragma unroll
    for (int it = 0; it < IT; ++it) acc[it] = f32x4{0.f, 0.f, 0.f, 0.f};
    mac();
  }
  template <int K2, bool TA2, bool TB2>
  __device__ __forceinline__ void run(const Mm<M, N, K2, TA2, TB2, NW>& init) {
#pragma unroll
    for (int it = 0; it < IT; ++it) acc[it] = init.acc[it];
    mac();
  }
  __device__ __forceinline__ void mac() {
#pragma unroll
    for (int k = 0; k < KS; ++k)
#pragma unroll
      for (int it = 0; it < IT; ++it) acc[it] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[it][k], bv[k], acc[it], 0, 0, 0);
  }
  template <typename Epi>
  __device__ __forceinline__ void store(int w, int l, Epi epi) const {
    const int g = l >> 4, c16 = l & 15;
    const int tn = w % TN;
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int tm = (w + NW * it) / TN;
#pragma unroll
      for (int r = 0; r < 4; ++r) epi(16 * tm + 4 * g + r, 16 * tn + c16, acc[it][r]);
    }
  }
};

// The same product with TB and no scales, for operands whose values are
// bfloat16 numbers held as floats (the bf16 inputs: keys and queries): the
// bf16 matrix cores (v_mfma_f32_16x16x32_bf16) form every product exactly
// and accumulate in float32, with an eighth of the instructions.  Lane
// group g supplies k = 32m + kperm(g, e) of its row, so both operands are
// read as two 16-byte runs per 32-wide block; results sit in the lanes as
// in Mm.
template <int M, int N, int K, int NW = 4>
struct MmBf {
  static constexpr int TN = N / 16, TM = M / 16, IT = TM * TN / NW, KB = K / 32;
  static_assert(K % 32 == 0, "K must be a multiple of 32");
  static_assert(TM * TN % NW == 0 && NW % TN == 0, "tiles must split evenly over the waves");
  frag::bf16x8 bv[KB];
  frag::bf16x8 av[IT][KB];
  f32x4 acc[IT];

  // the eight bf16 values of k = k0 .. k0 + 3 and k0 + 16 .. k0 + 19 of a
  // float row (exact: the floats are bf16 numbers)
  static __device__ __forceinline__ frag::bf16x8 pack(const float* row, int k0) {
    const uint4 lo = *reinterpret_cast<const uint4*>(row + k0);
    const uint4 hi = *reinterpret_cast<const uint4*>(row + k0 + 16);
    const uint4 v = make_uint4((lo.x >> 16) | (lo.y & 0xffff0000u), (lo.z >> 16) | (lo.w & 0xffff0000u),
                               (hi.x >> 16) | (hi.y & 0xffff0000u), (hi.z >> 16) | (hi.w & 0xffff0000u));
    return __builtin_bit_cast(frag::bf16x8, v);
  }
  __device__ __forceinline__ void load(const float* A, int pa, const float* B, int pb, int w, int l) {
    const int g = l >> 4, c16 = l & 15;
    const int tn = w % TN;
#pragma unroll
    for (int m = 0; m < KB; ++m) {
      const int k0 = 32 * m + 4 * g;
      bv[m] = pack(B + (16 * tn + c16) * pb, k0);
#pragma unroll
      for (int it = 0; it < IT; ++it) av[it][m] = pack(A + (16 * ((w + NW * it) / TN) + c16) * pa, k0);
    }
  }
  __device__ __forceinline__ void run() {
#pragma unroll
    for (int it = 0; it < IT; ++it) acc[it] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < KB; ++m)
#pragma unroll
      for (int it = 0; it < IT; ++it) acc[it] = frag::mfma32(av[it][m], bv[m], acc[it]);
  }
  template <typename Epi>
  __device__ __forceinline__ void store(int w, int l, Epi epi) const {
    const int g = l >> 4, c16 = l & 15;
    const int tn = w % TN;
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int tm = (w + NW * it) / TN;
#pragma unroll
      for (int r = 0; r < 4; ++r) epi(16 * tm + 4 * g + r, 16 * tn + c16, acc[it][r]);
    }
  }
};

// op(A) op(B) with one operand a bf16 input held as floats and the other any
// float matrix, on the bf16 matrix cores: the float operand (A when SA,
// else B), after its scale ks(k) along the contraction index, is split into
// three bf16 parts hi + mid + lo that sum to it exactly (each part takes the
// next eight significant bits of the 24; only values within a factor 2^16 of
// the smallest normal float lose bits), so each of the three products is exact
// and the result is the float32 product up to the order of its float32
// sums, in three bf16 MFMAs per 32-wide block of k where float32 takes
// eight.  Layouts as in Mm
// (A is M x K, stored K x M when TA; B is K x N, stored N x K when TB).
template <int M, int N, int K, bool TA, bool TB, bool SA, int NW = 4>
struct MmX3 {
  static constexpr int TN = N / 16, TM = M / 16, IT = TM * TN / NW, KB = K / 32;
  static_assert(K % 32 == 0, "K must be a multiple of 32");
  static_assert(TM * TN % NW == 0 && NW % TN == 0, "tiles must split evenly over the waves");
  frag::bf16x8 ar[SA ? 1 : IT][KB], br[SA ? KB : 1];   // the bf16 operand
  frag::bf16x8 as[SA ? IT : 1][KB][3], bs[SA ? 1 : KB][3];   // the split operand
  f32x4 acc[IT];

  // k = 32m + kperm(g, e) of row r of a matrix stored with k contiguous
  // (tr = false) or of column r of one stored with k as its row index
  static __device__ __forceinline__ void read8(const float* X, int p, int r, int kb, int g, bool tr, float (&v)[8]) {
    if (!tr) {
      const float4 lo = *reinterpret_cast<const float4*>(X + r * p + kb + 4 * g);
      const float4 hi = *reinterpret_cast<const float4*>(X + r * p + kb + 16 + 4 * g);
      v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w; v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = X[(kb + (e < 4 ? 4 * g + e : 12 + 4 * g + e)) * p + r];
    }
  }
  static __device__ __forceinline__ frag::bf16x8 exact(const float (&v)[8]) {
    uint32_t u[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) u[q] = (__float_as_uint(v[2 * q]) >> 16) | (__float_as_uint(v[2 * q + 1]) & 0xffff0000u);
    return __builtin_bit_cast(frag::bf16x8, make_uint4(u[0], u[1], u[2], u[3]));
  }
  // The parts by truncation: hi keeps the top eight significant bits of x,
  // x - hi (exact) has at most sixteen, mid keeps its top eight, and the
  // exact remainder lo has at most eight, so every part is a bf16 number
  // and the sixteen-bit halves are the parts' bf16 encodings.
  template <typename KScale>
  static __device__ __forceinline__ void split(float (&v)[8], int kb, int g, KScale ks, frag::bf16x8 (&d)[3]) {
    uint32_t p[3][8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = v[e] * ks(kb + (e < 4 ? 4 * g + e : 12 + 4 * g + e));
      const uint32_t hb = __float_as_uint(x) & 0xffff0000u;
      const float r1 = x - __uint_as_float(hb);
      const uint32_t mb = __float_as_uint(r1) & 0xffff0000u;
      const float r2 = r1 - __uint_as_float(mb);
      p[2][e] = hb;
      p[1][e] = mb;
      p[0][e] = __float_as_uint(r2);
    }
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      uint32_t u[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) u[q] = (p[j][2 * q] >> 16) | (p[j][2 * q + 1] & 0xffff0000u);
      d[j] = __builtin_bit_cast(frag::bf16x8, make_uint4(u[0], u[1], u[2], u[3]));
    }
  }
  template <typename KScale>
  __device__ __forceinline__ void load(const float* A, int pa, const float* B, int pb, int w, int l, KScale ks) {
    const int g = l >> 4, c16 = l & 15;
    const int tn = w % TN;
#pragma unroll
    for (int m = 0; m < KB; ++m) {
      float v[8];
      read8(B, pb, 16 * tn + c16, 32 * m, g, !TB, v);
      if (SA) br[SA ? m : 0] = exact(v);
      else split(v, 32 * m, g, ks, bs[SA ? 0 : m]);
#pragma unroll
      for (int it = 0; it < IT; ++it) {
        read8(A, pa, 16 * ((w + NW * it) / TN) + c16, 32 * m, g, TA, v);
        if (SA) split(v, 32 * m, g, ks, as[SA ? it : 0][m]);
        else ar[SA ? 0 : it][m] = exact(v);
      }
    }
  }
  __device__ __forceinline__ void load(const float* A, int pa, const float* B, int pb, int w, int l) {
    load(A, pa, B, pb, w, l, [](int) { return 1.f; });
  }
  template <typename KScale>
  __device__ __forceinline__ void load_k(const float* A, int pa, const float* B, int pb, int w, int l, KScale ks) {
    load(A, pa, B, pb, w, l, ks);
  }
  __device__ __forceinline__ void run() {
#pragma unroll
    for (int it = 0; it < IT; ++it) acc[it] = f32x4{0.f, 0.f, 0.f, 0.f};
    mac();
  }
  // the small parts first, so the float32 sums meet them before the large
  __device__ __forceinline__ void mac() {
#pragma unroll
    for (int m = 0; m < KB; ++m)
#pragma unroll
      for (int j = 0; j < 3; ++j)
#pragma unroll
        for (int it = 0; it < IT; ++it)
          acc[it] = SA ? frag::mfma32(as[SA ? it : 0][m][j], br[SA ? m : 0], acc[it])
                       : frag::mfma32(ar[SA ? 0 : it][m], bs[SA ? 0 : m][j], acc[it]);
  }
  template <typename Epi>
  __device__ __forceinline__ void store(int w, int l, Epi epi) const {
    const int g = l >> 4, c16 = l & 15;
    const int tn = w % TN;
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int tm = (w + NW * it) / TN;
#pragma unroll
      for (int r = 0; r < 4; ++r) epi(16 * tm + 4 * g + r, 16 * tn + c16, acc[it][r]);
    }
  }
};

// op(A) op(B) with the bf16 input operand on the side named by SA's
// complement: bf16 matrix cores with a three-way split when the inputs are
// bf16, Mm in float32 otherwise.  ks scales the other operand along k.
template <typename IO, int M, int N, int K, bool TA, bool TB, bool SA, int NW = 4>
struct InputProduct { using type = MmX3<M, N, K, TA, TB, SA, NW>; };
template <int M, int N, int K, bool TA, bool TB, bool SA, int NW>
struct InputProduct<float, M, N, K, TA, TB, SA, NW> { using type = Mm<M, N, K, TA, TB, NW>; };

// Products of two input matrices (x_i . x_s, q_i . x_s): on the bf16 matrix
// cores when the inputs are bf16, in float32 otherwise.
template <typename IO> struct InputGram { using type = Mm<kBC, kBC, kD, false, true>; };
template <> struct InputGram<bf16_t> { using type = MmBf<kBC, kBC, kD>; };

// One product: load, run, store.
template <int M, int N, int K, bool TA, bool TB, typename Epi>
__device__ __forceinline__ void mm(const float* A, int pa, const float* B, int pb, int w, int l, Epi epi) {
  Mm<M, N, K, TA, TB> f;
  f.load(A, pa, B, pb, w, l);
  f.run();
  f.store(w, l, epi);
}

// v plus its value in the lane a DPP move (control CTRL) names: quad_perm
// [1,0,3,2] (0xb1) and [2,3,0,1] (0x4e) pair lanes l ^ 1 and l ^ 2, the
// half-row mirror (0x141) pairs the two quads of eight lanes and the row
// mirror (0x140) the two halves of sixteen.  Called by every lane.
template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}

// The value of the lane N places lower in the same sixteen-lane DPP row, 0
// for the first N lanes of the row.
template <int N>
__device__ __forceinline__ float row_shr(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x110 + N, 0xf, 0xf, true));
}

// The value of the lane N places higher in the same sixteen-lane DPP row, 0
// for the last N lanes of the row.
template <int N>
__device__ __forceinline__ float row_shl(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x100 + N, 0xf, 0xf, true));
}

// Sum over the eight consecutive lanes that share a row.
__device__ __forceinline__ float sum8(float v) {
  v = dpp_add<0xb1>(v);
  v = dpp_add<0x4e>(v);
  return dpp_add<0x141>(v);
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
  float* maps;     // per chunk: PA, HD, GD (above)
  float* ckpt;     // per chunk: S entering the chunk, ((cg*4 + w)*64 + l)*4 + r <-> S[16w + 4(l>>4) + r][16cg + (l&15)]
  float* adj;      // per chunk: dL/dS at its end, ((cg*4 + w)*64 + l)*4 + r <-> Lam[16w + (l&15)][16cg + 4(l>>4) + r]
  float* fac;      // per chunk: the forward factors (above)
  int T, nchunks;
  float eps, eps_gamma;
};

// The forward quantities of one chunk, in LDS.
struct __align__(16) ChunkCore {
  float X[kBC][kPW];     // x_i = phi(k_{t0+i-1}); 0 at a fresh start and past T
  float Q[kBC][kPW];     // q_i; 0 past T
  float V[kBC][kPW];     // v_i; 0 past T
  float W[kBC][kPW];
  float U[kBC][kPW];
  float KX[kBC][kPN];    // x_i . x_s
  float AA[kBC][kPN];    // A, strictly lower; then T Diag(eta e^{gp}) (chunk kernel: the pair-term prefixes PT)
  float TT[kBC][kPN];    // T = (I + A)^{-1}
  float MM[kBC][kPN];    // M, lower with the diagonal
  float ZZ[16][20];      // A21 T11
  // log-decay prefixes g_i (through row i) and gp_i = g_{i-1}, each as a
  // float pair hi + lo, lo the part the float sums dropped; G = g_31
  float2 g[kBC], gp[kBC], G;
  float en[kBC], eta[kBC], lamv[kBC], den[kBC];
  float gam[kBC];        // gamma_i = 1 - eta_i lam_i, or eps_gamma where the clamp binds
  int flags[kBC];        // 1: eta from the formula, 2: the clamp binds, 4: live row
};

// Decays from the compensated prefixes (g = hi + lo, lo the part the float
// sums dropped): e^{g_r - g_s} as e^{hi_r - hi_s} (1 + lo_r - lo_s), whose
// hi difference rounds relative to itself, so a decay between nearby rows
// keeps float accuracy however large the prefixes grow (a binding clamp adds
// |log eps_gamma| per row); e^{g} likewise.
__device__ __forceinline__ float dexp(float2 r, float2 s) {
  const float e = __expf(r.x - s.x);
  return fmaf(e, r.y - s.y, e);
}
__device__ __forceinline__ float eexp(float2 h) {
  const float e = __expf(h.x);
  return fmaf(e, h.y, e);
}

// Eight consecutive elements of a row (16-byte aligned), held as loaded and
// widened to float only when used, so that every load of a phase can be
// issued before the first wait.
template <typename IO> struct Raw8;
template <> struct Raw8<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = reinterpret_cast<const float4*>(p)[0];
    b = reinterpret_cast<const float4*>(p)[1];
  }
  __device__ __forceinline__ void get(float (&o)[8]) const {
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w; o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
  }
};
template <> struct Raw8<bf16_t> {
  uint4 r;
  __device__ __forceinline__ void load(const bf16_t* p) { r = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void get(float (&o)[8]) const {
    const uint32_t u[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      o[2 * k] = __uint_as_float(u[k] << 16);
      o[2 * k + 1] = __uint_as_float(u[k] & 0xffff0000u);
    }
  }
};
// One element held as loaded (the bf16 bit pattern, or the float).
template <typename IO> struct Raw1;
template <> struct Raw1<float> {
  float x;
  __device__ __forceinline__ void load(const float* p) { x = *p; }
  __device__ __forceinline__ float get() const { return x; }
};
template <> struct Raw1<bf16_t> {
  uint32_t x;
  __device__ __forceinline__ void load(const bf16_t* p) { x = p->bits; }
  __device__ __forceinline__ float get() const { return __uint_as_float(x << 16); }
};

template <typename IO>
__device__ __forceinline__ float ld_row(const IO* base, int64_t row, int col) {
  return io<IO>::load(base, row * kD + col);
}

// This thread's share of a chunk's inputs: row tid >> 3, columns 8 (tid & 7) + 0..7.
template <typename IO>
struct ChunkRegs {
  Raw8<IO> x, q, v;
  float beta, lam;
  bool live, xlive, glive;
};

template <typename IO>
__device__ __forceinline__ void chunk_load(ChunkRegs<IO>& r, const BwdArgs& a, int64_t bh, int c, int tid) {
  // Loads are unconditional (rows past T and a missing previous key read a
  // valid row) and masked when stored, so no branch separates them.
  const int T = a.T;
  const int i = tid >> 3, f0 = (tid & 7) * 8;
  const int t = c * kBC + i;
  r.live = t < T;
  const int tc = r.live ? t : T - 1;
  const IO* K = static_cast<const IO*>(a.phi_k) + bh * T * kD;
  const IO* Qp = static_cast<const IO*>(a.phi_q) + bh * T * kD;
  const IO* V = static_cast<const IO*>(a.v) + bh * T * kD;
  const IO* kp = a.k_prev ? static_cast<const IO*>(a.k_prev) + bh * kD : K;
  r.xlive = r.live && (t >= 1 || a.k_prev != nullptr);
  // key row t - 1 for a live row t >= 1; any other row reads row 0 (T >= 1)
  r.x.load((t == 0 ? kp : K + int64_t(r.live ? t - 1 : 0) * kD) + f0);
  r.q.load(Qp + int64_t(tc) * kD + f0);
  r.v.load(V + int64_t(tc) * kD + f0);
  const int tg = c * kBC + (tid & 31);
  r.glive = tid < kBC && tg < T;
  const int tgc = tg < T ? tg : T - 1;
  r.beta = a.beta[bh * T + tgc];
  r.lam = a.lam[bh * T + tgc];
}

template <typename IO>
// enp: the thread's partial key energy, in double precision (the eight
// partials of row i at enp[8i ..]).
__device__ __forceinline__ void chunk_store(ChunkCore& cc, const ChunkRegs<IO>& r, int tid, double* enp,
                                            bool gate_inputs = true) {
  const int i = tid >> 3, f0 = (tid & 7) * 8;
  float x[8], q[8], v[8];
  r.x.get(x);
  r.q.get(q);
  r.v.get(v);
  float e = 0.f;
  double ed = 0.0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    x[k] = r.xlive ? x[k] : 0.f;
    q[k] = r.live ? q[k] : 0.f;
    v[k] = r.live ? v[k] : 0.f;
    e = fmaf(x[k], x[k], e);
    ed = fma(double(x[k]), double(x[k]), ed);
  }
  enp[tid] = ed;
#pragma unroll
  for (int k = 0; k < 8; k += 4) {
    *reinterpret_cast<float4*>(&cc.X[i][f0 + k]) = make_float4(x[k], x[k + 1], x[k + 2], x[k + 3]);
    *reinterpret_cast<float4*>(&cc.Q[i][f0 + k]) = make_float4(q[k], q[k + 1], q[k + 2], q[k + 3]);
    *reinterpret_cast<float4*>(&cc.V[i][f0 + k]) = make_float4(v[k], v[k + 1], v[k + 2], v[k + 3]);
  }
  e = sum8(e);
  if ((tid & 7) == 0) cc.en[i] = e;
  if (gate_inputs && tid < kBC) {
    cc.lamv[tid] = r.glive ? r.lam : 0.f;
    cc.den[tid] = r.glive ? r.beta : 0.f;   // beta until the gates replace it by the denominator
  }
}

// Gates, the Gram, A, M, the inverse T and the factors W, U of one chunk whose
// inputs are in LDS (after a barrier), on four waves.  The Gram and Q X^T are
// issued first; wave 0 forms the gates while its products run, and the
// decays are applied from the registers after the barrier.  Ends with a
// barrier.
template <typename IO>
__device__ void chunk_forward(ChunkCore& cc, const BwdArgs& a, int c, int tid, int w, int l, const double* enp) {
  const int T = a.T;
  const int t0 = c * kBC;
  const bool fresh = (a.k_prev == nullptr);
  typename InputGram<IO>::type fk, fm;
  fk.load(&cc.X[0][0], kPW, &cc.X[0][0], kPW, w, l);
  fm.load(&cc.Q[0][0], kPW, &cc.X[0][0], kPW, w, l);
  fk.run();
  fm.run();
  if (w == 0) {
    // gates of row i (Eq. 3.4; Section 4.3 clamp; Section 3 fresh-start
    // sentinel), then the chunk-local prefix sums of the log decays
    const int i = l, t = t0 + i;
    float lg = 0.f;
    if (i < kBC) {
      const bool live = t < T;
      const float lamv = cc.lamv[i], beta = cc.den[i];
      // gamma = 1 - beta lam / den = (den - beta lam) / den cancels down to
      // gamma wherever the decay is small, so the energy, the denominator
      // and the numerator den - beta lam are formed in double precision (the
      // row's key is exact in float): float sums would leave gamma a
      // relative error of about 1e-7 / gamma, which the gradient of the log
      // decay, divided by gamma, would carry (beta in (1, 2) puts gamma
      // anywhere in (0, 1))
      double e64 = 0.0;
#pragma unroll
      for (int k = 0; k < 8; ++k) e64 += enp[8 * i + k];
      const double den64 = e64 + double(lamv) + double(a.eps);
      const double num64 = fma(-double(beta), double(lamv), den64);
      const bool on = live && !(fresh && t == 0) && den64 != 0.0;
      const float den = float(den64);
      const float eta = on ? beta / den : 0.0f;
      const float gam = on ? float(num64) / den : 1.0f;
      // a binding clamp gives gamma = eps_gamma exactly
      const bool clamped = on && !(num64 >= double(a.eps_gamma) * den64);
      lg = live ? (clamped ? logf(a.eps_gamma) : logf(gam)) : 0.0f;
      cc.eta[i] = eta;
      cc.den[i] = den;
      cc.gam[i] = clamped ? a.eps_gamma : gam;
      cc.flags[i] = (on ? 1 : 0) | (clamped ? 2 : 0) | (live ? 4 : 0);
    }
    // inclusive prefix over the chunk, compensated: each partial sum is
    // carried as gi + ge, the rounding error of every addition (two-sum)
    // going into ge
    // (within 16-lane rows on DPP shifts, whose 0 past a row start adds
    // exactly; then row 1 adds row 0's total)
    float gi = lg, ge = 0.f;
    auto add2 = [&](float n, float ne) {
      const float sum = gi + n;
      const float nb = sum - gi;
      const float err = (gi - (sum - nb)) + (n - nb);
      gi = sum;
      ge += ne + err;
    };
    add2(row_shr<1>(gi), row_shr<1>(ge));
    add2(row_shr<2>(gi), row_shr<2>(ge));
    add2(row_shr<4>(gi), row_shr<4>(ge));
    add2(row_shr<8>(gi), row_shr<8>(ge));
    const float g15 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gi), 15));
    const float e15 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ge), 15));
    const bool row1 = (i & 31) >= 16;
    add2(row1 ? g15 : 0.f, row1 ? e15 : 0.f);
    // exclusive: the lane below's value (lane 16 takes lane 15's)
    const float gpv = row_shr<1>(gi) + ((i & 31) == 16 ? g15 : 0.f);
    const float gpe = row_shr<1>(ge) + ((i & 31) == 16 ? e15 : 0.f);
    if (i < kBC) {
      cc.g[i] = make_float2(gi, ge);
      cc.gp[i] = i == 0 ? make_float2(0.f, 0.f) : make_float2(gpv, gpe);
      if (i == kBC - 1) cc.G = make_float2(gi, ge);
    }
  }
  __syncthreads();
  // A = tril(Diag(eta) K o e^{gp_i - g_s}, -1), M = tril(Q X^T o e^{g_i - g_s})
  fk.store(w, l, [&](int r, int s, float v) {
    cc.KX[r][s] = v;
    cc.AA[r][s] = s < r ? cc.eta[r] * dexp(cc.gp[r], cc.g[s]) * v : 0.f;
  });
  fm.store(w, l, [&](int r, int s, float v) {
    cc.MM[r][s] = s <= r ? dexp(cc.g[r], cc.g[s]) * v : 0.f;
  });
  __syncthreads();
  // T11, T22 by substitution: lane j solves (I + A_bb) t = e_jj, b = j / 16
  if (tid < kBC) {
    const int b = tid >> 4, jj = tid & 15, o = 16 * b;
    float col[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float acc = i == jj ? 1.f : 0.f;
#pragma unroll
      for (int s = 0; s < i; ++s) acc = fmaf(-cc.AA[o + i][o + s], col[s], acc);
      col[i] = acc;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) cc.TT[o + i][o + jj] = col[i];
  } else if (tid >= 64 && tid < 64 + 256 / 2) {
    // upper-right block of T is zero
    const int e = tid - 64;
    cc.TT[e >> 3][16 + 2 * (e & 7)] = 0.f;
    cc.TT[e >> 3][17 + 2 * (e & 7)] = 0.f;
  }
  __syncthreads();
  if (tid < 256) {
    // Z = A21 T11
    const int i = tid >> 4, j = tid & 15;
    float z = 0.f;
#pragma unroll
    for (int s = 0; s < 16; ++s) z = fmaf(cc.AA[16 + i][s], cc.TT[s][j], z);
    cc.ZZ[i][j] = z;
  }
  __syncthreads();
  if (tid < 256) {
    // T21 = -T22 Z
    const int i = tid >> 4, j = tid & 15;
    float z = 0.f;
#pragma unroll
    for (int s = 0; s < 16; ++s) z = fmaf(cc.TT[16 + i][16 + s], cc.ZZ[s][j], z);
    cc.TT[16 + i][j] = -z;
  }
  __syncthreads();
}

// W = T Diag(eta e^{gp}) X and U = T Diag(eta) V, with TZ = T Diag(eta) in
// the caller's 32 x 36 scratch; AA becomes T Diag(eta e^{gp}).  Ends with a barrier.
template <typename IO>
__device__ void chunk_factors(ChunkCore& cc, float (*TZ)[kPN], int tid, int w, int l) {
  for (int e = tid; e < kBC * kBC; e += kThreads) {
    const int i = e >> 5, s = e & 31;
    const float t = cc.TT[i][s];
    cc.AA[i][s] = t * cc.eta[s] * eexp(cc.gp[s]);
    TZ[i][s] = t * cc.eta[s];
  }
  __syncthreads();
  typename InputProduct<IO, kBC, kD, kBC, false, false, true>::type fw, fu;
  fw.load(&cc.AA[0][0], kPN, &cc.X[0][0], kPW, w, l);
  fu.load(&TZ[0][0], kPN, &cc.V[0][0], kPW, w, l);
  fw.run();
  fu.run();
  fw.store(w, l, [&](int r, int s, float v) { cc.W[r][s] = v; });
  fu.store(w, l, [&](int r, int s, float v) { cc.U[r][s] = v; });
  __syncthreads();
}

// ---- launch 1: chunk maps --------------------------------------------------------
// Persistent like the chunk kernel: workgroup b handles chunks b, b +
// gridDim.x, ... and loads the next chunk's inputs while it works on the
// current one.
template <typename IO>
struct MapRegs {
  ChunkRegs<IO> r;
  Raw8<IO> odr;
  bool olive;
};

template <typename IO>
__device__ __forceinline__ void map_load(MapRegs<IO>& m, const BwdArgs& a, int job, int tid) {
  const int64_t bh = job / a.nchunks;
  const int c = job % a.nchunks;
  const int T = a.T;
  chunk_load<IO>(m.r, a, bh, c, tid);
  const int orow = c * kBC + (tid >> 3);
  m.olive = orow < T;
  m.odr.load(static_cast<const IO*>(a.dO) + (bh * T + (orow < T ? orow : T - 1)) * kD + (tid & 7) * 8);
}

template <typename IO>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
falcon1_bwd_maps_kernel(BwdArgs a, int total) {
  __shared__ ChunkCore cc;
  __shared__ float TZ[kBC][kPN];
  __shared__ __align__(16) float DO[kBC][kPW];
  __shared__ double ENP[kBC * 8];
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;   // wave-uniform
  const int first = blockIdx.x;
  if (first >= total) return;   // whole workgroup
  MapRegs<IO> in;
  map_load<IO>(in, a, first, tid);
  for (int job = first; job < total; job += gridDim.x) {
  const int c = job % a.nchunks;
  {
    chunk_store<IO>(cc, in.r, tid, ENP);
    float od[8];
    in.odr.get(od);
#pragma unroll
    for (int k = 0; k < 8; ++k) od[k] = in.olive ? od[k] : 0.f;
    const int i = tid >> 3, f0 = (tid & 7) * 8;
    *reinterpret_cast<float4*>(&DO[i][f0]) = make_float4(od[0], od[1], od[2], od[3]);
    *reinterpret_cast<float4*>(&DO[i][f0 + 4]) = make_float4(od[4], od[5], od[6], od[7]);
  }
  __syncthreads();
  // the next chunk's inputs (this chunk's again after the last one)
  map_load<IO>(in, a, job + int(gridDim.x) < total ? job + int(gridDim.x) : job, tid);
  chunk_forward<IO>(cc, a, c, tid, w, l, ENP);
  chunk_factors<IO>(cc, TZ, tid, w, l);
  {
    // W, U, T and the gates for the chunk kernel
    float* fo = a.fac + int64_t(job) * kFacFloats;
    for (int q = tid; q < 512; q += kThreads) {
      const int i = q >> 4, f = 4 * (q & 15);
      reinterpret_cast<float4*>(fo + kFacW)[q] = *reinterpret_cast<const float4*>(&cc.W[i][f]);
      reinterpret_cast<float4*>(fo + kFacU)[q] = *reinterpret_cast<const float4*>(&cc.U[i][f]);
    }
    {
      const int i = tid >> 3, f = 4 * (tid & 7);
      reinterpret_cast<float4*>(fo + kFacT)[tid] = *reinterpret_cast<const float4*>(&cc.TT[i][f]);
    }
    {
      const int k = tid >> 5, i = tid & 31;
      float v;
      switch (k) {
        case 0: v = cc.eta[i]; break;
        case 1: v = cc.g[i].x; break;
        case 2: v = cc.gp[i].x; break;
        case 3: v = cc.den[i]; break;
        case 4: v = cc.lamv[i]; break;
        case 5: v = __int_as_float(cc.flags[i]); break;
        case 6: v = cc.g[i].y; break;
        default: v = cc.gp[i].y; break;
      }
      fo[kFacGates + tid] = v;
      if (tid < kBC) fo[kFacGates + 256 + tid] = cc.gam[tid];
    }
  }
  // KX and AA (two adjacent 32 x 36 arrays, dead after the factors) hold Qt.
  float (*QT)[kPW] = reinterpret_cast<float (*)[kPW]>(&cc.KX[0][0]);
  static_assert(sizeof(cc.KX) + sizeof(cc.AA) >= sizeof(float) * kBC * kPW, "Qt does not fit");
  static_assert(offsetof(ChunkCore, AA) == offsetof(ChunkCore, KX) + sizeof(cc.KX), "KX, AA not adjacent");
  // Qt = Diag(e^g) Q - M W
  mm<kBC, kD, kBC, false, false>(&cc.MM[0][0], kPN, &cc.W[0][0], kPW, w, l, [&](int r, int s, float v) {
    QT[r][s] = eexp(cc.g[r]) * cc.Q[r][s] - v;
  });
  __syncthreads();
  // P^T = e^G I - W^T Diag(e^{G-g}) X, H = X^T Diag(e^{G-g}) U and
  // G^T = dO^T Qt, each written straight from the accumulators: the tile
  // (tm, tn) of a wave is one 1 KiB run of its map.
  float* out = a.maps + int64_t(job) * kMapFloats;
  const float eG = eexp(cc.G);
  auto xs = [&](int t) { return dexp(cc.G, cc.g[t]); };
  auto put = [&](float* base, int idx, const f32x4& v) {
    reinterpret_cast<float4*>(base)[idx] = make_float4(v[0], v[1], v[2], v[3]);
  };
  const int g4 = 4 * (l >> 4), c16 = l & 15;
  {
    typename InputProduct<IO, kD, kD, kBC, true, false, true>::type fpt;
    fpt.load_k(&cc.W[0][0], kPW, &cc.X[0][0], kPW, w, l, xs);
    fpt.run();
#pragma unroll
    for (int it = 0; it < fpt.IT; ++it) {
      const int tm = it, tn = w;   // N = 64 over four waves: column block w, row block it
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float d = (16 * tm + g4 + r == 16 * tn + c16) ? eG : 0.f;
        fpt.acc[it][r] = d - fpt.acc[it][r];
      }
      // P^T tile (tm, tn) is PA block (w = tn, m = tm)
      put(out + kOffPA, (tn * 4 + tm) * 64 + l, fpt.acc[it]);
    }
  }
  {
    typename InputProduct<IO, kD, kD, kBC, true, false, false>::type fh, fg;
    fh.load_k(&cc.X[0][0], kPW, &cc.U[0][0], kPW, w, l, xs);
    fg.load(&DO[0][0], kPW, &QT[0][0], kPW, w, l);
    fh.run();
    fg.run();
#pragma unroll
    for (int it = 0; it < fh.IT; ++it) {
      const int tm = it, tn = w;
      // H tile (tm, tn) is HD block (w = tm, cg = tn); G^T tile (tm, tn) is GD block (w = tn, cg = tm)
      put(out + kOffHD, (tm * 4 + tn) * 64 + l, fh.acc[it]);
      put(out + kOffGD, (tn * 4 + tm) * 64 + l, fg.acc[it]);
    }
  }
  __syncthreads();   // LDS is refilled for the next chunk
  }
}

// ---- launch 2: the state chain and the adjoint chain ---------------------------
// Columns of S evolve independently under S' = P S + H, and so do the rows of
// Lam^T under Lam^T' = Lam^T P + G^T, so each sequence's chains split
// into four 16-column groups.  One workgroup runs one (chain, sequence,
// group); its four waves own the 16-row blocks of the 64 x 16 block, held in
// MFMA accumulators, and share the block through LDS.  Each chunk's operands
// are loaded kRing chunks ahead of their use.  The four groups
// of a (chain, sequence) are placed on one XCD (workgroups go round-robin over
// the eight XCDs), so P is fetched from HBM once per XCD L2.
// Double-buffered by the parity of the step, so one barrier per step
// suffices: a step writes the buffers the step before last read, and every
// wave has passed the last step's barrier after those reads.
union ChainSmem {
  float Bt[2][16][kPW];  // state chain: S[:, 16cg .. 16cg+15] transposed (Bt[c][k] = S[k][16cg + c])
  struct {
    float L[2][16][kPW]; // adjoint chain: Lam^T[16cg .. 16cg+15][:]
    float P[2][kD][kPW]; // adjoint chain: this chunk's P
  } j;
};

constexpr int kRing = 3;   // chunks of operands in flight per chain

// The chain loops run full groups of kRing steps whose prefetches are
// unconditional (a prefetch past the last chunk re-reads the last chunk), so
// the compiler knows how many loads follow each one and waits only for the
// oldest; the last n % kRing steps run without prefetches.
template <typename IO>
__device__ __forceinline__ void chain_state(const BwdArgs& a, ChainSmem& sm, int64_t bh, int cg, int w, int l) {
  const int g = l >> 4, c16 = l & 15;
  const int n = a.nchunks;
  // S0 block in accumulator order: lane holds S[16w + 4g + r][16cg + c16]
  f32x4 S;
#pragma unroll
  for (int r = 0; r < 4; ++r) S[r] = a.S0 ? a.S0[bh * kD * kD + (16 * w + 4 * g + r) * kD + 16 * cg + c16] : 0.f;
  const float* mp = a.maps + bh * n * kMapFloats;
  float4 pa[kRing][4], hd[kRing];
  auto load = [&](int c, float4 (&p4)[4], float4& h) __attribute__((always_inline)) {
    const float* cp = mp + (c < n ? c : n - 1) * kMapFloats;
#pragma unroll
    for (int m = 0; m < 4; ++m) p4[m] = reinterpret_cast<const float4*>(cp + kOffPA)[(w * 4 + m) * 64 + l];
    h = reinterpret_cast<const float4*>(cp + kOffHD)[(w * 4 + cg) * 64 + l];
  };
  auto step = [&](int c, const float4 (&p4)[4], const float4& h) __attribute__((always_inline)) {
    // S (entering chunk c) to LDS and to the checkpoint, then S <- P S + H
    float (*Bt)[kPW] = sm.Bt[c & 1];
    *reinterpret_cast<float4*>(&Bt[c16][16 * w + 4 * g]) = make_float4(S[0], S[1], S[2], S[3]);
    float* ck = a.ckpt + (bh * n + c) * kD * kD;
    reinterpret_cast<float4*>(ck)[(cg * 4 + w) * 64 + l] = make_float4(S[0], S[1], S[2], S[3]);
    __syncthreads();
    // k = 16m + 4g + e; one accumulator per k block m, so the four dependent
    // MFMA chains interleave
    float4 b4[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) b4[m] = *reinterpret_cast<const float4*>(&Bt[c16][16 * m + 4 * g]);
    f32x4 acc[4] = {{h.x, h.y, h.z, h.w}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[m] = __builtin_amdgcn_mfma_f32_16x16x4f32(p4[m].x, b4[m].x, acc[m], 0, 0, 0);
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[m] = __builtin_amdgcn_mfma_f32_16x16x4f32(p4[m].y, b4[m].y, acc[m], 0, 0, 0);
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[m] = __builtin_amdgcn_mfma_f32_16x16x4f32(p4[m].z, b4[m].z, acc[m], 0, 0, 0);
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[m] = __builtin_amdgcn_mfma_f32_16x16x4f32(p4[m].w, b4[m].w, acc[m], 0, 0, 0);
    S = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  };
  // the ring slots are named explicitly (slot d holds chunk c0 + d), so they
  // stay in registers
  static_assert(kRing == 3, "the ring is unrolled by hand");
  load(0, pa[0], hd[0]);
  load(1, pa[1], hd[1]);
  load(2, pa[2], hd[2]);
  int c0 = 0;
  for (; c0 + kRing <= n; c0 += kRing) {
    step(c0 + 0, pa[0], hd[0]);
    load(c0 + 0 + kRing, pa[0], hd[0]);
    step(c0 + 1, pa[1], hd[1]);
    load(c0 + 1 + kRing, pa[1], hd[1]);
    step(c0 + 2, pa[2], hd[2]);
    load(c0 + 2 + kRing, pa[2], hd[2]);
  }
  if (c0 + 0 < n) step(c0 + 0, pa[0], hd[0]);
  if (c0 + 1 < n) step(c0 + 1, pa[1], hd[1]);
}

template <typename IO>
__device__ __forceinline__ void chain_adjoint(const BwdArgs& a, ChainSmem& sm, int64_t bh, int cg, int w, int l) {
  const int g = l >> 4, c16 = l & 15;
  const int n = a.nchunks;
  // Lam^T block in accumulator order: lane holds Lam^T[16cg + 4g + r][16w + c16] = Lam[16w + c16][16cg + 4g + r]
  f32x4 Lt;
#pragma unroll
  for (int r = 0; r < 4; ++r)
    Lt[r] = a.dS_T ? a.dS_T[bh * kD * kD + (16 * w + c16) * kD + 16 * cg + 4 * g + r] : 0.f;
  const float* mp = a.maps + bh * n * kMapFloats;
  float4 pb[kRing][4], gd[kRing];
  // operands of step s, which processes chunk n - 1 - s
  auto load = [&](int s, float4 (&p4)[4], float4& g4) __attribute__((always_inline)) {
    const float* cp = mp + (s < n ? n - 1 - s : 0) * kMapFloats;
#pragma unroll
    for (int m = 0; m < 4; ++m) p4[m] = reinterpret_cast<const float4*>(cp + kOffPA)[(w * 4 + m) * 64 + l];
    g4 = reinterpret_cast<const float4*>(cp + kOffGD)[(w * 4 + cg) * 64 + l];
  };
  auto step = [&](int s, const float4 (&p4)[4], const float4& g4) __attribute__((always_inline)) {
    // Lam^T (at the end of chunk c) to LDS and to the adjoint store, then
    // Lam^T <- Lam^T P + G^T
    const int c = n - 1 - s;
    float (*L)[kPW] = sm.j.L[s & 1];
    float (*P)[kPW] = sm.j.P[s & 1];
#pragma unroll
    for (int r = 0; r < 4; ++r) L[4 * g + r][16 * w + c16] = Lt[r];
    // this wave's rows 16w..16w+15 of P (PA order) into LDS; the product below
    // reads P's column block w
    // (stored component-wise: a 16-byte store of the slot itself makes the
    // compiler keep the whole ring in scratch memory)
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const float4 q = p4[m];
      float* dst = &P[16 * w + c16][16 * m + 4 * g];
      dst[0] = q.x; dst[1] = q.y; dst[2] = q.z; dst[3] = q.w;
    }
    float* ad = a.adj + (bh * n + c) * kD * kD;
    reinterpret_cast<float4*>(ad)[(cg * 4 + w) * 64 + l] = make_float4(Lt[0], Lt[1], Lt[2], Lt[3]);
    __syncthreads();
    // k = 16m + 4g + e; one accumulator per k block m (interleaved chains)
    float4 a4[4], b4[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      a4[m] = *reinterpret_cast<const float4*>(&L[c16][16 * m + 4 * g]);
      b4[m] = make_float4(P[16 * m + 4 * g + 0][16 * w + c16], P[16 * m + 4 * g + 1][16 * w + c16],
                          P[16 * m + 4 * g + 2][16 * w + c16], P[16 * m + 4 * g + 3][16 * w + c16]);
    }
    f32x4 acc[4] = {{g4.x, g4.y, g4.z, g4.w}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[m] = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[m].x, b4[m].x, acc[m], 0, 0, 0);
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[m] = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[m].y, b4[m].y, acc[m], 0, 0, 0);
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[m] = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[m].z, b4[m].z, acc[m], 0, 0, 0);
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[m] = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[m].w, b4[m].w, acc[m], 0, 0, 0);
    Lt = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  };
  load(0, pb[0], gd[0]);
  load(1, pb[1], gd[1]);
  load(2, pb[2], gd[2]);
  int s0 = 0;
  for (; s0 + kRing <= n; s0 += kRing) {
    step(s0 + 0, pb[0], gd[0]);
    load(s0 + 0 + kRing, pb[0], gd[0]);
    step(s0 + 1, pb[1], gd[1]);
    load(s0 + 1 + kRing, pb[1], gd[1]);
    step(s0 + 2, pb[2], gd[2]);
    load(s0 + 2 + kRing, pb[2], gd[2]);
  }
  if (s0 + 0 < n) step(s0 + 0, pb[0], gd[0]);
  if (s0 + 1 < n) step(s0 + 1, pb[1], gd[1]);
  if (a.dS0) {
    float* d = a.dS0 + bh * kD * kD + (16 * w + c16) * kD + 16 * cg + 4 * g;
    *reinterpret_cast<float4*>(d) = make_float4(Lt[0], Lt[1], Lt[2], Lt[3]);
  }
}

// At most 168 registers: three waves per SIMD keep all 2 x 4 x B x H
// workgroups of the 8 x 12 training shape resident at once (three per CU),
// so no chain waits for a free CU.
template <typename IO>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3, 3)))
falcon1_bwd_chain_kernel(BwdArgs a, int nunits) {
  __shared__ ChainSmem sm;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;
  // unit u = (sequence, chain); its four column groups share one XCD
  const int b = blockIdx.x;
  const int slot = b >> 3;
  const int cg = slot & 3;
  const int u = (slot >> 2) * 8 + (b & 7);
  if (u >= nunits) return;   // whole workgroup
  const int64_t bh = u >> 1;
  if (u & 1)
    chain_adjoint<IO>(a, sm, bh, cg, w, l);
  else
    chain_state<IO>(a, sm, bh, cg, w, l);
}

// ---- launch 3: reverse mode through one chunk ----------------------------------
// Eight waves: the chunk's LDS (161 KB) allows one workgroup per CU, and a
// single wave per SIMD issues fp32 MFMAs at two thirds of the rate two waves
// reach, so two waves share each SIMD.
constexpr int kThreads3 = 512;
constexpr int kWaves3 = kThreads3 / 64;

struct __align__(16) GradSmem {
  ChunkCore cc;
  float SC[kD][kPW];     // S entering the chunk
  float LL[kD][kPW];     // dL/dS at the end of the chunk
  float DO[kBC][kPW];    // dO, then dZ
  float DQT[kBC][kPW];   // dQt, then dY
  float DW[kBC][kPW];    // Xh Lam, then dW
  float DU[kBC][kPW];    // dU
  float RR[kBC][kPW];    // U - W S, then the dX accumulator
  float DXH[kBC][kPW];   // dXh
  float DM[kBC][kPN];    // T Diag(eta); then dM o D; then D2 = dA o e^{gp_i - g_s}
  float QX[kBC][kPN];    // q_i . x_s
  float dg[kBC], dgp[kBC], deta[kBC], dgt[kBC];   // dgt: the Xh terms
  float trp[kWaves3];
};

// Sum over the sixteen consecutive lanes that share a row.
__device__ __forceinline__ float sum16(float v) {
  return dpp_add<0x140>(sum8(v));
}


// Exclusive prefix sum over the sixteen lanes of a row.
__device__ __forceinline__ float excl16(float v) {
  v += row_shr<1>(v);
  v += row_shr<2>(v);
  v += row_shr<4>(v);
  v += row_shr<8>(v);
  return row_shr<1>(v);
}

// This thread's share of one chunk's inputs, held as loaded.  Every wave
// issues the same loads from addresses chosen without a branch (a branch
// between different loads made the compiler copy the loaded registers, and
// so wait for the loads, right after issuing them): waves 0-3 take the keys
// and queries, waves 4-7 the values and dO, all eight the state, the
// adjoint and W, U; T and the gates go to every 256 threads.
template <typename IO>
struct GradRegs {
  Raw8<IO> m0, m1;     // waves 0-3: x, q; waves 4-7: v, dO (row (tid & 255) >> 3, columns 8 (tid & 7) ..)
  bool live0, live1;   // the rows' masks (x: a live row with a key; q, v, dO: a live row)
  float4 s4[2], l4[2];
  float4 wf, uf, tf;   // W, U (all threads), T (threads < 256)
  float gf;            // gates (threads < 256), gamma (threads 256..)
};

template <typename IO>
__device__ __forceinline__ void grad_load(GradRegs<IO>& g, const BwdArgs& a, int64_t bh, int c, int tid, int w) {
  const int T = a.T;
  const int u = tid & 255;
  const int i = u >> 3, f0 = (u & 7) * 8;
  const int t = c * kBC + i;
  const bool live = t < T;
  const int tc = live ? t : T - 1;
  const bool lo = w < 4;
  const IO* K = static_cast<const IO*>(a.phi_k) + bh * T * kD;
  const IO* kp = a.k_prev ? static_cast<const IO*>(a.k_prev) + bh * kD : K;
  // key row t - 1 for a live row t >= 1; any other row reads row 0 (T >= 1)
  const IO* xr = t == 0 ? kp : K + int64_t(live ? t - 1 : 0) * kD;
  const IO* vr = static_cast<const IO*>(a.v) + (bh * T + tc) * kD;
  const IO* qr = static_cast<const IO*>(a.phi_q) + (bh * T + tc) * kD;
  const IO* dr = static_cast<const IO*>(a.dO) + (bh * T + tc) * kD;
  g.m0.load((lo ? xr : vr) + f0);
  g.m1.load((lo ? qr : dr) + f0);
  g.live0 = lo ? live && (t >= 1 || a.k_prev != nullptr) : live;
  g.live1 = live;
  const float4* ck = reinterpret_cast<const float4*>(a.ckpt + (bh * a.nchunks + c) * kD * kD);
  const float4* ad = reinterpret_cast<const float4*>(a.adj + (bh * a.nchunks + c) * kD * kD);
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    g.s4[k] = ck[tid + k * kThreads3];
    g.l4[k] = ad[tid + k * kThreads3];
  }
  const float* fo = a.fac + (bh * a.nchunks + c) * kFacFloats;
  g.wf = reinterpret_cast<const float4*>(fo + kFacW)[tid];
  g.uf = reinterpret_cast<const float4*>(fo + kFacU)[tid];
  g.tf = reinterpret_cast<const float4*>(fo + kFacT)[u];
  // threads 256.. take gamma (row tid & 31)
  g.gf = fo[kFacGates + (tid < 256 ? tid : 256 + (tid & 31))];
}

template <typename IO>
__device__ __forceinline__ void grad_store(GradSmem& sm, const GradRegs<IO>& g, int tid, int w) {
  const int u = tid & 255;
  {
    const int i = u >> 3, f0 = (u & 7) * 8;
    float m0[8], m1[8];
    g.m0.get(m0);
    g.m1.get(m1);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      m0[k] = g.live0 ? m0[k] : 0.f;
      m1[k] = g.live1 ? m1[k] : 0.f;
    }
    float* d0 = w < 4 ? &sm.cc.X[i][f0] : &sm.cc.V[i][f0];
    float* d1 = w < 4 ? &sm.cc.Q[i][f0] : &sm.DO[i][f0];
    *reinterpret_cast<float4*>(d0) = make_float4(m0[0], m0[1], m0[2], m0[3]);
    *reinterpret_cast<float4*>(d0 + 4) = make_float4(m0[4], m0[5], m0[6], m0[7]);
    *reinterpret_cast<float4*>(d1) = make_float4(m1[0], m1[1], m1[2], m1[3]);
    *reinterpret_cast<float4*>(d1 + 4) = make_float4(m1[4], m1[5], m1[6], m1[7]);
  }
  {
    ChunkCore& cc = sm.cc;
    const int i = tid >> 4, f = 4 * (tid & 15);
    *reinterpret_cast<float4*>(&cc.W[i][f]) = g.wf;
    *reinterpret_cast<float4*>(&cc.U[i][f]) = g.uf;
    if (w < 4) {
      *reinterpret_cast<float4*>(&cc.TT[u >> 3][4 * (u & 7)]) = g.tf;
      {
        const int k = u >> 5, r = u & 31;
        switch (k) {
          case 0: cc.eta[r] = g.gf; break;
          case 1: cc.g[r].x = g.gf; break;
          case 2: cc.gp[r].x = g.gf; break;
          case 3: cc.den[r] = g.gf; break;
          case 4: cc.lamv[r] = g.gf; break;
          case 5: cc.flags[r] = __float_as_int(g.gf); break;
          case 6: cc.g[r].y = g.gf; break;
          default: cc.gp[r].y = g.gf; break;
        }
        // g_31 is G
        if (k == 1 && r == kBC - 1) cc.G.x = g.gf;
        if (k == 6 && r == kBC - 1) cc.G.y = g.gf;
      }
    } else if (tid < 256 + kBC) {
      cc.gam[tid & 31] = g.gf;
    }
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int q = tid + k * kThreads3;
    const int cg = q >> 8, ww = (q >> 6) & 3, lo = q & 15, hi = (q >> 4) & 3;
    sm.SC[16 * ww + 4 * hi + 0][16 * cg + lo] = g.s4[k].x;
    sm.SC[16 * ww + 4 * hi + 1][16 * cg + lo] = g.s4[k].y;
    sm.SC[16 * ww + 4 * hi + 2][16 * cg + lo] = g.s4[k].z;
    sm.SC[16 * ww + 4 * hi + 3][16 * cg + lo] = g.s4[k].w;
    sm.LL[16 * ww + lo][16 * cg + 4 * hi + 0] = g.l4[k].x;
    sm.LL[16 * ww + lo][16 * cg + 4 * hi + 1] = g.l4[k].y;
    sm.LL[16 * ww + lo][16 * cg + 4 * hi + 2] = g.l4[k].z;
    sm.LL[16 * ww + lo][16 * cg + 4 * hi + 3] = g.l4[k].w;
  }
}

// Persistent: workgroup b handles chunks b, b + gridDim.x, ... (sequence-
// major order) and loads the next chunk's inputs while it works on the
// current one, so the loads' latency is hidden behind a whole chunk.
template <typename IO>
__global__ void __launch_bounds__(kThreads3) falcon1_bwd_chunk_kernel(BwdArgs a, int total) {
  __shared__ GradSmem sm;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;
  const int T = a.T;
  ChunkCore& cc = sm.cc;
  // rows of 64 shared by 16 lanes: row ri, columns 4 rp + 0..3
  const int ri = tid >> 4, rp = tid & 15;
  const int first = blockIdx.x;
  if (first >= total) return;   // whole workgroup
  GradRegs<IO> in;
  grad_load<IO>(in, a, first / a.nchunks, first % a.nchunks, tid, w);
  for (int job = first; job < total; job += gridDim.x) {
  const int64_t bh = job / a.nchunks;
  const int c = job % a.nchunks;
  const int t0 = c * kBC;
  grad_store<IO>(sm, in, tid, w);
  __syncthreads();
  {
    // the next chunk's inputs (this chunk's again after the last one)
    const int next = job + gridDim.x < total ? job + int(gridDim.x) : job;
    grad_load<IO>(in, a, next / a.nchunks, next % a.nchunks, tid, w);
  }
  {
    // tr(Lam S^T) = sum of Lam o S, an 8-float slice per thread
    float trace = 0.f;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int e = tid * 8 + 4 * k, rr = e >> 6, cl = e & 63;
      const float4 x = *reinterpret_cast<const float4*>(&sm.LL[rr][cl]);
      const float4 y = *reinterpret_cast<const float4*>(&sm.SC[rr][cl]);
      trace = fmaf(x.x, y.x, fmaf(x.y, y.y, fmaf(x.z, y.z, fmaf(x.w, y.w, trace))));
    }
    // the wave's sum: sixteen-lane sums, then the four rows' totals
    trace = sum16(trace);
    const float tw = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(trace), 0)) +
                     __int_as_float(__builtin_amdgcn_readlane(__float_as_int(trace), 16)) +
                     __int_as_float(__builtin_amdgcn_readlane(__float_as_int(trace), 32)) +
                     __int_as_float(__builtin_amdgcn_readlane(__float_as_int(trace), 48));
    if (l == 0) sm.trp[w] = tw;
  }
  {
    // Gram (waves 0-3) and Q X^T (waves 4-7); M = tril(Q X^T) o D.  The gates,
    // T, W and U come from the maps kernel.
    typename InputGram<IO>::type f;
    f.load(w < 4 ? &cc.X[0][0] : &cc.Q[0][0], kPW, &cc.X[0][0], kPW, w & 3, l);
    f.run();
    if (w < 4) {
      f.store(w & 3, l, [&](int r, int s2, float v) { cc.KX[r][s2] = v; });
    } else {
      f.store(w & 3, l, [&](int r, int s2, float v) {
        sm.QX[r][s2] = v;
        cc.MM[r][s2] = s2 <= r ? dexp(cc.g[r], cc.g[s2]) * v : 0.f;
      });
    }
  }
  __syncthreads();
  const float eG = eexp(cc.G);
  auto xs = [&](int i) { return dexp(cc.G, cc.g[i]); };
  {
    // Xh Lam (into DW), dU = Xh Lam + M^T dO, R = U - W S_c, dQt = dO S_c^T
    Mm<kBC, kD, kD, false, false, kWaves3> fxl, fws;
    Mm<kBC, kD, kD, false, true, kWaves3> fdq;
    Mm<kBC, kD, kBC, true, false, kWaves3> fmo;
    fxl.load(&cc.X[0][0], kPW, &sm.LL[0][0], kPW, w, l, xs);
    fws.load(&cc.W[0][0], kPW, &sm.SC[0][0], kPW, w, l);
    fdq.load(&sm.DO[0][0], kPW, &sm.SC[0][0], kPW, w, l);
    fmo.load(&cc.MM[0][0], kPN, &sm.DO[0][0], kPW, w, l);
    fxl.run();
    fws.run();
    fdq.run();
    fmo.run(fxl);
    fxl.store(w, l, [&](int r, int s, float v) { sm.DW[r][s] = v; });
    fmo.store(w, l, [&](int r, int s, float v) { sm.DU[r][s] = v; });
    fws.store(w, l, [&](int r, int s, float v) { sm.RR[r][s] = cc.U[r][s] - v; });
    fdq.store(w, l, [&](int r, int s, float v) { sm.DQT[r][s] = v; });
  }
  __syncthreads();
  {
    // dW = -(Xh Lam) S_c^T - M^T dQt, dXh = R Lam^T, dM = dO U^T - dQt W^T
    // (-dQt W^T on waves 0-3, dO U^T on waves 4-7)
    Mm<kBC, kD, kD, false, true, kWaves3> fxs, fxh;
    Mm<kBC, kD, kBC, true, false, kWaves3> fmq;
    Mm<kBC, kBC, kD, false, true> fmx;
    fxs.load(&sm.DW[0][0], kPW, &sm.SC[0][0], kPW, w, l);
    fmq.load(&cc.MM[0][0], kPN, &sm.DQT[0][0], kPW, w, l);
    fxh.load(&sm.RR[0][0], kPW, &sm.LL[0][0], kPW, w, l);
    fmx.load(w < 4 ? &sm.DQT[0][0] : &sm.DO[0][0], kPW, w < 4 ? &cc.W[0][0] : &cc.U[0][0], kPW, w & 3, l);
    __syncthreads();   // every wave has read Xh Lam from DW
    fxs.run();
    fmq.run(fxs);
    fxh.run();
    fmx.run();
    fmq.store(w, l, [&](int r, int s, float v) { sm.DW[r][s] = -v; });
    fxh.store(w, l, [&](int r, int s, float v) { sm.DXH[r][s] = v; });
    if (w < 4) fmx.store(w & 3, l, [&](int r, int s, float v) { sm.DM[r][s] = -v; });
    __syncthreads();
    // dM o D, D_{is} = e^{g_i-g_s} for s <= i
    if (w >= 4)
      fmx.store(w & 3, l, [&](int r, int s, float v) {
        sm.DM[r][s] = s <= r ? (sm.DM[r][s] + v) * dexp(cc.g[r], cc.g[s]) : 0.f;
      });
  }
  __syncthreads();
  {
    // decay terms of M, Qt and Xh (sixteen lanes per row).  The gradient of
    // the log decay of row i takes, from each decayed product, only the terms
    // whose decay spans row i, each of which carries gamma_i: from Qt rows
    // r >= i, from Xh rows r < i, from M (and later A) the pairs s < i <= r.
    // Summed that way it keeps float accuracy relative to gamma_i, which the
    // division by gamma_i in the gate step needs; totals of a row minus a
    // column would cancel O(1) terms.  For M the pair term is
    // dM o M = (dM o D) o (Q X^T); each row r turns its strictly lower part
    // into exclusive prefixes along the row, stored transposed in PT (the
    // chunk kernel leaves A's array unused), so that row i of PT summed over
    // columns r >= i is the M share of row i.
    float (*PT)[kPN] = cc.AA;
    const int i = ri, s0 = 2 * rp;
    float qd = 0.f, xd = 0.f;
    {
      const float4 q4 = *reinterpret_cast<const float4*>(&cc.Q[i][4 * rp]);
      const float4 t4 = *reinterpret_cast<const float4*>(&sm.DQT[i][4 * rp]);
      const float4 x4 = *reinterpret_cast<const float4*>(&cc.X[i][4 * rp]);
      const float4 h4 = *reinterpret_cast<const float4*>(&sm.DXH[i][4 * rp]);
      qd = q4.x * t4.x + q4.y * t4.y + q4.z * t4.z + q4.w * t4.w;
      xd = x4.x * h4.x + x4.y * h4.y + x4.z * h4.z + x4.w * h4.w;
    }
    const float w0 = s0 < i ? sm.DM[i][s0] * sm.QX[i][s0] : 0.f;
    const float w1 = s0 + 1 < i ? sm.DM[i][s0 + 1] * sm.QX[i][s0 + 1] : 0.f;
    const float ex = excl16(w0 + w1);
    PT[s0][i] = ex;
    PT[s0 + 1][i] = ex + w0;
    qd = sum16(qd); xd = sum16(xd);
    if (rp == 0) {
      sm.dg[i] = eexp(cc.g[i]) * qd;
      sm.dgt[i] = xs(i) * xd;
    }
  }
  // dQ = Diag(e^g) dQt + (dM o D) X;  dX = Diag(e^{G-g}) dXh + (dM o D)^T Q
  float* dq_out = a.dphi_q + bh * T * kD;
  {
    Mm<kBC, kD, kBC, false, false, kWaves3> fq;
    Mm<kBC, kD, kBC, true, false, kWaves3> fx;
    fq.load(&sm.DM[0][0], kPN, &cc.X[0][0], kPW, w, l);
    fx.load(&sm.DM[0][0], kPN, &cc.Q[0][0], kPW, w, l);
    fq.run();
    fx.run();
    fq.store(w, l, [&](int r, int s2, float v) {
      if (t0 + r < T) dq_out[int64_t(t0 + r) * kD + s2] = eexp(cc.g[r]) * sm.DQT[r][s2] + v;
    });
    fx.store(w, l, [&](int r, int s2, float v) { sm.RR[r][s2] = xs(r) * sm.DXH[r][s2] + v; });
  }
  __syncthreads();
  // dY = T^T dW (into DQT), dZ = T^T dU (into DO)
  float (*DY)[kPW] = sm.DQT;
  float (*DZ)[kPW] = sm.DO;
  {
    Mm<kBC, kD, kBC, true, false, kWaves3> fy, fz;
    fy.load(&cc.TT[0][0], kPN, &sm.DW[0][0], kPW, w, l);
    fz.load(&cc.TT[0][0], kPN, &sm.DU[0][0], kPW, w, l);
    fy.run();
    fz.run();
    fy.store(w, l, [&](int r, int s2, float v) { DY[r][s2] = v; });
    fz.store(w, l, [&](int r, int s2, float v) { DZ[r][s2] = v; });
  }
  __syncthreads();
  float* dv_out = a.dv + bh * T * kD;
  {
    // dA = -dY W^T - dZ U^T (strictly lower part used; dY W^T on waves 0-3,
    // dZ U^T on waves 4-7)
    Mm<kBC, kBC, kD, false, true> fa;
    fa.load(w < 4 ? &DY[0][0] : &DZ[0][0], kPW, w < 4 ? &cc.W[0][0] : &cc.U[0][0], kPW, w & 3, l);
    fa.run();
    // Y = Diag(eta e^{gp}) X, Z = Diag(eta) V: dX += Diag(eta e^{gp}) dY,
    // dV = Diag(eta) dZ, and the eta / gp terms
    {
      const int i = ri, f = 4 * rp;
      const float egp = eexp(cc.gp[i]), eta = cc.eta[i];
      const float4 dy = *reinterpret_cast<const float4*>(&DY[i][f]);
      const float4 dz = *reinterpret_cast<const float4*>(&DZ[i][f]);
      const float4 x = *reinterpret_cast<const float4*>(&cc.X[i][f]);
      const float4 v = *reinterpret_cast<const float4*>(&cc.V[i][f]);
      float4 dx = *reinterpret_cast<const float4*>(&sm.RR[i][f]);
      float xy = x.x * dy.x + x.y * dy.y + x.z * dy.z + x.w * dy.w;
      float vz = v.x * dz.x + v.y * dz.y + v.z * dz.z + v.w * dz.w;
      const float sy = eta * egp;
      dx.x = fmaf(sy, dy.x, dx.x); dx.y = fmaf(sy, dy.y, dx.y);
      dx.z = fmaf(sy, dy.z, dx.z); dx.w = fmaf(sy, dy.w, dx.w);
      *reinterpret_cast<float4*>(&sm.RR[i][f]) = dx;
      if (t0 + i < T)
        *reinterpret_cast<float4*>(dv_out + int64_t(t0 + i) * kD + f) =
            make_float4(eta * dz.x, eta * dz.y, eta * dz.z, eta * dz.w);
      xy = sum16(xy); vz = sum16(vz);
      if (rp == 0) {
        sm.deta[i] = egp * xy + vz;
        sm.dgp[i] = eta * egp * xy;
      }
    }
    if (w < 4) fa.store(w & 3, l, [&](int r, int s2, float v) { sm.DM[r][s2] = -v; });
    __syncthreads();
    // A_{is} = eta_i e^{gp_i-g_s} k_{is}: D2 = dA o e^{gp_i-g_s} (s < i)
    if (w >= 4)
      fa.store(w & 3, l, [&](int r, int s2, float v) {
        sm.DM[r][s2] = s2 < r ? (sm.DM[r][s2] - v) * dexp(cc.gp[r], cc.g[s2]) : 0.f;
      });
  }
  __syncthreads();
  {
    // eta_i's share of A, and A's pair terms eta_i D2 o K for s < i' < i,
    // added as exclusive row prefixes into PT (entries s < i)
    float (*PT)[kPN] = cc.AA;
    const int i = ri, s0 = 2 * rp;
    const float eta = cc.eta[i];
    float row = 0.f, wa[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int s2 = s0 + k;
      const float p = sm.DM[i][s2] * cc.KX[i][s2];
      row += p;
      wa[k] = s2 < i ? eta * p : 0.f;
    }
    const float ex = excl16(wa[0] + wa[1]);
    if (s0 < i) PT[s0][i] += ex;
    if (s0 + 1 < i) PT[s0 + 1][i] += ex + wa[0];
    row = sum16(row);
    if (rp == 0) sm.deta[i] += row;
  }
  {
    // dK = Diag(eta) D2 (strictly lower): dX += dK X + dK^T X = Diag(eta) D2 X + D2^T Diag(eta) X
    auto eta_of = [&](int i) { return cc.eta[i]; };
    Mm<kBC, kD, kBC, false, false, kWaves3> f1;
    Mm<kBC, kD, kBC, true, false, kWaves3> f2;
    f1.load(&sm.DM[0][0], kPN, &cc.X[0][0], kPW, w, l, eta_of);
    f2.load(&sm.DM[0][0], kPN, &cc.X[0][0], kPW, w, l, [](int) { return 1.f; }, eta_of);
    f1.run();
    f2.run(f1);
    f2.store(w, l, [&](int r, int s2, float v) { sm.RR[r][s2] += v; });
  }
  __syncthreads();
  // gates: g -> log decay -> (eta, lam); eta -> (beta, lam, ||x||^2).  One
  // wave; every operand is loaded first and the sums run on DPP lane moves,
  // since the other seven waves wait for this step.
  if (w == 0) {
    const int i = l, ic = l & 31;
    // the pair terms of M and A spanning row c: row c of PT over the columns
    // r >= c, lanes c and c + 32 taking columns 0-15 and 16-31
    const int c = ic, r0 = (l >> 5) * 16;
    const float4* pt = reinterpret_cast<const float4*>(&cc.AA[c][r0]);
    float4 pv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) pv[k] = pt[k];
    const float dgi = sm.dg[ic], dgpn = ic + 1 < kBC ? sm.dgp[ic + 1] : 0.f, zi = sm.dgt[ic];
    float tr = 0.f;
#pragma unroll
    for (int r = 0; r < kWaves3; ++r) tr += sm.trp[r];
    const int fl = cc.flags[ic];
    const float eta = cc.eta[ic], lamv = cc.lamv[ic], den = cc.den[ic], detai = sm.deta[ic];
    float pairs = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int r = r0 + 4 * k;
      pairs += (r >= c ? pv[k].x : 0.f) + (r + 1 >= c ? pv[k].y : 0.f) + (r + 2 >= c ? pv[k].z : 0.f) +
               (r + 3 >= c ? pv[k].w : 0.f);
    }
    pairs += __shfl_xor(pairs, 32);   // lanes l and l ^ 32 hold the two halves
    // dlg_i: the Qt, Y and state terms of rows r >= i (suffix sums), the Xh
    // terms of rows r < i (exclusive prefix sums) and the pair terms; the
    // scans run within 16-lane rows, then row 0 takes row 1's total (suffix)
    // and row 1 takes row 0's (prefix)
    float dlg = dgi + dgpn + (ic == kBC - 1 ? eG * tr : 0.f);
    dlg += row_shl<1>(dlg);
    dlg += row_shl<2>(dlg);
    dlg += row_shl<4>(dlg);
    dlg += row_shl<8>(dlg);
    float z = zi;
    z += row_shr<1>(z);
    z += row_shr<2>(z);
    z += row_shr<4>(z);
    z += row_shr<8>(z);
    const float up = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(dlg), 16));
    const float lo = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(z), 15));
    dlg += ic < 16 ? up : 0.f;
    z += ic >= 16 ? lo : 0.f;
    // exclusive: the lane below's inclusive prefix (0 at each row start, where
    // lane 16 adds row 0's total).  The lane move runs in every lane, outside
    // any select: a DPP read from a lane switched off by a branch yields 0.
    const float zb = row_shr<1>(z) + (ic == 16 ? lo : 0.f);
    dlg += zb + pairs;
    if (i < kBC) {
      // decay path where the clamp does not bind (alpha = eta lam, gamma = 1 - alpha)
      const bool decay = (fl & 4) && !(fl & 2);
      const float dalpha = decay ? -dlg * __builtin_amdgcn_rcpf(decay ? cc.gam[ic] : 1.0f) : 0.f;
      const float deta = detai + dalpha * lamv;
      // step size eta = beta / den where it comes from the formula
      const bool onr = fl & 1;
      const float rden = __builtin_amdgcn_rcpf(onr ? den : 1.0f);
      const float dbeta = onr ? deta * rden : 0.f;
      const float dE = onr ? -deta * eta * rden : 0.f;
      const float dlam = dalpha * eta + dE;
      const int t = t0 + i;
      if (t < T) {
        a.dbeta[bh * T + t] = dbeta;
        a.dlam[bh * T + t] = dlam;
      }
      sm.dgp[i] = dE;     // reused: d||x_i||^2
    }
  }
  __syncthreads();
  // x_t = phi(k_{t-1}): row i of dX is the gradient of key t0 + i - 1
  float* dk_out = a.dphi_k + bh * T * kD;
  const bool fresh = (a.k_prev == nullptr);
  {
    const int i = ri, f0 = 4 * rp, t = t0 + i;
    const float dE2 = 2.0f * sm.dgp[i];
    const float4 x = *reinterpret_cast<const float4*>(&cc.X[i][f0]);
    const float4 d = *reinterpret_cast<const float4*>(&sm.RR[i][f0]);
    const float4 o = make_float4(fmaf(dE2, x.x, d.x), fmaf(dE2, x.y, d.y), fmaf(dE2, x.z, d.z), fmaf(dE2, x.w, d.w));
    float* dst = nullptr;
    if (t >= 1 && t < T) dst = dk_out + int64_t(t - 1) * kD + f0;
    else if (t == 0 && !fresh && a.dk_prev) dst = a.dk_prev + bh * kD + f0;
    if (dst) *reinterpret_cast<float4*>(dst) = o;
  }
  // the last key feeds no token of this call
  if (c == a.nchunks - 1)
    for (int f = tid; f < kD; f += kThreads3) dk_out[int64_t(T - 1) * kD + f] = 0.f;
  __syncthreads();   // LDS is refilled for the next chunk
  }
}

}  // namespace

size_t bwd_workspace_bytes(const ProblemArgs& p) {
  const int64_t nchunks = (int64_t(p.T) + kBC - 1) / kBC;
  const int64_t n = int64_t(p.B) * p.H * nchunks;
  return size_t(n) * (kMapFloats + 2 * kD * kD + kFacFloats) * sizeof(float);
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
  a.fac = a.adj + n * kD * kD;
  a.T = p.T; a.nchunks = nchunks; a.eps = p.eps; a.eps_gamma = p.eps_gamma;
  const int nunits = int(2 * BH);
  const unsigned chain_blocks = unsigned((nunits + 7) / 8) * 32u;
  // one chunk-kernel workgroup per CU (its LDS allows no more)
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu <= 0)
    ncu = 256;
  const int jobs = int(n);
  const unsigned chunk_blocks = unsigned(jobs < ncu ? jobs : ncu);
  // two maps workgroups per CU (LDS)
  const unsigned map_blocks = unsigned(jobs < 2 * ncu ? jobs : 2 * ncu);
  if (p.bf16) {
    hipLaunchKernelGGL(falcon1_bwd_maps_kernel<bf16_t>, dim3(map_blocks), dim3(kThreads), 0, st, a, jobs);
    hipLaunchKernelGGL(falcon1_bwd_chain_kernel<bf16_t>, dim3(chain_blocks), dim3(kThreads), 0, st, a, nunits);
    hipLaunchKernelGGL(falcon1_bwd_chunk_kernel<bf16_t>, dim3(chunk_blocks), dim3(kThreads3), 0, st, a, jobs);
  } else {
    hipLaunchKernelGGL(falcon1_bwd_maps_kernel<float>, dim3(map_blocks), dim3(kThreads), 0, st, a, jobs);
    hipLaunchKernelGGL(falcon1_bwd_chain_kernel<float>, dim3(chain_blocks), dim3(kThreads), 0, st, a, nunits);
    hipLaunchKernelGGL(falcon1_bwd_chunk_kernel<float>, dim3(chunk_blocks), dim3(kThreads3), 0, st, a, jobs);
  }
  return hipGetLastError();
}

}  // namespace falcon
