// Fused chunk-parallel Falcon-1 forward on MFMA (gfx950), bf16 I/O,
// dk = dv = 64, chunk C = 64.
//
// One workgroup owns one (batch, head) sequence for its whole length.  Its
// six waves split into two roles that run concurrently:
//
//  * two CHAIN waves; wave w owns value columns 32w..32w+31 of the float32
//    state S (kept in MFMA result registers for the whole sequence):
//      a3  R = U - W S (rows eta_i r_i), S <- e^{g_63} S + (Diag(e^{g_63-g}) X)^T R;
//      a4  O = Diag(e^g) Q S + M R, stored as bf16;
//    they also stream the sequence's keys, queries and gates from HBM into
//    an LDS ring two chunks ahead (direct global-to-LDS loads, 1 KiB per
//    instruction, fully coalesced).
//  * a FACTOR GROUP of four waves that builds the state-independent factors
//    of the next chunk while the chain works on the current one:
//      a1  x_i = phi(k_{t0+i-1}), E_i = ||x_i||^2, eta_i (Eq. 3.4 with the
//          fresh-start sentinel), log gamma_i = log1p(-min(eta_i lam_i,
//          1 - eps_gamma)) (Section 4.3) and the chunk-local prefix g_i (the
//          log-space renormalisation of Section 4.4 applied per chunk);
//      a2  the decayed strictly-lower Gram matrix
//          A_{i,s} = eta_i e^{g_{i-1}-g_s} (x_i . x_s), T = (I + A)^{-1}
//          (16x16 diagonal blocks by column elimination in registers with
//          DPP broadcasts, off-diagonal blocks by MFMA block products),
//          W = T Diag(eta e^{g_{s-1}}) X and U = T Diag(eta) V ("one
//          multi-RHS TriSolve per chunk" of the WY form), the decayed read
//          mask M_{i,s} = e^{g_i-g_s} (q_i . x_s) for s <= i (read after
//          write) and the decayed keys (Diag(e^{g_63-g}) X)^T.
//    Wave f0 carries the inverse (the critical path); f1..f3 share the mask,
//    the key/value transposes and the W and U products.
//
// Hand-over is through LDS: a 3-entry input ring, 2 factor slots and a pair
// of T buffers, each guarded by counters with workgroup-scope
// release/acquire.  Every wait is bounded (spin limit + abort flag), so no
// schedule can hang.  Every input byte is read from HBM once (values by the
// U waves, the rest by the chain's ring loads) and every output byte is
// written once.
//
// MFMA operand convention.  v_mfma_f32_16x16x32_bf16 takes, in lane l, row
// (l & 15) of A and column (l & 15) of B with eight k-values each; the
// result holds column (l & 15), rows 4 (l >> 4) .. +3.  Products whose two
// operands are rows of the inputs give lane group g = l >> 4 the eight
// contiguous k-values 8g..8g+7 of a 32-wide block (one 16-byte read).
// Products that consume results feed lane group g the k-values
// {4g..4g+3, 16+4g..16+4g+3}: then two stacked result tiles are exactly
// the next operand fragment, which keeps S and R in registers, and a
// product with a selection matrix turns token-major rows into the
// feature-major fragments that contract over tokens.  Either way A and B
// use the same order, so every sum is unchanged.

#include "falcon_device.h"
#include "falcon_launch.h"
#include "falcon_mfma_frag.h"

namespace falcon {

namespace {

using namespace frag;


constexpr int kC = 64;            // chunk length
constexpr int kD = 64;            // dk = dv
constexpr int kP = 72;            // bf16 row pitch of T in LDS (elements)
constexpr int kNI = 3;            // input ring entries
constexpr int kNS = 2;            // factor slots
constexpr int kChain = 2;         // chain waves
constexpr int kFactor = 4;        // factor waves
constexpr int kThreads = 64 * (kChain + kFactor);
constexpr int kSlotWriters = 3;    // factor waves f1..f3 fill a slot
constexpr int kSpinLimit = 1 << 22;

// Gates of one chunk (a1), in the orders their readers want them.  "_t"
// arrays hold row i = 16 ib + c16 at [c16 * 4 + ib], so that one 16-byte read
// gives a lane the values of its column c16 in all four row blocks.
struct ChunkGates {
  float graw[kC];                 // g_s, token order
  float sxg[kC];                  // eta_s e^{g_{s-1}}
  float sxh[kC];                  // e^{g_63 - g_s}
  float eta[kC];                  // eta_s
  float eta_t[kC];                // eta_i
  float gprev_t[kC];              // g_{i-1}
  float graw_t[kC];               // g_i
  float gexp_t[kC];               // e^{g_i}
  float glast[4];                 // e^{g_63}
};

// One chunk of input as staged from HBM: 64 rows of 128 bytes, the 16-byte
// segment q of row r stored at position q ^ ((r >> 1) & 7) (conflict-free
// reads of 16 consecutive rows), and the chunk's gates.
struct InputEntry {
  uint16_t x[kC * kD];            // keys phi(k_{t0+r-1})
  uint16_t q[kC * kD];            // queries phi(q_{t0+r})
  ChunkGates gt;
};

// Factors of one chunk, as consumed by the chain waves.
struct Slot {
  uint16_t wf[4 * 2 * 64 * 8];    // -W, A fragments [ib][m][lane][8]
  uint16_t mf[4 * 2 * 64 * 8];    // M^T, B fragments [ib][m][lane][8]
  uint16_t xh[4 * 2 * 64 * 8];    // (Diag(e^{g_63-g}) X)^T, A fragments [fb][m][lane][8]
  uint16_t uf[4 * 4 * 64 * 4];    // U result tiles [ib][cb][lane][4], bf16
};

struct Smem {
  InputEntry in[kNI];
  Slot slot[kNS];
  uint16_t tb[2][kC * kP];        // T = (I + A)^{-1}, row-major, by chunk parity
  float abt[4][16][16];           // diagonal blocks of -A: [b][s][i] = -A[16b+i][16b+s]
  int in_ready[kNI];              // +1 when an entry's loads (issued by wave f1) have landed
  int in_free[kNI];               // +1 per chain wave when done with an entry
  int slot_full[kNS];             // +1 per factor wave f1..f3 when its part is written
  int slot_free[kNS];             // +1 per chain wave when it has read a slot
  int t_ready[2];                 // chunk + 1 whose T is complete in tb[parity]
  int t_used[2];                  // +1 per factor wave 1..3 done reading tb[parity]
  int abort_flag;
};

// Column elimination for a unit lower-triangular 16x16 block: lane j holds
// column j of the negated strictly-lower part (ncol[i] = -A[i][j]) and of
// the inverse (t[i]).  Step S adds -A[i][S] t[S] to every row i > S, the
// factor broadcast from lane S of the 16-lane row by the multiply-add's own
// DPP source modifier (row_newbcast).  Each statement starts with two wait
// states, which covers the DPP read-after-VALU-write hazard on its sources.
#define FALCON_FMAC(D, A, S) "v_fmac_f32_dpp %" #D ", %" #A ", %" #S
#define FALCON_BCAST(N) " row_newbcast:" #N " row_mask:0xf bank_mask:0xf\n\t"
#define ELIM4(S, I)                                                                     \
  asm volatile("s_nop 1\n\t" FALCON_FMAC(0, 4, 8) FALCON_BCAST(S) FALCON_FMAC(1, 5, 8)   \
               FALCON_BCAST(S) FALCON_FMAC(2, 6, 8) FALCON_BCAST(S) FALCON_FMAC(3, 7, 8)   \
               FALCON_BCAST(S)                                                          \
               : "+v"(t[I]), "+v"(t[I + 1]), "+v"(t[I + 2]), "+v"(t[I + 3])              \
               : "v"(ncol[I]), "v"(ncol[I + 1]), "v"(ncol[I + 2]), "v"(ncol[I + 3]), "v"(t[S]))
#define ELIM3(S, I)                                                                     \
  asm volatile("s_nop 1\n\t" FALCON_FMAC(0, 3, 6) FALCON_BCAST(S) FALCON_FMAC(1, 4, 6)   \
               FALCON_BCAST(S) FALCON_FMAC(2, 5, 6) FALCON_BCAST(S)                      \
               : "+v"(t[I]), "+v"(t[I + 1]), "+v"(t[I + 2])                              \
               : "v"(ncol[I]), "v"(ncol[I + 1]), "v"(ncol[I + 2]), "v"(t[S]))
#define ELIM2(S, I)                                                                     \
  asm volatile("s_nop 1\n\t" FALCON_FMAC(0, 2, 4) FALCON_BCAST(S) FALCON_FMAC(1, 3, 4)   \
               FALCON_BCAST(S)                                                          \
               : "+v"(t[I]), "+v"(t[I + 1])                                             \
               : "v"(ncol[I]), "v"(ncol[I + 1]), "v"(t[S]))
#define ELIM1(S, I)                                                                     \
  asm volatile("s_nop 1\n\t" FALCON_FMAC(0, 1, 2) FALCON_BCAST(S)                        \
               : "+v"(t[I]) : "v"(ncol[I]), "v"(t[S]))

__device__ __forceinline__ void eliminate16(float (&t)[16], const float (&ncol)[16]) {
  ELIM4(0, 1); ELIM4(0, 5); ELIM4(0, 9); ELIM3(0, 13);
  ELIM4(1, 2); ELIM4(1, 6); ELIM4(1, 10); ELIM2(1, 14);
  ELIM4(2, 3); ELIM4(2, 7); ELIM4(2, 11); ELIM1(2, 15);
  ELIM4(3, 4); ELIM4(3, 8); ELIM4(3, 12);
  ELIM4(4, 5); ELIM4(4, 9); ELIM3(4, 13);
  ELIM4(5, 6); ELIM4(5, 10); ELIM2(5, 14);
  ELIM4(6, 7); ELIM4(6, 11); ELIM1(6, 15);
  ELIM4(7, 8); ELIM4(7, 12);
  ELIM4(8, 9); ELIM3(8, 13);
  ELIM4(9, 10); ELIM2(9, 14);
  ELIM4(10, 11); ELIM1(10, 15);
  ELIM4(11, 12);
  ELIM3(12, 13);
  ELIM2(13, 14);
  ELIM1(14, 15);
}
#undef ELIM4
#undef ELIM3
#undef ELIM2
#undef ELIM1
#undef FALCON_BCAST
#undef FALCON_FMAC

__device__ __forceinline__ bool wait_at_least(int* flag, int target, int* abort_flag) {
  for (int it = 0; it < kSpinLimit; ++it) {
    const int v = __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (__builtin_amdgcn_readfirstlane(v) >= target) {
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
__device__ __forceinline__ bool aborted(int* abort_flag) {
  return __hip_atomic_load(abort_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) != 0;
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
// Ring staging (wave f1): the keys, queries and gates of chunk c are fetched
// into registers with fully coalesced 16-byte loads (one instruction covers
// eight whole rows), and written to the swizzled ring entry later, once the
// loads have had a chunk's worth of work to land.  Rows past the sequence are
// fetched from a valid row (their step size is 0, so their finite values
// never reach a result); so is the fresh-start key row -1 (eta_1 = 0).
// ---------------------------------------------------------------------------
struct RingRegs {
  bf16x8 x[8];
  bf16x8 q[8];
  float beta, lam;
};

__device__ __forceinline__ void ring_fetch(RingRegs& R, const Seq& sq, int c, int l) {
  const int t0 = c * kC;
  const int T = sq.T;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = 8 * j + (l >> 3);
    const int kt = t0 + r - 1;
    const bf16_t* xs = kt < 0 ? (sq.k_prev ? sq.k_prev : sq.K) : sq.K + int64_t(kt < T ? kt : T - 1) * kD;
    const int tok = t0 + r < T ? t0 + r : T - 1;
    R.x[j] = *reinterpret_cast<const bf16x8*>(xs + 8 * (l & 7));
    R.q[j] = *reinterpret_cast<const bf16x8*>(sq.Q + int64_t(tok) * kD + 8 * (l & 7));
  }
  const int tok = t0 + l < T ? t0 + l : T - 1;
  R.beta = sq.beta[tok];
  R.lam = sq.lam[tok];
}

// Writes the staged rows of chunk c into entry E and derives the chunk's
// gates (a1) from the staged registers: x_i = phi(k_{t0+i-1}), E_i = ||x_i||^2,
// eta_i (Eq. 3.4, 0 at a fresh start and past the sequence), the clamped log
// decay of Section 4.3 and its chunk-local inclusive prefix g_i (the
// log-space renormalisation of Section 4.4 applied per chunk).
__device__ __forceinline__ void ring_store(InputEntry& E, const RingRegs& R, const Seq& sq, int c, int l,
                                           float eps, float eps_gamma, bool fresh) {
  const int g = l >> 4, c16 = l & 15;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = 8 * j + (l >> 3);
    const int off = r * kD + 8 * seg_pos(r, l & 7);
    *reinterpret_cast<bf16x8*>(E.x + off) = R.x[j];
    *reinterpret_cast<bf16x8*>(E.q + off) = R.q[j];
  }
  float eta, gi, gprev, glast;
  chunk_gates(R.x, R.beta, R.lam, c * kC + l, sq.T, eps, eps_gamma, fresh, l, eta, gi, gprev, glast);
  ChunkGates& G = E.gt;
  G.graw[l] = gi;
  G.sxg[l] = eta * __expf(gprev);
  G.sxh[l] = __expf(glast - gi);
  G.eta[l] = eta;
  G.eta_t[c16 * 4 + g] = eta;
  G.gprev_t[c16 * 4 + g] = gprev;
  G.graw_t[c16 * 4 + g] = gi;
  G.gexp_t[c16 * 4 + g] = __expf(gi);
  if (l == 0) G.glast[0] = __expf(glast);
}

// ---------------------------------------------------------------------------
// Factor group: wave fw of the four builds its share of the slot of chunk c.
// ---------------------------------------------------------------------------
struct ValueFrags {
  bf16x8 v[4];      // V rows of the four row blocks, k block 32*vk .. +31 (contiguous order)
};

__device__ __forceinline__ void load_values(ValueFrags& L, const Seq& sq, int c, int vk, int l) {
  const int g = l >> 4, c16 = l & 15;
#pragma unroll
  for (int sb = 0; sb < 4; ++sb) {
    int tok = c * kC + 16 * sb + c16;
    tok = tok < sq.T ? tok : sq.T - 1;
    L.v[sb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(sq.V + int64_t(tok) * kD + 32 * vk + 8 * g));
  }
}

// kRole: 0 for wave f0, 1 for f1, 2 for f2 and f3 (fw tells them apart).
template <int kRole>
__device__ bool factor_chunk(Smem& sm, ValueFrags& VF, const Seq& sq, int c, int fw, int l,
                             float eps, float eps_gamma, bool fresh, int nchunks) {
  const int g = l >> 4, c16 = l & 15;
  const int t0 = c * kC;
  const InputEntry& E = sm.in[c % kNI];
  Slot& S = sm.slot[c % kNS];
  uint16_t* tb = sm.tb[c & 1];
  const ChunkGates& G = E.gt;
  if (!wait_at_least(&sm.in_ready[c % kNI], c / kNI + 1, &sm.abort_flag)) return false;

  // key fragments: rows 16 ib + c16, k block m (contiguous order); wave f0
  // needs both k blocks, f1 the first (key blocks 0-1), f2 and f3 the second
  constexpr int m_lo = kRole == 2 ? 1 : 0;
  constexpr int m_hi = kRole == 1 ? 1 : 2;
  bf16x8 xf[4][2];
#pragma unroll
  for (int ib = 0; ib < 4; ++ib)
#pragma unroll
    for (int m = m_lo; m < m_hi; ++m) xf[ib][m] = ring_frag_c(E.x, 16 * ib + c16, m, g);

  if constexpr (kRole == 0) {
    // ---- decayed Gram: A^T tile (sb, ib) = X_sb X_ib^T, scaled ------------
    const f32x4 eta_i = ld4(&G.eta_t[c16 * 4]);
    const f32x4 gpv_i = ld4(&G.gprev_t[c16 * 4]);
    f32x4 gs_s[4];                                           // g_s for s = 16 sb + 4 g + r
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) gs_s[sb] = ld4(&G.graw[16 * sb + 4 * g]);
    s16x4 a10, a32;      // A blocks (1,0) and (3,2) as K=16 A fragments
    bf16x8 a2lo, a3lo;   // A rows 32-47 / 48-63, columns 0-31, as K=32 A fragments
    {
      f32x4 a_off[6];
#pragma unroll
      for (int n = 0; n < 10; ++n) {
        int ib, sb;
        lower_tile(n, ib, sb);
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
    // ---- T = (I + A)^{-1}: diagonal blocks by column elimination ----------
    float t[16];
    {
      float ncol[16];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 v = ld4(&sm.abt[g][c16][4 * q4]);        // -A[16g+i][16g+c16], all i
        ncol[4 * q4] = v[0]; ncol[4 * q4 + 1] = v[1]; ncol[4 * q4 + 2] = v[2]; ncol[4 * q4 + 3] = v[3];
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) t[i] = (i == c16) ? 1.0f : 0.0f;
      eliminate16(t, ncol);
    }
    // tb[c & 1] held T of chunk c - 2: wait until f1..f3 are done with it.
    if (!wait_at_least(&sm.t_used[c & 1], 3 * (c / 2), &sm.abort_flag)) return false;
#pragma unroll
    for (int i = 0; i < 16; ++i) tb[(16 * g + i) * kP + 16 * g + c16] = bf(t[i]);
    // ---- off-diagonal 16x16 blocks: T_hl = -T_hh A_hl T_ll for (1,0), (3,2)
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
    // ---- lower-left 32x32 block: T_21 = -T_22 A_21 T_11 (2x2 block sense) --
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
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    if (l == 0) __hip_atomic_store(&sm.t_ready[c & 1], c + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    return true;
  }

  // ---- waves f1..f3 ---------------------------------------------------------
  // Work split: f1: staging of chunk c + 1, key transposes fb 0..1, W fb 0..1;
  // f2: key transposes fb 2, values cb 0..1, mask tiles 0..4, W fb 2;
  // f3: key transposes fb 3, values cb 2..3, mask tiles 5..9, W fb 3.
  const int fb0 = kRole == 1 ? 0 : fw;                          // first key block: 0, 2, 3
  constexpr int nfb = kRole == 1 ? 2 : 1;
  if (!wait_at_least(&sm.slot_free[c % kNS], 2 * (c / kNS), &sm.abort_flag)) return false;
  // wave f1 streams the ring entry of chunk c + 1 (it held chunk c - 2)
  const bool load_next = kRole == 1 && c + 1 < nchunks;
  RingRegs rr;
  if (load_next) ring_fetch(rr, sq, c + 1, l);

  // ---- decayed key transposes on the matrix cores --------------------------
  // D(sb, fb) = X_sb I_fb; lane holds X[16sb+4g+r][16fb+c16].
  bf16x8 xg[2][2];                                           // (Diag(eta e^{g_{s-1}}) X)^T
  {
    f32x4 sxg_s[4], sxh_s[4];
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) {
      sxg_s[sb] = ld4(&G.sxg[16 * sb + 4 * g]);
      sxh_s[sb] = ld4(&G.sxh[16 * sb + 4 * g]);
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      if (k < nfb) {
        const int fb = fb0 + k;
        constexpr int mk = kRole == 1 ? 0 : 1;                // fb >> 1, known per role
        const bf16x8 sel = select_frag(fb & 1, g, c16);
        f32x4 d[4];
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) d[sb] = mfma32(xf[sb][mk], sel, zero4());
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          xg[k][m] = frag_acc(d[2 * m] * sxg_s[2 * m], d[2 * m + 1] * sxg_s[2 * m + 1]);
          store_frag(&S.xh[((fb * 2 + m) * 64 + l) * 8],
                     frag_acc(d[2 * m] * sxh_s[2 * m], d[2 * m + 1] * sxh_s[2 * m + 1]));
        }
      }
    }
  }
  // ---- value transposes (waves f2, f3): Diag(eta) V for two column blocks --
  bf16x8 vt[2][2];                                           // [cb][m]
  if constexpr (kRole == 2) {
    f32x4 eta_s[4];
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) eta_s[sb] = ld4(&G.eta[16 * sb + 4 * g]);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const bf16x8 sel = select_frag(k, g, c16);
      f32x4 d[4];
#pragma unroll
      for (int sb = 0; sb < 4; ++sb) d[sb] = mfma32(VF.v[sb], sel, zero4());
#pragma unroll
      for (int m = 0; m < 2; ++m) vt[k][m] = frag_acc(d[2 * m] * eta_s[2 * m], d[2 * m + 1] * eta_s[2 * m + 1]);
    }
    // this wave's next chunk is c + 1
    if (c + 1 < nchunks) load_values(VF, sq, c + 1, fw - 2, l);
    // ---- decayed read mask: M^T tile (sb, ib) = X_sb Q_ib^T, s <= i -------
    const f32x4 gra_i = ld4(&G.graw_t[c16 * 4]);
    const int n0 = fw == 2 ? 0 : 5;
#pragma unroll
    for (int n5 = 0; n5 < 5; ++n5) {
      int ib, sb;
      lower_tile(n0 + n5, ib, sb);
      f32x4 acc = zero4();
#pragma unroll
      for (int m = 0; m < 2; ++m)
        acc = mfma32(ring_frag_c(E.x, 16 * sb + c16, m, g), ring_frag_c(E.q, 16 * ib + c16, m, g), acc);
      const int i = 16 * ib + c16;
      const f32x4 gs = ld4(&G.graw[16 * sb + 4 * g]);
      const float gi_ib = ib == 0 ? gra_i[0] : ib == 1 ? gra_i[1] : ib == 2 ? gra_i[2] : gra_i[3];
      f32x4 mv;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int s_ = 16 * sb + 4 * g + r;
        mv[r] = s_ <= i ? __expf(gi_ib - gs[r]) * acc[r] : 0.0f;
      }
      store_half(&S.mf[((ib * 2 + (sb >> 1)) * 64 + l) * 8 + 4 * (sb & 1)], mv);
    }
  }
  if (load_next) {
    const int e = (c + 1) % kNI;
    if (!wait_at_least(&sm.in_free[e], 2 * ((c + 1) / kNI), &sm.abort_flag)) return false;
    ring_store(sm.in[e], rr, sq, c + 1, l, eps, eps_gamma, fresh);
    signal_add(&sm.in_ready[e], l);
  }
  // ---- wait for T, then W^T tiles (fb, ib) = X~^T T^T and U = T V~ ---------
  if (!wait_at_least(&sm.t_ready[c & 1], c + 1, &sm.abort_flag)) return false;
  bf16x8 tf[4][2];
#pragma unroll
  for (int ib = 0; ib < 4; ++ib) {
    tf[ib][0] = frag_lds(&tb[(16 * ib + c16) * kP], 0, g);
    tf[ib][1] = frag_lds(&tb[(16 * ib + c16) * kP], 32, g);
  }
  signal_add(&sm.t_used[c & 1], l);
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    if (k < nfb) {
      const int fb = fb0 + k;
#pragma unroll
      for (int ib = 0; ib < 4; ++ib) {
        f32x4 acc = mfma32(xg[k][0], tf[ib][0], zero4());
        if (ib >= 2) acc = mfma32(xg[k][1], tf[ib][1], acc);   // T is lower triangular
        store_half(&S.wf[((ib * 2 + (fb >> 1)) * 64 + l) * 8 + 4 * (fb & 1)], -acc);
      }
    }
  }
  if constexpr (kRole == 2) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int cb = 2 * (fw - 2) + k;
#pragma unroll
      for (int ib = 0; ib < 4; ++ib) {
        f32x4 u = mfma32(tf[ib][0], vt[k][0], zero4());
        if (ib >= 2) u = mfma32(tf[ib][1], vt[k][1], u);
        store_half(&S.uf[((ib * 4 + cb) * 64 + l) * 4], u);
      }
    }
  }
  signal_add(&sm.slot_full[c % kNS], l);
  return true;
}

// ---------------------------------------------------------------------------
// Chain wave w: consumes chunk c for value columns 32w..32w+31.
// ---------------------------------------------------------------------------
__device__ bool chain_chunk(Smem& sm, f32x4 (&Sst)[4][2], const Seq& sq, int c, int w, int l,
                            bf16_t* o_bh, int nchunks) {
  const int g = l >> 4, c16 = l & 15;
  const int t0 = c * kC;
  if (!wait_at_least(&sm.slot_full[c % kNS], kSlotWriters * (c / kNS + 1), &sm.abort_flag)) return false;
  const Slot& S = sm.slot[c % kNS];
  const InputEntry& E = sm.in[c % kNI];

  // ---- slot reads: U tiles and -W fragments, then R = U - W S --------------
  f32x4 R[4][2];
  bf16x8 sb[2][2];                                           // S fragments [cb][m]
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    sb[k][0] = frag_acc(Sst[0][k], Sst[1][k]);
    sb[k][1] = frag_acc(Sst[2][k], Sst[3][k]);
  }
#pragma unroll
  for (int ib = 0; ib < 4; ++ib) {
    const bf16x8 w0 = load_frag(&S.wf[((ib * 2 + 0) * 64 + l) * 8]);
    const bf16x8 w1 = load_frag(&S.wf[((ib * 2 + 1) * 64 + l) * 8]);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      f32x4 u = load_half(&S.uf[((ib * 4 + 2 * w + k) * 64 + l) * 4]);
      u = mfma32(w0, sb[k][0], u);
      R[ib][k] = mfma32(w1, sb[k][1], u);
    }
  }
  // ---- slot reads: mask and decayed-key fragments, output and decay scales --
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
  const f32x4 gexp_i = ld4(&E.gt.gexp_t[c16 * 4]);
  const float glast = E.gt.glast[0];
  bf16x8 qf[4][2];                                           // queries of row block ib
#pragma unroll
  for (int ib = 0; ib < 4; ++ib) {
    qf[ib][0] = ring_frag_p(E.q, 16 * ib + c16, 0, g);
    qf[ib][1] = ring_frag_p(E.q, 16 * ib + c16, 1, g);
  }
  signal_add(&sm.slot_free[c % kNS], l);                     // slot and entry contents are in registers
  signal_add(&sm.in_free[c % kNI], l);

  bf16x8 rb[2][2];                                           // R fragments [cb][m]
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    rb[k][0] = frag_acc(R[0][k], R[1][k]);
    rb[k][1] = frag_acc(R[2][k], R[3][k]);
  }
  // ---- O^T tiles: e^{g_i} S^T Q^T + R^T M^T; lane holds o[t0+16ib+c16][32w+16k+4g+r]
#pragma unroll
  for (int ib = 0; ib < 4; ++ib) {
    const int i = 16 * ib + c16;
    const bf16x8 q0 = qf[ib][0], q1 = qf[ib][1];
    const int tok = t0 + i;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      f32x4 acc = mfma32(sb[k][0], q0, zero4());
      acc = mfma32(sb[k][1], q1, acc);
      acc = acc * gexp_i[ib];
      acc = mfma32(rb[k][0], mfr[ib][0], acc);
      if (ib >= 2) acc = mfma32(rb[k][1], mfr[ib][1], acc);
      if (tok < sq.T) {
        *reinterpret_cast<uint2*>(o_bh + int64_t(tok) * kD + 32 * w + 16 * k + 4 * g) =
            make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
      }
    }
  }
  // ---- S <- e^{g_63} S + (Diag(e^{g_63-g}) X)^T R ---------------------------
#pragma unroll
  for (int fb = 0; fb < 4; ++fb)
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      f32x4 acc = Sst[fb][k] * glast;
      acc = mfma32(xhr[fb][0], rb[k][0], acc);
      Sst[fb][k] = mfma32(xhr[fb][1], rb[k][1], acc);
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
  for (int e = tid; e < 2 * kC * kP; e += kThreads) sm.tb[e / (kC * kP)][e % (kC * kP)] = 0;
  for (int s = 0; s < kNS; ++s)
    for (int e = tid; e < 4 * 2 * 64 * 8; e += kThreads) sm.slot[s].mf[e] = 0;
  if (tid < kNI) { sm.in_ready[tid] = 0; sm.in_free[tid] = 0; }
  if (tid < kNS) { sm.slot_full[tid] = 0; sm.slot_free[tid] = 0; }
  if (tid < 2) { sm.t_ready[tid] = 0; sm.t_used[tid] = 0; }
  if (tid == 0) sm.abort_flag = 0;
  __syncthreads();

  if (wave < kChain) {
    const int w = wave;
    f32x4 Sst[4][2];
#pragma unroll
    for (int fb = 0; fb < 4; ++fb)
#pragma unroll
      for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          Sst[fb][k][r] = S0 ? S0[(bh * kD + 16 * fb + 4 * g + r) * kD + 32 * w + 16 * k + c16] : 0.0f;
    for (int c = 0; c < nchunks; ++c) {
      if (!chain_chunk(sm, Sst, sq, c, w, l, o + bh * T * kD, nchunks)) break;
    }
    if (S_T) {
#pragma unroll
      for (int fb = 0; fb < 4; ++fb)
#pragma unroll
        for (int k = 0; k < 2; ++k)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            S_T[(bh * kD + 16 * fb + 4 * g + r) * kD + 32 * w + 16 * k + c16] = Sst[fb][k][r];
    }
  } else {
    const int fw = wave - kChain;
    const bool fresh = (k_prev == nullptr);
    ValueFrags VF;
    if (fw == 0) {
      for (int c = 0; c < nchunks; ++c)
        if (!factor_chunk<0>(sm, VF, sq, c, fw, l, eps, eps_gamma, fresh, nchunks)) break;
    } else if (fw == 1) {
      // prologue: the first ring entry
      {
        RingRegs rr;
        ring_fetch(rr, sq, 0, l);
        ring_store(sm.in[0], rr, sq, 0, l, eps, eps_gamma, fresh);
        signal_add(&sm.in_ready[0], l);
      }
      for (int c = 0; c < nchunks; ++c)
        if (!factor_chunk<1>(sm, VF, sq, c, fw, l, eps, eps_gamma, fresh, nchunks)) break;
    } else {
      load_values(VF, sq, 0, fw - 2, l);
      for (int c = 0; c < nchunks; ++c)
        if (!factor_chunk<2>(sm, VF, sq, c, fw, l, eps, eps_gamma, fresh, nchunks)) break;
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
