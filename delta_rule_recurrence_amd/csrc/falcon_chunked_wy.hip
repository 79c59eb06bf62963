// Chunked Falcon-1 forward in two launches (gfx950, bf16 I/O, dk = dv = 64,
// chunk C = 64).
//
// The chunk form (the log-space renormalisation of Section 4.4 with window 1,
// applied per chunk; g_i the chunk-local prefix of log gamma):
//   A_{i,s} = eta_i e^{g_{i-1}-g_s} (x_i . x_s) for s < i,   T = (I + A)^{-1}
//   W = T Diag(eta e^{g_{s-1}}) X,   U = T Diag(eta) V
//   R = U - W S,   S' = e^{g_63} S + (Diag(e^{g_63-g}) X)^T R
//   O = Diag(e^g) Q S + (tril0(Q X^T) o [e^{g_i-g_s}]) R.
// W and U depend only on the chunk's own keys, values and gates (the "WY"
// factors of Section 4.2's chunk-parallel implementation).  They are built
// for every chunk of every sequence at once (launch 1, one workgroup per
// chunk, the whole chip busy) and written to the workspace in MFMA fragment
// order; launch 2 then runs the short sequential part, the state passing and
// the outputs, one workgroup per sequence, streaming the factors back.

#include "falcon_device.h"
#include "falcon_launch.h"
#include "falcon_mfma_frag.h"

namespace falcon {

namespace {

using namespace frag;

constexpr int kC = 64;
constexpr int kD = 64;
constexpr int kP = 72;                  // bf16 row pitch of T in LDS
// Per-chunk factor block in the workspace: -W fragments, U tiles and the
// decayed keys (8 KiB each, bf16), then the chunk's gates (1 KiB, float).
constexpr int kFactorBytes = 25600;
constexpr int kFacU = 4096;             // bf16 element offsets of the parts
constexpr int kFacXh = 8192;
constexpr int kFacGates = 12288;        // float gates: g_s [64], g_i at [c16*4+ib] [64], e^{g_i} same order [64], e^{g_63}
constexpr int kSpinLimit = 1 << 22;

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
// Launch 1: WY factors of one chunk per workgroup (four waves).
// ============================================================================

struct WyGates {
  float graw[kC];                 // g_s, token order
  float sxg[kC];                  // eta_s e^{g_{s-1}}
  float sxh[kC];                  // e^{g_63 - g_s}
  float eta[kC];                  // eta_s
  float eta_t[kC];                // eta_i at [c16 * 4 + ib] for i = 16 ib + c16
  float gprev_t[kC];              // g_{i-1}, same order
};

struct WySmem {
  uint16_t x[kC * kD];            // keys, swizzled rows
  uint16_t v[kC * kD];            // values, swizzled rows
  uint16_t tb[kC * kP];           // T, row-major
  float abt[4][16][16];           // diagonal blocks of -A: [b][s][i] = -A[16b+i][16b+s]
  WyGates G;
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

// Workspace block of one chunk: -W as A fragments [ib][m][lane][8] (lane row =
// token 16 ib + c16, k = features 32 m + kperm), U as result tiles
// [ib][cb][lane][4] (lane holds U[16ib+4g+r][16cb+c16]), the decayed keys
// (Diag(e^{g_63-g}) X)^T as A fragments [fb][m][lane][8] (lane row = feature
// 16 fb + c16, k = tokens 32 m + kperm), all bf16, then the gates in float.
__global__ void __launch_bounds__(256, 2)
falcon1_wy_kernel(const bf16_t* __restrict__ phi_k, const bf16_t* __restrict__ v,
                  const float* __restrict__ beta, const float* __restrict__ lam,
                  const bf16_t* __restrict__ k_prev, uint16_t* __restrict__ factors, int T, int nchunks,
                  float eps, float eps_gamma) {
  __shared__ WySmem sm;
  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63;
  const int g = l >> 4, c16 = l & 15;
  const int64_t bh = blockIdx.x / nchunks;
  const int c = blockIdx.x % nchunks;
  const Seq sq = make_seq(phi_k, nullptr, v, beta, lam, k_prev, bh, T);
  const bool fresh = (k_prev == nullptr);
  uint16_t* out = factors + int64_t(blockIdx.x) * (kFactorBytes / 2);

  // ---- stage keys and values: wave w rows 16w..16w+15, 8 lanes per row -----
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = 16 * w + 8 * j + (l >> 3);
    const int off = r * kD + 8 * seg_pos(r, l & 7);
    *reinterpret_cast<bf16x8*>(sm.x + off) = *reinterpret_cast<const bf16x8*>(key_row(sq, c, r) + 8 * (l & 7));
    *reinterpret_cast<bf16x8*>(sm.v + off) = *reinterpret_cast<const bf16x8*>(token_row(sq.V, sq, c, r) + 8 * (l & 7));
  }
  // T's upper blocks are never written
  for (int e = tid; e < kC * kP / 2; e += 256) reinterpret_cast<uint32_t*>(sm.tb)[e] = 0u;
  __syncthreads();
  // ---- a1: gates (wave 0) ----------------------------------------------------
  if (w == 0) {
    bf16x8 x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = 8 * j + (l >> 3);
      x[j] = *reinterpret_cast<const bf16x8*>(sm.x + r * kD + 8 * seg_pos(r, l & 7));
    }
    const int tok = c * kC + l < T ? c * kC + l : T - 1;
    float eta, gi, gprev, glast;
    chunk_gates(x, sq.beta[tok], sq.lam[tok], c * kC + l, T, eps, eps_gamma, fresh, l, eta, gi, gprev, glast);
    sm.G.graw[l] = gi;
    sm.G.sxg[l] = eta * __expf(gprev);
    sm.G.sxh[l] = __expf(glast - gi);
    sm.G.eta[l] = eta;
    sm.G.eta_t[c16 * 4 + g] = eta;
    sm.G.gprev_t[c16 * 4 + g] = gprev;
    float* gout = reinterpret_cast<float*>(out + kFacGates);
    gout[l] = gi;
    gout[64 + c16 * 4 + g] = gi;
    gout[128 + c16 * 4 + g] = __expf(gi);
    gout[192 + l] = __expf(glast);
  }
  __syncthreads();
  bf16x8 xg[2][2];              // waves 1, 2: (Diag(eta e^{g_{s-1}}) X)^T for key blocks 2(w-1), 2(w-1)+1
  bf16x8 vt[4][2];              // wave 3: Diag(eta) V for value blocks 0..3, as B fragments
  if (w == 0) {
    build_inverse(sm, l);
  } else if (w <= 2) {
    const int mk = w - 1;       // feature half
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const bf16x8 sel = select_frag(h, g, c16);
      f32x4 d[4];
#pragma unroll
      for (int sb = 0; sb < 4; ++sb) d[sb] = mfma32(ring_frag_c(sm.x, 16 * sb + c16, mk, g), sel, zero4());
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        xg[h][m] = frag_acc(d[2 * m] * ld4(&sm.G.sxg[32 * m + 4 * g]), d[2 * m + 1] * ld4(&sm.G.sxg[32 * m + 16 + 4 * g]));
        *reinterpret_cast<bf16x8*>(out + kFacXh + (((2 * mk + h) * 2 + m) * 64 + l) * 8) =
            frag_acc(d[2 * m] * ld4(&sm.G.sxh[32 * m + 4 * g]), d[2 * m + 1] * ld4(&sm.G.sxh[32 * m + 16 + 4 * g]));
      }
    }
  } else {
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const bf16x8 sel = select_frag(cb & 1, g, c16);
      f32x4 d[4];
#pragma unroll
      for (int sb = 0; sb < 4; ++sb) d[sb] = mfma32(ring_frag_c(sm.v, 16 * sb + c16, cb >> 1, g), sel, zero4());
#pragma unroll
      for (int m = 0; m < 2; ++m)
        vt[cb][m] = frag_acc(d[2 * m] * ld4(&sm.G.eta[32 * m + 4 * g]), d[2 * m + 1] * ld4(&sm.G.eta[32 * m + 16 + 4 * g]));
    }
  }
  __syncthreads();                                           // T complete
  if (w == 0) return;
  bf16x8 tf[4][2];
#pragma unroll
  for (int ib = 0; ib < 4; ++ib) {
    tf[ib][0] = frag_lds(&sm.tb[(16 * ib + c16) * kP], 0, g);
    tf[ib][1] = frag_lds(&sm.tb[(16 * ib + c16) * kP], 32, g);
  }
  if (w <= 2) {
    // -W^T tiles (fb, ib) for fb = 2m, 2m+1 stack into the A fragment (ib, m)
    const int m = w - 1;
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) {
      f32x4 d0 = mfma32(xg[0][0], tf[ib][0], zero4());
      f32x4 d1 = mfma32(xg[1][0], tf[ib][0], zero4());
      if (ib >= 2) {                                          // T is lower triangular
        d0 = mfma32(xg[0][1], tf[ib][1], d0);
        d1 = mfma32(xg[1][1], tf[ib][1], d1);
      }
      *reinterpret_cast<bf16x8*>(out + ((ib * 2 + m) * 64 + l) * 8) = frag_acc(-d0, -d1);
    }
  } else {
    uint16_t* uo = out + kFacU;
#pragma unroll
    for (int ib = 0; ib < 4; ++ib)
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        f32x4 u = mfma32(tf[ib][0], vt[cb][0], zero4());
        if (ib >= 2) u = mfma32(tf[ib][1], vt[cb][1], u);
        store_half(uo + ((ib * 4 + cb) * 64 + l) * 4, u);
      }
  }
}

// ============================================================================
// Launch 2: state passing and outputs, one workgroup per sequence.
//
// Seven waves: s0 stages the keys and queries of chunk c + 1 and s1 its factor
// block into a 3-entry LDS ring; one mask wave builds the decayed read mask of
// chunk c into one of two slots; chain waves c0..c3 (value columns
// 16 w .. 16 w + 15, fp32 state in MFMA result registers) run R = U - W S, the
// outputs and the state update.  Hand-over is through LDS counters with
// bounded waits.
// ============================================================================

constexpr int kNI = 3;
constexpr int kNS = 2;
constexpr int kChainWaves = 4;
constexpr int kStageWaves = 2;
constexpr int kMaskWaves = 1;
constexpr int kChainThreads = 64 * (kStageWaves + kMaskWaves + kChainWaves);

struct ChainEntry {
  uint16_t x[kC * kD];            // keys, swizzled rows
  uint16_t q[kC * kD];            // queries, swizzled rows
  uint16_t fac[kFactorBytes / 2]; // the chunk's factor block (with its gates)
  __device__ const float* gates() const { return reinterpret_cast<const float*>(fac + kFacGates); }
};

struct ChainSlot {
  uint16_t mf[4 * 2 * 64 * 8];    // M^T as B fragments [ib][m][lane][8]
};

struct ChainSmem {
  ChainEntry in[kNI];
  ChainSlot slot[kNS];
  int in_ready[kNI];              // +1 per staging wave when its part of an entry is filled
  int in_free[kNI];               // +1 per chain wave done with an entry
  int slot_full[kNS];             // +1 per mask wave when its tiles of a slot are written
  int slot_free[kNS];             // +1 per chain wave done with a slot
  int abort_flag;
};

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

struct RowRegs {
  bf16x8 x[8], q[8];
};

__device__ __forceinline__ void rows_fetch(RowRegs& R, const Seq& sq, int c, int l) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = 8 * j + (l >> 3);
    R.x[j] = *reinterpret_cast<const bf16x8*>(key_row(sq, c, r) + 8 * (l & 7));
    R.q[j] = *reinterpret_cast<const bf16x8*>(token_row(sq.Q, sq, c, r) + 8 * (l & 7));
  }
}

__device__ __forceinline__ void rows_store(ChainEntry& E, const RowRegs& R, int l) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = 8 * j + (l >> 3);
    const int off = r * kD + 8 * seg_pos(r, l & 7);
    *reinterpret_cast<bf16x8*>(E.x + off) = R.x[j];
    *reinterpret_cast<bf16x8*>(E.q + off) = R.q[j];
  }
}

constexpr int kFacFrags = kFactorBytes / 16 / 64;   // 16-byte fragments per lane in a factor block

struct FacRegs {
  bf16x8 f[kFacFrags];
};

__device__ __forceinline__ void fac_fetch(FacRegs& R, const uint16_t* fac, int l) {
#pragma unroll
  for (int j = 0; j < kFacFrags; ++j) R.f[j] = *reinterpret_cast<const bf16x8*>(fac + (j * 64 + l) * 8);
}
__device__ __forceinline__ void fac_store(ChainEntry& E, const FacRegs& R, int l) {
#pragma unroll
  for (int j = 0; j < kFacFrags; ++j) *reinterpret_cast<bf16x8*>(E.fac + (j * 64 + l) * 8) = R.f[j];
}

__global__ void __launch_bounds__(kChainThreads)
falcon1_chain_kernel(const bf16_t* __restrict__ phi_k, const bf16_t* __restrict__ phi_q,
                     const float* __restrict__ beta, const float* __restrict__ lam, const float* S0,
                     const bf16_t* __restrict__ k_prev, const uint16_t* __restrict__ factors,
                     bf16_t* __restrict__ o, float* S_T, int T, float eps, float eps_gamma) {
  __shared__ ChainSmem sm;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, l = tid & 63;
  const int g = l >> 4, c16 = l & 15;
  const int64_t bh = blockIdx.x;
  const int nchunks = (T + kC - 1) / kC;
  const Seq sq = make_seq(phi_k, phi_q, nullptr, beta, lam, k_prev, bh, T);
  const bool fresh = (k_prev == nullptr);
  const uint16_t* fac_bh = factors + bh * nchunks * (kFactorBytes / 2);

  // halves of the mask fragments above the diagonal are never written
  for (int s = 0; s < kNS; ++s)
    for (int e = tid; e < 4 * 2 * 64 * 8 / 2; e += kChainThreads) reinterpret_cast<uint32_t*>(sm.slot[s].mf)[e] = 0u;
  if (tid < kNI) { sm.in_ready[tid] = 0; sm.in_free[tid] = 0; }
  if (tid < kNS) { sm.slot_full[tid] = 0; sm.slot_free[tid] = 0; }
  if (tid == 0) sm.abort_flag = 0;
  __syncthreads();

  if (wave == 0) {
    // ---- s0: keys and queries, one chunk ahead ------------------------------
    RowRegs R;
    if (nchunks > 0) rows_fetch(R, sq, 0, l);
    for (int c = 0; c < nchunks; ++c) {
      const int e = c % kNI;
      if (!wait_at_least(&sm.in_free[e], kChainWaves * (c / kNI), &sm.abort_flag)) break;
      rows_store(sm.in[e], R, l);
      signal_add(&sm.in_ready[e], l);
      if (c + 1 < nchunks) rows_fetch(R, sq, c + 1, l);
    }
    return;
  }
  if (wave == 1) {
    // ---- s1: the chunk's factor block, one chunk ahead ---------------------
    FacRegs R;
    if (nchunks > 0) fac_fetch(R, fac_bh, l);
    for (int c = 0; c < nchunks; ++c) {
      const int e = c % kNI;
      if (!wait_at_least(&sm.in_free[e], kChainWaves * (c / kNI), &sm.abort_flag)) break;
      fac_store(sm.in[e], R, l);
      signal_add(&sm.in_ready[e], l);
      if (c + 1 < nchunks) fac_fetch(R, fac_bh + int64_t(c + 1) * (kFactorBytes / 2), l);
    }
    return;
  }
  if (wave < kStageWaves + kMaskWaves) {
    // ---- mask waves: decayed read mask, tiles [n0, n0 + 10 / kMaskWaves) -----
    constexpr int kTiles = 10 / kMaskWaves;
    const int n0 = kTiles * (wave - kStageWaves);
    for (int c = 0; c < nchunks; ++c) {
      const ChainEntry& E = sm.in[c % kNI];
      ChainSlot& Sl = sm.slot[c % kNS];
      if (!wait_at_least(&sm.in_ready[c % kNI], kStageWaves * (c / kNI + 1), &sm.abort_flag)) break;
      if (!wait_at_least(&sm.slot_free[c % kNS], kChainWaves * (c / kNS), &sm.abort_flag)) break;
      const float* gts = E.gates();
      const f32x4 gra_i = ld4(&gts[64 + c16 * 4]);
      // M^T tile (sb, ib) = X_sb Q_ib^T scaled by e^{g_i-g_s}, s <= i
#pragma unroll
      for (int nt = 0; nt < kTiles; ++nt) {
        int ib, sb;
        lower_tile(n0 + nt, ib, sb);
        f32x4 acc = mfma32(ring_frag_c(E.x, 16 * sb + c16, 0, g), ring_frag_c(E.q, 16 * ib + c16, 0, g), zero4());
        acc = mfma32(ring_frag_c(E.x, 16 * sb + c16, 1, g), ring_frag_c(E.q, 16 * ib + c16, 1, g), acc);
        const f32x4 gs = ld4(&gts[16 * sb + 4 * g]);
        const float gi_ib = ib == 0 ? gra_i[0] : ib == 1 ? gra_i[1] : ib == 2 ? gra_i[2] : gra_i[3];
        const int i = 16 * ib + c16;
        f32x4 mv;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int s_ = 16 * sb + 4 * g + r;
          mv[r] = s_ <= i ? __expf(gi_ib - gs[r]) * acc[r] : 0.0f;
        }
        store_half(&Sl.mf[((ib * 2 + (sb >> 1)) * 64 + l) * 8 + 4 * (sb & 1)], mv);
      }
      signal_add(&sm.slot_full[c % kNS], l);
    }
    return;
  }
  // ---- chain waves ------------------------------------------------------------
  const int cb = wave - kStageWaves - kMaskWaves;            // value columns 16 cb .. 16 cb + 15
  f32x4 S[4];                                                // S[fb]: lane holds S[16fb+4g+r][16cb+c16]
#pragma unroll
  for (int fb = 0; fb < 4; ++fb)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      S[fb][r] = S0 ? S0[(bh * kD + 16 * fb + 4 * g + r) * kD + 16 * cb + c16] : 0.0f;
  bf16_t* o_bh = o + bh * T * kD;
  for (int c = 0; c < nchunks; ++c) {
    const ChainEntry& E = sm.in[c % kNI];
    const ChainSlot& Sl = sm.slot[c % kNS];
    if (!wait_at_least(&sm.slot_full[c % kNS], kMaskWaves * (c / kNS + 1), &sm.abort_flag)) break;
    // everything this wave needs from the entry and the slot, into registers
    bf16x8 wf[4][2], mfr[4][2], xhr[4][2], qf[4][2];
    f32x4 uf[4];
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) {
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        wf[ib][m] = load_frag(&E.fac[((ib * 2 + m) * 64 + l) * 8]);
        xhr[ib][m] = load_frag(&E.fac[kFacXh + ((ib * 2 + m) * 64 + l) * 8]);
        qf[ib][m] = ring_frag_p(E.q, 16 * ib + c16, m, g);
      }
      mfr[ib][0] = load_frag(&Sl.mf[((ib * 2 + 0) * 64 + l) * 8]);
      if (ib >= 2) mfr[ib][1] = load_frag(&Sl.mf[((ib * 2 + 1) * 64 + l) * 8]);
      uf[ib] = load_half(&E.fac[kFacU + ((ib * 4 + cb) * 64 + l) * 4]);
    }
    const f32x4 gexp_i = ld4(&E.gates()[128 + c16 * 4]);
    const float glast = E.gates()[192];
    signal_add(&sm.slot_free[c % kNS], l);
    signal_add(&sm.in_free[c % kNI], l);
    // R = U - W S (rows eta_i r_i); lane holds R[16ib+4g+r][16cb+c16]
    const bf16x8 sb0 = frag_acc(S[0], S[1]);
    const bf16x8 sb1 = frag_acc(S[2], S[3]);
    f32x4 R[4];
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) {
      f32x4 u = mfma32(wf[ib][0], sb0, uf[ib]);
      R[ib] = mfma32(wf[ib][1], sb1, u);
    }
    const bf16x8 rb0 = frag_acc(R[0], R[1]);
    const bf16x8 rb1 = frag_acc(R[2], R[3]);
    // O^T tiles: e^{g_i} S^T Q^T + R^T M^T; lane holds o[t0+16ib+c16][16cb+4g+r]
    const int t0 = c * kC;
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) {
      f32x4 acc = mfma32(sb0, qf[ib][0], zero4());
      acc = mfma32(sb1, qf[ib][1], acc);
      acc = acc * gexp_i[ib];
      acc = mfma32(rb0, mfr[ib][0], acc);
      if (ib >= 2) acc = mfma32(rb1, mfr[ib][1], acc);
      const int tok = t0 + 16 * ib + c16;
      if (tok < T)
        *reinterpret_cast<uint2*>(o_bh + int64_t(tok) * kD + 16 * cb + 4 * g) =
            make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
    }
    // S <- e^{g_63} S + (Diag(e^{g_63-g}) X)^T R
#pragma unroll
    for (int fb = 0; fb < 4; ++fb) {
      f32x4 acc = S[fb] * glast;
      acc = mfma32(xhr[fb][0], rb0, acc);
      S[fb] = mfma32(xhr[fb][1], rb1, acc);
    }
  }
  if (S_T) {
#pragma unroll
    for (int fb = 0; fb < 4; ++fb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        S_T[(bh * kD + 16 * fb + 4 * g + r) * kD + 16 * cb + c16] = S[fb][r];
  }
}

}  // namespace

bool chunked_wy_applies(const ProblemArgs& a) {
  return a.bf16 && a.variant == kF1 && a.dk == kD && a.dv == kD && a.C == kC && a.T > 0;
}

size_t chunked_wy_workspace_bytes(const ProblemArgs& a) {
  const int64_t nchunks = (int64_t(a.T) + kC - 1) / kC;
  return size_t(int64_t(a.B) * a.H * nchunks) * kFactorBytes;
}

hipError_t launch_chunked_wy(const ProblemArgs& a, hipStream_t st) {
  const int64_t BH = int64_t(a.B) * a.H;
  const int nchunks = (a.T + kC - 1) / kC;
  if (BH == 0 || nchunks == 0) return hipSuccess;
  uint16_t* factors = static_cast<uint16_t*>(a.workspace);
  hipLaunchKernelGGL(falcon1_wy_kernel, dim3(unsigned(BH * nchunks)), dim3(256), 0, st,
                     static_cast<const bf16_t*>(a.phi_k), static_cast<const bf16_t*>(a.v), a.beta, a.lam,
                     static_cast<const bf16_t*>(a.k_prev), factors, a.T, nchunks, a.eps, a.eps_gamma);
  hipLaunchKernelGGL(falcon1_chain_kernel, dim3(unsigned(BH)), dim3(kChainThreads), 0, st,
                     static_cast<const bf16_t*>(a.phi_k), static_cast<const bf16_t*>(a.phi_q), a.beta, a.lam,
                     a.S0, static_cast<const bf16_t*>(a.k_prev), factors, static_cast<bf16_t*>(a.o), a.S_T,
                     a.T, a.eps, a.eps_gamma);
  return hipGetLastError();
}

}  // namespace falcon
