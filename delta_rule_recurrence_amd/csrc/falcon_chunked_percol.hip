// Chunked forward of the per-column rules (Falcon-2 and Falcon-2A) on gfx950,
// bf16 I/O, dk = dv = 64, chunk C = 64.
//
// Falcon-2 gives every value column j its own NLMS step size
// eta_{t,j} = beta_{t,j} / (||x_t||^2 + lam_t + eps) and decay
// gamma_{t,j} = 1 - min(eta_{t,j} lam_t, 1 - eps_gamma) (Section 4.2, Eq. 4.7,
// and the clamp of Section 4.3), so column j of S follows the scalar rule on
// its own.  Within a chunk with incoming state S, per column j (g_{i,j} the
// chunk-local prefix of log gamma):
//   rho_{i,j} + sum_{s<i} eta_{i,j} e^{g_{i-1,j}-g_{s,j}} (x_i.x_s) rho_{s,j}
//        = eta_{i,j} (v_{i,j} - e^{g_{i-1,j}} (X S)_{i,j})
// (the merged residual system of Section 4.2; rho_{i,j} = eta_{i,j} v_{i,j}
// for the additive Falcon-2A), and
//   o_{i,j} = e^{g_{i,j}} (Q S)_{i,j} + sum_{s<=i} e^{g_{i,j}-g_{s,j}} (q_i.x_s) rho_{s,j}
//   S'_{:,j} = e^{g_{63,j}} S_{:,j} + sum_s e^{g_{63,j}-g_{s,j}} x_s rho_{s,j}.
// The decays differ per column, so the triangular system is solved per
// column, in four 16-row blocks.  Lane layout in the solve: a 16-lane row of a
// wave is one value column, lane li is row 16b + li of block b.
//  * Earlier blocks enter through w_s = e^{g_{16b-1}-g_s} rho_s (kept per column
//    in LDS, every factor <= 1): row i gets
//    eta_i e^{g_{i-1}-g_{16b-1}} sum_{s<16b} (x_i.x_s) w_s, off the critical path.
//  * Inside the block, forward substitution runs in registers: step s adds
//    -c_{i,s} rho_s to every later row, rho_s broadcast from lane s by a DPP
//    row broadcast (row_newbcast), 15 dependent steps per block.
//  * The products shared by all columns (x_i.x_s, q_i.x_s, X S, Q S and the
//    state update) run on the matrix cores; each solve block forms its own
//    rows of X S and Q S from a bf16 copy of the state.
// One workgroup (four waves, four value columns each) per (batch, head,
// 16-column slice).  Per chunk two phases: the solve (during which the next
// chunk's rows go into the second LDS row buffer), then the outputs, the
// state update (wave w owns state rows 16w..16w+15) and the next chunk's Gram
// products.  Rows are fetched into registers a chunk ahead.

#include <vector>

#include "falcon_device.h"
#include "falcon_launch.h"
#include "falcon_mfma_frag.h"

namespace falcon {

namespace {

using namespace frag;

constexpr int kC = 64;
constexpr int kD = 64;
constexpr int kSlice = 16;                  // value columns per workgroup
constexpr int kThreads = 256;
constexpr int kDP = 20;                     // float row pitch of the diagonal Gram blocks (16-byte reads conflict-free)
constexpr int kSbP = 72;                    // bf16 pitch of the state copy sb

// Per-column arrays hold kSlice columns of kC rows, column by column, row i
// of column j at j kC + (i ^ 16 (j & 3)): a solve read of row 16B + li in
// column 4w + g lands in bank 16 (B ^ g) + li, so the 64 lanes of a wave hit
// 64 distinct banks, and every aligned run of four rows stays contiguous.
__device__ __forceinline__ int cix(int j, int i) { return j * kC + (i ^ ((j & 3) << 4)); }

struct PcSmem {
  uint16_t x[2][kC * kD];                   // keys phi(k_{t0+r-1}), swizzled rows, of two chunks
  uint16_t q[2][kC * kD];                   // queries, swizzled rows, of two chunks
  float kqd[4][16][kDP];                    // diagonal blocks: [b][i-16b][s-16b] = x_i . x_s for s < i, else 0
  float pqd[4][16][kDP];                    // diagonal blocks: [b][i-16b][s-16b] = q_i . x_s for s < i, else 0
  uint16_t kqf[3][2][64 * 8];               // frag(KQ)[b][m] for b = 1..3, entries s < 16 b only, bf16
  uint16_t pqf[3][2][64 * 8];               // frag(PQ)[b][m], same
  float vb[kSlice * kC];                    // v_{i,j} at cix(j, i)
  float bt[kSlice * kC];                    // beta_{i,j} at cix(j, i)
  float lm[kC];                             // lam_i
  float en[kC];                             // ||x_i||^2
  float pd[kC];                             // q_i . x_i
  float w[kSlice * kC];                     // per column j: e^{g_b-g_s} rho_s at cix(j, s), b = end of the last solved block
  float e63[kSlice];                        // e^{g_63} per column
  uint16_t ob[kC][kSlice];                  // outputs of the chunk, bf16
  uint16_t sb[kSlice][kSbP];                // the slice's state in bf16, column by column: sb[j][k] = S[k][j0 + j]
};

// Lane N of the lane's 16-lane row (DPP row_newbcast; every lane has a
// source, so no fill value is needed and the move can fuse into its user).
template <int N>
__device__ __forceinline__ float row_bcast(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x150 + N, 0xf, 0xf, false));
}
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
constexpr float kLog2e = 1.4426950408889634f;

// log2 of the clamped decay 1 - min(eta lam, 1 - eps_gamma) (Section 4.3) in
// float32, as log2(u) (1 - gamma) / (1 - u) with u = 1 - alpha rounded: the
// ratio cancels the rounding of u (Kahan's compensated log1p), so small alpha
// keeps its relative accuracy; log2 and the reciprocal are the hardware's.
// Also returns gamma itself (u).
// Branch-free: both forms are computed and blended by a 0/1 weight (when
// u rounds to 1 the log is exactly 0 and the ratio finite, so the blend is
// exact), which keeps the hardware log and reciprocal out of a lane-masked
// branch.
__device__ __forceinline__ float log2_gamma(float eta, float lam, float eps_gamma, float& gamma) {
  // a binding clamp takes u = eps_gamma exactly and alpha = 1 - u (ratio 1)
  const float a = eta * lam;
  const bool unclamped = 1.0f - a >= eps_gamma;
  const float u = unclamped ? 1.0f - a : eps_gamma;
  const float alpha = unclamped ? a : 1.0f - u;
  const float d = u - 1.0f;
  gamma = u;
  const float tiny = d == 0.0f ? 1.0f : 0.0f;
  const float ratio = -alpha * __builtin_amdgcn_rcpf(d - tiny);
  return __builtin_amdgcn_logf(u) * ratio - kLog2e * alpha * tiny;
}

// The next chunk's inputs, fetched into registers during the current chunk.
struct ChunkRegs {
  bf16x8 x[2], q[2];                        // rows r = 32 j + (tid >> 3), segment tid & 7
  bf16x8 v;                                 // tid < 128: row tid >> 1, columns j0 + 8 (tid & 1) ..
  float4 bt;                                // row tid >> 2, columns j0 + 4 (tid & 3) ..
  float lm;                                 // tid < 64: row tid
};

__device__ __forceinline__ void fetch_chunk(ChunkRegs& R, const bf16_t* K, const bf16_t* Q, const bf16_t* V,
                                            const float* Bt, const float* Lm, const bf16_t* kp, int T, int t0,
                                            int j0, int tid) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = 32 * j + (tid >> 3);
    const int kt = t0 + r - 1;
    const bf16_t* xsrc = kt < 0 ? (kp ? kp : K) : K + int64_t(kt < T ? kt : T - 1) * kD;
    const int tok = t0 + r < T ? t0 + r : T - 1;
    R.x[j] = *reinterpret_cast<const bf16x8*>(xsrc + 8 * (tid & 7));
    R.q[j] = *reinterpret_cast<const bf16x8*>(Q + int64_t(tok) * kD + 8 * (tid & 7));
  }
  if (tid < 128) {
    const int r = tid >> 1;
    const int tok = t0 + r < T ? t0 + r : T - 1;
    R.v = *reinterpret_cast<const bf16x8*>(V + int64_t(tok) * kD + j0 + 8 * (tid & 1));
  }
  {
    const int r = tid >> 2;
    const int tok = t0 + r < T ? t0 + r : T - 1;
    R.bt = *reinterpret_cast<const float4*>(Bt + int64_t(tok) * kD + j0 + 4 * (tid & 3));
  }
  if (tid < 64) R.lm = Lm[t0 + tid < T ? t0 + tid : T - 1];
}

// A chunk's keys and queries into one of the two row buffers.
__device__ __forceinline__ void stage_xq(uint16_t* xb, uint16_t* qb, const ChunkRegs& R, int tid) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = 32 * j + (tid >> 3);
    const int off = r * kD + 8 * seg_pos(r, tid & 7);
    *reinterpret_cast<bf16x8*>(xb + off) = R.x[j];
    *reinterpret_cast<bf16x8*>(qb + off) = R.q[j];
  }
}

// A chunk's values, beta and lam.
__device__ __forceinline__ void stage_gates(PcSmem& sm, const ChunkRegs& R, int tid) {
  if (tid < 128) {
    const int r = tid >> 1;
#pragma unroll
    for (int e = 0; e < 8; ++e) sm.vb[cix(8 * (tid & 1) + e, r)] = static_cast<float>(R.v[e]);
  }
  {
    const int r = tid >> 2, j = 4 * (tid & 3);
    sm.bt[cix(j, r)] = R.bt.x;
    sm.bt[cix(j + 1, r)] = R.bt.y;
    sm.bt[cix(j + 2, r)] = R.bt.z;
    sm.bt[cix(j + 3, r)] = R.bt.w;
  }
  if (tid < 64) sm.lm[tid] = R.lm;
}

// One 16-row block B of the per-column system and of the outputs, for the
// lane's column jl and row i = 16 B + li.  g is kept in log2 units, so every
// decay is one exp2.  gcarry holds g at the end of the previous block (0
// before block 0) and is advanced to the end of this one.
template <bool kReg, int B>
__device__ __forceinline__ void solve_block(PcSmem& sm, const uint16_t* xb, const uint16_t* qb, const bf16x8& sa0,
                                            const bf16x8& sa1, int w, int jl, int li, int t0, int T, bool fresh,
                                            float eps, float eps_gamma, float& gcarry) {
  const int i = 16 * B + li;
  const int t = t0 + i;
  const bool live = t < T;
  const int g = jl - 4 * w;
  // (X S)_{i,jl} and (Q S)_{i,jl} on the matrix cores: A's row a is the
  // state's column 4w + (a >> 2) (sa0, sa1), B's column li is row i of X (of
  // Q), so the result rows 4g..4g+3 of lane (g, li) are all row i of the
  // lane's own column 4w + g
  bf16x8 m_x0 = {}, m_x1 = {};
  const bf16x8 m_q0 = ring_frag_c(qb, i, 0, g), m_q1 = ring_frag_c(qb, i, 1, g);
  f32x4 m_qs = mfma32(sa0, m_q0, zero4());
  m_qs = mfma32(sa1, m_q1, m_qs);
  f32x4 m_xs = zero4();
  if constexpr (kReg) {
    m_x0 = ring_frag_c(xb, i, 0, g);
    m_x1 = ring_frag_c(xb, i, 1, g);
    m_xs = mfma32(sa0, m_x0, zero4());
    m_xs = mfma32(sa1, m_x1, m_xs);
  }
  // step size and decay of row i in column jl (branch-free: every operand is
  // loaded and the reciprocal taken whatever the row); g by a scan over the
  // 16 rows
  const float lmi = sm.lm[i], bti = sm.bt[cix(jl, i)];
  const float den = sm.en[i] + lmi + eps;
  const bool on = live && !(fresh && t == 0) && den != 0.0f;
  const float eta = on ? bti * __builtin_amdgcn_rcpf(on ? den : 1.0f) : 0.0f;
  float gam;
  const float lg0 = log2_gamma(eta, lmi, eps_gamma, gam);
  const float lg = live ? lg0 : 0.0f;
  gam = live ? gam : 1.0f;
  float gi = lg;
  gi += row_shr<1>(gi);
  gi += row_shr<2>(gi);
  gi += row_shr<4>(gi);
  gi += row_shr<8>(gi);
  gi += gcarry;
  const float gsh = row_shr<1>(gi);
  const float gprev = li == 0 ? gcarry : gsh;
  const float glast = row_bcast<15>(gi);
  // earlier blocks, through w_s = e^{g_{16B-1}-g_s} rho_s
  const float qsv = m_qs[0], xsv = m_xs[0];
  float a = kReg ? eta * (sm.vb[cix(jl, i)] - exp2_fast(gprev) * xsv) : eta * sm.vb[cix(jl, i)];
  float o = exp2_fast(gi) * qsv;
  // operands and results of the earlier-block MFMAs, kept live (below) past
  // every inline-asm statement of the block
  bf16x8 m_a0 = {}, m_a1 = {}, m_k0 = {}, m_k1 = {}, m_p0 = {}, m_p1 = {};
  f32x4 ek4 = zero4(), ep4 = zero4();
  if constexpr (B > 0) {
    // the earlier blocks on the matrix cores, bf16 operands: D = W' KQ_B^T,
    // row a of W' the wave's own column 4 w + (a >> 2), so every component of
    // the lane's result row 4 g + r is EK[16B + li][4 w + g] (and EP likewise):
    // no value crosses to another wave.  W' rows beyond the solved blocks
    // meet zero Gram entries.
    const int l = 16 * g + li;
    const int ja = 4 * w + (li >> 2);
    m_a0 = frag_acc(ld4(&sm.w[cix(ja, 4 * g)]), ld4(&sm.w[cix(ja, 16 + 4 * g)]));
    if constexpr (kReg) {
      m_k0 = load_frag(&sm.kqf[B - 1][0][l * 8]);
      ek4 = mfma32(m_a0, m_k0, zero4());
    }
    m_p0 = load_frag(&sm.pqf[B - 1][0][l * 8]);
    ep4 = mfma32(m_a0, m_p0, zero4());
    if constexpr (B == 3) {
      m_a1 = frag_acc(ld4(&sm.w[cix(ja, 32 + 4 * g)]), ld4(&sm.w[cix(ja, 48 + 4 * g)]));
      if constexpr (kReg) {
        m_k1 = load_frag(&sm.kqf[2][1][l * 8]);
        ek4 = mfma32(m_a1, m_k1, ek4);
      }
      m_p1 = load_frag(&sm.pqf[2][1][l * 8]);
      ep4 = mfma32(m_a1, m_p1, ep4);
    }
    if constexpr (kReg) a -= eta * exp2_fast(gprev - gcarry) * ek4[0];
    o += exp2_fast(gi - gcarry) * ep4[0];
  }
  // in-block decays e^{g_{i-1}-g_s} = gamma_{s+1} ... gamma_{i-1} for
  // s = 16B + sl < i, as a suffix product over sl with gamma_{sl+1} taken from
  // lane sl + 1 by the DPP operand of the multiply; for s >= i - 1 the product
  // restarts at 1 (the Gram entries are 0 for s >= i, and every factor stays
  // in [0, 1]).  The leading s_nop covers the DPP read-after-write hazard on
  // gam.
  float ed[15];
  ed[14] = 1.0f;
#define FALCON_ED(SL, NOP)                                                                       \
  {                                                                                              \
    float p;                                                                                     \
    asm volatile(NOP "v_mul_f32_dpp %0, %1, %2 row_newbcast:" #SL " row_mask:0xf bank_mask:0xf" \
                 : "=v"(p) : "v"(gam), "v"(ed[SL]));                                             \
    ed[SL - 1] = (SL) < li ? p : 1.0f;                                                           \
  }
  FALCON_ED(14, "s_nop 1\n\t") FALCON_ED(13, "") FALCON_ED(12, "") FALCON_ED(11, "") FALCON_ED(10, "")
  FALCON_ED(9, "") FALCON_ED(8, "") FALCON_ED(7, "") FALCON_ED(6, "") FALCON_ED(5, "") FALCON_ED(4, "")
  FALCON_ED(3, "") FALCON_ED(2, "") FALCON_ED(1, "")
#undef FALCON_ED
  float kr[16], pr[16];
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4) {
    const f32x4 p4 = ld4(&sm.pqd[B][li][4 * s4]);
    pr[4 * s4] = p4[0]; pr[4 * s4 + 1] = p4[1]; pr[4 * s4 + 2] = p4[2]; pr[4 * s4 + 3] = p4[3];
    if constexpr (kReg) {
      const f32x4 k4 = ld4(&sm.kqd[B][li][4 * s4]);
      kr[4 * s4] = k4[0]; kr[4 * s4 + 1] = k4[1]; kr[4 * s4 + 2] = k4[2]; kr[4 * s4 + 3] = k4[3];
    }
  }
  if constexpr (kReg) {
    // forward substitution: after step sl, lane sl holds rho_{16B+sl}
    float nc[15];
#pragma unroll
    for (int sl = 0; sl < 15; ++sl) nc[sl] = -eta * ed[sl] * kr[sl];
    // a += a[lane SL] * nc[SL]: one multiply-add whose first source is read from
    // lane SL of the 16-lane row; the leading s_nop covers the DPP
    // read-after-write hazard on a
#define FALCON_SUB(SL)                                                                                \
  asm("s_nop 1\n\tv_fmac_f32_dpp %0, %0, %1 row_newbcast:" #SL " row_mask:0xf bank_mask:0xf" \
               : "+v"(a) : "v"(nc[SL]));
    FALCON_SUB(0) FALCON_SUB(1) FALCON_SUB(2) FALCON_SUB(3) FALCON_SUB(4) FALCON_SUB(5) FALCON_SUB(6)
    FALCON_SUB(7) FALCON_SUB(8) FALCON_SUB(9) FALCON_SUB(10) FALCON_SUB(11) FALCON_SUB(12) FALCON_SUB(13)
    FALCON_SUB(14)
#undef FALCON_SUB
  }
  const float rho = a;
  // in-block part of the read: e^{g_i-g_s} = gamma_i e^{g_{i-1}-g_s} for s < i
  // (the Gram entries are 0 for s >= i), and the diagonal term q_i.x_i rho_i
  {
    float o0 = 0.f, o1 = 0.f;
#define FALCON_RD(SL, ACC)                                                                              \
  {                                                                                                     \
    const float cf = ed[SL] * pr[SL];                                                                   \
    asm("s_nop 1\n\tv_fmac_f32_dpp %0, %1, %2 row_newbcast:" #SL " row_mask:0xf bank_mask:0xf" \
                 : "+v"(ACC) : "v"(rho), "v"(cf));                                                      \
  }
    FALCON_RD(0, o0) FALCON_RD(1, o1) FALCON_RD(2, o0) FALCON_RD(3, o1) FALCON_RD(4, o0) FALCON_RD(5, o1)
    FALCON_RD(6, o0) FALCON_RD(7, o1) FALCON_RD(8, o0) FALCON_RD(9, o1) FALCON_RD(10, o0) FALCON_RD(11, o1)
    FALCON_RD(12, o0) FALCON_RD(13, o1) FALCON_RD(14, o0)
#undef FALCON_RD
    o += exp2_fast(lg) * (o0 + o1) + sm.pd[i] * rho;
  }
  // The inline-asm DPP statements above write registers the compiler's
  // hazard checks cannot see.  With every operand and result register of the
  // MFMAs live until here, the allocator cannot give an asm output a register
  // an MFMA still reads or writes (unused result components would otherwise
  // be free to it).  The substitution and read statements depend on the MFMA
  // results, so they follow the compiler's wait for them and may be scheduled
  // freely (not volatile); the decay statements do not, so they stay
  // volatile and in place before this point.
  asm volatile("" ::"v"(m_a0), "v"(m_a1), "v"(m_k0), "v"(m_k1), "v"(m_p0), "v"(m_p1), "v"(ek4), "v"(ep4));
  asm volatile("" ::"v"(m_q0), "v"(m_q1), "v"(m_x0), "v"(m_x1), "v"(m_qs), "v"(m_xs), "v"(sa0), "v"(sa1));
  sm.ob[i][jl] = bf(o);
  // w to the end of this block: earlier entries decay by e^{g_last-g_carry},
  // this block's entries are e^{g_last-g_s} rho_s
  {
    const float blk = exp2_fast(glast - gcarry);
#pragma unroll
    for (int k = 0; k < B; ++k) sm.w[cix(jl, 16 * k + li)] *= blk;
    sm.w[cix(jl, i)] = exp2_fast(glast - gi) * rho;
  }
  gcarry = glast;
}

// Sequence and first value column of workgroup b: the four 16-column slices
// of a sequence are workgroups b, b + 8, b + 16, b + 24 (consecutive
// workgroups go to different XCDs, so the slices share one XCD and its L2).
// Shared by the kernel and the host-side bounds model.
__host__ __device__ inline void percol_slice(int b, int64_t& bh, int& j0) {
  bh = int64_t(b / 32) * 8 + b % 8;
  j0 = ((b / 8) & 3) * kSlice;
}

template <bool kReg>
__global__ void __launch_bounds__(kThreads, 2)
falcon2_chunked_kernel(const bf16_t* __restrict__ phi_k, const bf16_t* __restrict__ phi_q,
                       const bf16_t* __restrict__ v, const float* __restrict__ beta,
                       const float* __restrict__ lam, const float* S0,
                       const bf16_t* __restrict__ k_prev, bf16_t* __restrict__ o, float* S_T, int T,
                       int64_t BH, float eps, float eps_gamma) {
  __shared__ PcSmem sm;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;   // wave-uniform
  const int g = l >> 4, c16 = l & 15;
  const int jl = 4 * w + g, li = c16;                 // solve layout: column jl of the slice, block row li
  // the slices of a sequence share one XCD, so the keys and queries that
  // every slice reads come from HBM once
  int64_t bh;
  int j0;
  percol_slice(blockIdx.x, bh, j0);
  if (bh >= BH) return;
  const bool fresh = (k_prev == nullptr);
  const bf16_t* K = phi_k + bh * T * kD;
  const bf16_t* Q = phi_q + bh * T * kD;
  const bf16_t* V = v + bh * T * kD;
  const float* Bt = beta + bh * T * kD;
  const float* Lm = lam + bh * T;
  const bf16_t* kp = k_prev ? k_prev + bh * kD : nullptr;

  // wave w holds rows 16w..16w+15 of the slice's state: lane holds S[16w+4g+r][j0+c16]
  f32x4 S;
#pragma unroll
  for (int r = 0; r < 4; ++r) S[r] = S0 ? S0[(bh * kD + 16 * w + 4 * g + r) * kD + j0 + c16] : 0.0f;

  const int nchunks = (T + kC - 1) / kC;
  // the earlier-block products read whole columns of w, solved or not: start
  // them at zero (never NaN), later chunks leave finite values behind
  for (int e = tid; e < kSlice * kC; e += kThreads) sm.w[e] = 0.0f;

  // ---- products shared by all columns, on the matrix cores ------------------
  // Diagonal Gram and read block b in float32 (lane holds rows i = 16b+4g+r,
  // column s = 16b+c16; strict lower triangle, the diagonal to en and pd).
  auto diag = [&](const uint16_t* xb, const uint16_t* qb, int b) {
    const bf16x8 xs0 = ring_frag_c(xb, 16 * b + c16, 0, g), xs1 = ring_frag_c(xb, 16 * b + c16, 1, g);
    f32x4 dk = mfma32(xs0, xs0, zero4());
    dk = mfma32(xs1, xs1, dk);
    f32x4 dp = mfma32(ring_frag_c(qb, 16 * b + c16, 0, g), xs0, zero4());
    dp = mfma32(ring_frag_c(qb, 16 * b + c16, 1, g), xs1, dp);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool upper = c16 >= 4 * g + r;
      sm.kqd[b][4 * g + r][c16] = upper ? 0.0f : dk[r];
      sm.pqd[b][4 * g + r][c16] = upper ? 0.0f : dp[r];
      if (4 * g + r == c16) {
        sm.en[16 * b + c16] = dk[r];
        sm.pd[16 * b + c16] = dp[r];
      }
    }
  };
  // For the earlier-block sums, the fragments frag(KQ)[b][m], frag(PQ)[b][m]
  // of rows 16b.. over s < 16b, built from tiles T(sb, b) whose lane holds
  // x_{16sb+4g+r} . x_{16b+c16} (and the same with q_{16b+c16}); tiles with
  // sb >= b are zero.
  auto tile = [&](const uint16_t* xb, const uint16_t* qb, int sb, int b, f32x4& tk, f32x4& tp) {
    const bf16x8 a0 = ring_frag_c(xb, 16 * sb + c16, 0, g), a1 = ring_frag_c(xb, 16 * sb + c16, 1, g);
    tk = mfma32(a0, ring_frag_c(xb, 16 * b + c16, 0, g), zero4());
    tk = mfma32(a1, ring_frag_c(xb, 16 * b + c16, 1, g), tk);
    tp = mfma32(a0, ring_frag_c(qb, 16 * b + c16, 0, g), zero4());
    tp = mfma32(a1, ring_frag_c(qb, 16 * b + c16, 1, g), tp);
  };
  auto frags = [&](const uint16_t* xb, const uint16_t* qb, int b, int m, bool two) {
    f32x4 k0, p0, k1 = zero4(), p1 = zero4();
    tile(xb, qb, 2 * m, b, k0, p0);
    if (two) tile(xb, qb, 2 * m + 1, b, k1, p1);
    store_frag(&sm.kqf[b - 1][m][l * 8], frag_acc(k0, k1));
    store_frag(&sm.pqf[b - 1][m][l * 8], frag_acc(p0, p1));
  };
  // the wave's share of the fragments (four, six, eight and eight products)
  auto gram_frags = [&](const uint16_t* xb, const uint16_t* qb) {
    if (w == 0) frags(xb, qb, 3, 1, false);
    else if (w == 1) frags(xb, qb, 1, 0, false);
    else if (w == 2) frags(xb, qb, 2, 0, true);
    else frags(xb, qb, 3, 0, true);
  };
  // the state's bf16 copy, column by column, for the X S and Q S products
  auto put_state = [&]() { store_half(&sm.sb[c16][16 * w + 4 * g], S); };
  // rows 16w.. of the state: S <- e^{g_63} S + X^T W, X^T's rows from
  // products with a selection matrix
  auto state_update = [&](const uint16_t* xb) {
    const float dec = sm.e63[c16];
    // frag(W^T): lane holds w_{c16, 32m + kperm(g, e)}
    bf16x8 u[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) u[m] = frag_acc(ld4(&sm.w[cix(c16, 32 * m + 4 * g)]), ld4(&sm.w[cix(c16, 32 * m + 16 + 4 * g)]));
    const bf16x8 sel = select_frag(w & 1, g, c16);
    f32x4 d[4];
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) d[sb] = mfma32(ring_frag_c(xb, 16 * sb + c16, w >> 1, g), sel, zero4());
    f32x4 acc = S * dec;
    acc = mfma32(frag_acc(d[0], d[1]), u[0], acc);
    S = mfma32(frag_acc(d[2], d[3]), u[1], acc);
  };

  // Chunk c keeps its rows in buffer c & 1.  Per chunk: the solve (which
  // forms X S and Q S block by block from the bf16 state, and during which
  // the next chunk's rows are staged into the other buffer), then the
  // outputs, the state update and the next chunk's Gram products.  The next
  // chunk's rows are fetched into registers a chunk ahead.
  ChunkRegs R;
  fetch_chunk(R, K, Q, V, Bt, Lm, kp, T, 0, j0, tid);
  stage_xq(sm.x[0], sm.q[0], R, tid);
  stage_gates(sm, R, tid);
  put_state();
  if (nchunks > 1) fetch_chunk(R, K, Q, V, Bt, Lm, kp, T, kC, j0, tid);
  __syncthreads();
  diag(sm.x[0], sm.q[0], w);
  gram_frags(sm.x[0], sm.q[0]);
  __syncthreads();
  for (int c = 0; c < nchunks; ++c) {
    const int t0 = c * kC, buf = c & 1, nb = buf ^ 1;
    const bool more = c + 1 < nchunks;
    // ---- per-column rows, block by block ------------------------------------
    {
      // the state's columns 4w + (li >> 2) as A fragments of the X S, Q S products
      const bf16x8 sa0 = load_frag(&sm.sb[4 * w + (li >> 2)][8 * g]);
      const bf16x8 sa1 = load_frag(&sm.sb[4 * w + (li >> 2)][32 + 8 * g]);
      const uint16_t* xb = sm.x[buf];
      const uint16_t* qb = sm.q[buf];
      float gcarry = 0.f;
      solve_block<kReg, 0>(sm, xb, qb, sa0, sa1, w, jl, li, t0, T, fresh, eps, eps_gamma, gcarry);
      if (more) stage_xq(sm.x[nb], sm.q[nb], R, tid);
      solve_block<kReg, 1>(sm, xb, qb, sa0, sa1, w, jl, li, t0, T, fresh, eps, eps_gamma, gcarry);
      solve_block<kReg, 2>(sm, xb, qb, sa0, sa1, w, jl, li, t0, T, fresh, eps, eps_gamma, gcarry);
      solve_block<kReg, 3>(sm, xb, qb, sa0, sa1, w, jl, li, t0, T, fresh, eps, eps_gamma, gcarry);
      if (li == 0) sm.e63[jl] = exp2_fast(gcarry);
    }
    __syncthreads();
    // ---- outputs of the chunk (rows of the slice) -----------------------------
    if (tid < 2 * kC) {
      const int r = tid >> 1;
      if (t0 + r < T)
        *reinterpret_cast<uint4*>(o + (bh * T + t0 + r) * kD + j0 + 8 * (tid & 1)) =
            *reinterpret_cast<const uint4*>(&sm.ob[r][8 * (tid & 1)]);
    }
    if (more) {
      stage_gates(sm, R, tid);
      if (c + 2 < nchunks) fetch_chunk(R, K, Q, V, Bt, Lm, kp, T, t0 + 2 * kC, j0, tid);
    }
    // ---- state update, the next chunk's Gram products ------------------------
    state_update(sm.x[buf]);
    put_state();
    if (more) {
      diag(sm.x[nb], sm.q[nb], w);
      gram_frags(sm.x[nb], sm.q[nb]);
    }
    __syncthreads();
  }
  if (S_T) {
#pragma unroll
    for (int r = 0; r < 4; ++r) S_T[(bh * kD + 16 * w + 4 * g + r) * kD + j0 + c16] = S[r];
  }
}

}  // namespace

bool chunked_percol_applies(const ProblemArgs& a) {
  return a.bf16 && (a.variant == kF2 || a.variant == kF2A) && a.dk == kD && a.dv == kD && a.C == kC;
}

hipError_t launch_chunked_percol(const ProblemArgs& a, hipStream_t st) {
  const int64_t BH = int64_t(a.B) * a.H;
  const int64_t nwg = (BH + 7) / 8 * 8 * (kD / kSlice);
  if (kBoundsCheck) {
    // every (sequence, slice) exactly once, the slices of a sequence on one XCD;
    // chunk 0 is fetched before the chunk loop, so T > 0
    FALCON_HOST_CHECK(a.T > 0 && nwg <= INT32_MAX);
    std::vector<int> seen(size_t(BH) * (kD / kSlice), 0);
    for (int64_t b = 0; b < nwg; ++b) {
      int64_t bh;
      int j0;
      percol_slice(int(b), bh, j0);
      FALCON_HOST_CHECK(bh >= 0 && j0 >= 0 && j0 + kSlice <= kD && j0 % kSlice == 0);
      FALCON_HOST_CHECK(b % 8 == bh % 8);
      if (bh < BH) ++seen[size_t(bh) * (kD / kSlice) + j0 / kSlice];
    }
    for (int v : seen) FALCON_HOST_CHECK(v == 1);
  }
  const dim3 grid{unsigned(nwg)};
  if (a.variant == kF2)
    hipLaunchKernelGGL(falcon2_chunked_kernel<true>, grid, dim3(kThreads), 0, st,
                       static_cast<const bf16_t*>(a.phi_k), static_cast<const bf16_t*>(a.phi_q),
                       static_cast<const bf16_t*>(a.v), a.beta, a.lam, a.S0,
                       static_cast<const bf16_t*>(a.k_prev), static_cast<bf16_t*>(a.o), a.S_T, a.T, BH, a.eps,
                       a.eps_gamma);
  else
    hipLaunchKernelGGL(falcon2_chunked_kernel<false>, grid, dim3(kThreads), 0, st,
                       static_cast<const bf16_t*>(a.phi_k), static_cast<const bf16_t*>(a.phi_q),
                       static_cast<const bf16_t*>(a.v), a.beta, a.lam, a.S0,
                       static_cast<const bf16_t*>(a.k_prev), static_cast<bf16_t*>(a.o), a.S_T, a.T, BH, a.eps,
                       a.eps_gamma);
  return hipGetLastError();
}

}  // namespace falcon
