// Chunk-tile forward of Falcon-1A on MFMA (gfx950), bf16 I/O, dk = dv = 64,
// chunk C = 64, for sequences long enough to need many compute units each.
//
// Falcon-1A writes additively (Section 4.3: S_t = gamma_t S_{t-1} +
// eta_t x_t v_t^T), so a chunk's effect on the state does not depend on the
// state it meets:
//     S_{c+1} = e^{g_63} S_c + (Diag(e^{g_63 - g}) X)^T Diag(eta) V
//     O_c     = Diag(e^g) Q S_c + (tril0(Q X^T) o [e^{g_i - g_s}]) Diag(eta) V
// (the log-space renormalisation of Section 4.4 with window 1, applied per
// chunk).  A sequence is cut into tiles of kTileChunks chunks and the forward
// runs as three launches, none of which waits on another workgroup:
//   1. every tile (one wave each) sweeps its chunks from S = 0 and stores its
//      local state change ("aggregate") and its total log decay;
//   2. per sequence, an element-parallel scan over the tiles forms the state
//      at each tile's start, S_{t+1} = e^{L_t} S_t + aggregate_t, streaming
//      the aggregates (this is the only sequential step, and it is a
//      per-element multiply-add);
//   3. every tile sweeps its chunks again from its true start state, writing
//      the outputs.
// Aggregates and start states live in the workspace in "register order":
// entry ((fb * 4 + cb) * 64 + lane) * 4 + r holds S[16 fb + 4 g + r][16 cb + c16]
// with g = lane >> 4, c16 = lane & 15, so each wave moves them with 16-byte
// accesses.

#include "falcon_device.h"
#include "falcon_launch.h"
#include "falcon_mfma_frag.h"

namespace falcon {

namespace {

using namespace frag;

constexpr int kC = 64;
constexpr int kD = 64;
constexpr int kTileChunks = 8;
constexpr int kScanThreads = 256;   // a scan block covers 1024 state elements, 4 per thread
constexpr int kScanDepth = 8;       // tiles of aggregates in flight per scan thread
constexpr int kStateFloats = kD * kD;

// One staged chunk: key, query and value rows (swizzled) and its gates.
struct Stage {
  uint16_t x[kC * kD];            // keys phi(k_{t0+r-1})
  uint16_t q[kC * kD];            // queries phi(q_{t0+r})
  uint16_t v[kC * kD];            // values v_{t0+r}
  float graw[kC];                 // g_s, token order
  float sxh[kC];                  // e^{g_63 - g_s}
  float eta[kC];                  // eta_s
  float graw_t[kC];               // g_i at [c16 * 4 + ib] for i = 16 ib + c16
  float gexp_t[kC];               // e^{g_i}, same order
};

// Workspace: per tile its aggregate, its start state (both register order,
// 16 KiB each) and its total log decay.
struct ScanWorkspace {
  float* agg;
  float* start;
  float* logdecay;
};

struct ScanLayout {
  size_t off_start, off_logd, total;
  explicit ScanLayout(int64_t ntiles) {
    off_start = size_t(ntiles) * kStateFloats * 4;
    off_logd = 2 * off_start;
    total = off_logd + ((4 * size_t(ntiles) + 255) & ~size_t(255));
  }
};

struct Seq {
  const bf16_t* K;
  const bf16_t* Q;
  const bf16_t* V;
  const float* beta;
  const float* lam;
  const bf16_t* k_prev;
  int T;
};

// Rows t0 .. t0+63 of a [T, 64] matrix (clamped to T - 1) into a swizzled
// stage buffer.
__device__ __forceinline__ void stage_rows(uint16_t* dst, const bf16_t* src, int t0, int T, int l) {
  bf16x8 v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = 8 * j + (l >> 3);
    const int tok = t0 + r < T ? t0 + r : T - 1;
    v[j] = *reinterpret_cast<const bf16x8*>(src + int64_t(tok) * kD + 8 * (l & 7));
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = 8 * j + (l >> 3);
    *reinterpret_cast<bf16x8*>(dst + r * kD + 8 * seg_pos(r, l & 7)) = v[j];
  }
}

// Stages chunk c (all of it, or keys and values only) and its gates.  One
// wave: every LDS access is in program order, so no barrier is needed.
__device__ __forceinline__ float stage_chunk(Stage& st, const Seq& sq, int c, int l, bool with_q,
                                             float eps, float eps_gamma, bool fresh) {
  const int t0 = c * kC;
  const int T = sq.T;
  const int g = l >> 4, c16 = l & 15;
  // one matrix at a time: 8 coalesced 16-byte loads (8 whole rows each), then
  // their swizzled LDS writes; the key registers stay live for the gates
  bf16x8 x[8];
  const int tok = t0 + l < T ? t0 + l : T - 1;
  const float beta = sq.beta[tok], lam = sq.lam[tok];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = 8 * j + (l >> 3);
    const int kt = t0 + r - 1;
    const bf16_t* xs = kt < 0 ? (sq.k_prev ? sq.k_prev : sq.K) : sq.K + int64_t(kt < T ? kt : T - 1) * kD;
    x[j] = *reinterpret_cast<const bf16x8*>(xs + 8 * (l & 7));
  }
  stage_rows(st.v, sq.V, t0, T, l);
  if (with_q) stage_rows(st.q, sq.Q, t0, T, l);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = 8 * j + (l >> 3);
    *reinterpret_cast<bf16x8*>(st.x + r * kD + 8 * seg_pos(r, l & 7)) = x[j];
  }
  float eta, gi, gprev, glast;
  chunk_gates(x, beta, lam, t0 + l, T, eps, eps_gamma, fresh, l, eta, gi, gprev, glast);
  st.graw[l] = gi;
  st.sxh[l] = __expf(glast - gi);
  st.eta[l] = eta;
  st.graw_t[c16 * 4 + g] = gi;
  st.gexp_t[c16 * 4 + g] = __expf(gi);
  return glast;
}

// The rows of one chunk held in registers (coalesced loads: 8 whole rows per
// instruction), so the next chunk's loads can be in flight while the current
// one is computed.
struct ChunkRegs {
  bf16x8 x[8], q[8], v[8];
  float beta, lam;
};

__device__ __forceinline__ void fetch_chunk(ChunkRegs& R, const Seq& sq, int c, int l) {
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
    R.v[j] = *reinterpret_cast<const bf16x8*>(sq.V + int64_t(tok) * kD + 8 * (l & 7));
  }
  const int tok = t0 + l < T ? t0 + l : T - 1;
  R.beta = sq.beta[tok];
  R.lam = sq.lam[tok];
}

// Writes fetched rows into the stage and derives the chunk's gates; returns g_63.
__device__ __forceinline__ float commit_chunk(Stage& st, const ChunkRegs& R, int c, int T, int l,
                                              float eps, float eps_gamma, bool fresh) {
  const int g = l >> 4, c16 = l & 15;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = 8 * j + (l >> 3);
    const int off = r * kD + 8 * seg_pos(r, l & 7);
    *reinterpret_cast<bf16x8*>(st.x + off) = R.x[j];
    *reinterpret_cast<bf16x8*>(st.q + off) = R.q[j];
    *reinterpret_cast<bf16x8*>(st.v + off) = R.v[j];
  }
  float eta, gi, gprev, glast;
  chunk_gates(R.x, R.beta, R.lam, c * kC + l, T, eps, eps_gamma, fresh, l, eta, gi, gprev, glast);
  st.graw[l] = gi;
  st.sxh[l] = __expf(glast - gi);
  st.eta[l] = eta;
  st.graw_t[c16 * 4 + g] = gi;
  st.gexp_t[c16 * 4 + g] = __expf(gi);
  return glast;
}

// Diag(eta) V for value block cb, as fragments over tokens (k) with lane
// column = value column 16 cb + c16: B operand of the state update, A
// operand of the intra-chunk read.
__device__ __forceinline__ void value_frags(const Stage& st, int cb, int g, int c16, bf16x8 (&vt)[2]) {
  const bf16x8 sel = select_frag(cb & 1, g, c16);
  f32x4 d[4];
#pragma unroll
  for (int sb = 0; sb < 4; ++sb)
    d[sb] = mfma32(ring_frag_c(st.v, 16 * sb + c16, cb >> 1, g), sel, zero4());   // V[16sb+4g+r][16cb+c16]
#pragma unroll
  for (int m = 0; m < 2; ++m)
    vt[m] = frag_acc(d[2 * m] * ld4(&st.eta[32 * m + 4 * g]), d[2 * m + 1] * ld4(&st.eta[32 * m + 16 + 4 * g]));
}

// (Diag(e^{g_63-g}) X)^T for key block fb: A operand, lane row = feature.
__device__ __forceinline__ void key_frags(const Stage& st, int fb, int g, int c16, bf16x8 (&xh)[2]) {
  const bf16x8 sel = select_frag(fb & 1, g, c16);
  f32x4 d[4];
#pragma unroll
  for (int sb = 0; sb < 4; ++sb)
    d[sb] = mfma32(ring_frag_c(st.x, 16 * sb + c16, fb >> 1, g), sel, zero4());   // X[16sb+4g+r][16fb+c16]
#pragma unroll
  for (int m = 0; m < 2; ++m)
    xh[m] = frag_acc(d[2 * m] * ld4(&st.sxh[32 * m + 4 * g]), d[2 * m + 1] * ld4(&st.sxh[32 * m + 16 + 4 * g]));
}

// Value block cb of S <- e^{g_63} S + (Diag(e^{g_63-g}) X)^T Diag(eta) V;
// S[fb][cb] holds S[16fb+4g+r][16cb+c16].
__device__ __forceinline__ void state_update_cb(f32x4 (&S)[4][4], int cb, const bf16x8 (&xh)[4][2],
                                                const bf16x8 (&vt)[2], float decay) {
#pragma unroll
  for (int fb = 0; fb < 4; ++fb) {
    f32x4 acc = S[fb][cb] * decay;
    acc = mfma32(xh[fb][0], vt[0], acc);
    S[fb][cb] = mfma32(xh[fb][1], vt[1], acc);
  }
}

__device__ __forceinline__ void store_state(float* dst, const f32x4 (&S)[4][4], int l) {
#pragma unroll
  for (int fb = 0; fb < 4; ++fb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
      *reinterpret_cast<f32x4*>(dst + ((fb * 4 + cb) * 64 + l) * 4) = S[fb][cb];
}

struct TileArgs {
  const bf16_t* phi_k;
  const bf16_t* phi_q;
  const bf16_t* v;
  const float* beta;
  const float* lam;
  const bf16_t* k_prev;
  bf16_t* o;
  int T, ntiles_seq;
  float eps, eps_gamma;
};

__device__ __forceinline__ Seq seq_of(const TileArgs& a, int64_t bh) {
  Seq sq;
  sq.K = a.phi_k + bh * a.T * kD;
  sq.Q = a.phi_q + bh * a.T * kD;
  sq.V = a.v + bh * a.T * kD;
  sq.beta = a.beta + bh * a.T;
  sq.lam = a.lam + bh * a.T;
  sq.k_prev = a.k_prev ? a.k_prev + bh * kD : nullptr;
  sq.T = a.T;
  return sq;
}

// Stage reached through an opaque offset, so that LDS addresses are rebuilt
// every chunk instead of being hoisted (and spilled) across the chunk loop.
__device__ __forceinline__ Stage& opaque(Stage& st) {
  int zero = 0;
  asm volatile("" : "+v"(zero));
  return *reinterpret_cast<Stage*>(reinterpret_cast<char*>(&st) + zero);
}

// ---- launch 1: tile aggregates ------------------------------------------------
__global__ void __launch_bounds__(64, 2)
falcon1a_tile_agg_kernel(TileArgs a, ScanWorkspace ws) {
  __shared__ Stage st_;
  const int l = threadIdx.x;
  const int g = l >> 4, c16 = l & 15;
  const int t = blockIdx.x;                       // tile t of sequence t / ntiles_seq
  const int64_t bh = t / a.ntiles_seq;
  const int tile = t % a.ntiles_seq;
  const int nchunks = (a.T + kC - 1) / kC;
  const int c0 = tile * kTileChunks;
  const int c1 = c0 + kTileChunks < nchunks ? c0 + kTileChunks : nchunks;
  const Seq sq = seq_of(a, bh);
  const bool fresh = (a.k_prev == nullptr);
  f32x4 S[4][4];
#pragma unroll
  for (int fb = 0; fb < 4; ++fb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) S[fb][cb] = zero4();
  float logd = 0.f;
  for (int c = c0; c < c1; ++c) {
    Stage& st = opaque(st_);
    const float glast = stage_chunk(st, sq, c, l, false, a.eps, a.eps_gamma, fresh);
    const float decay = __expf(glast);
    bf16x8 xh[4][2];
#pragma unroll
    for (int fb = 0; fb < 4; ++fb) key_frags(st, fb, g, c16, xh[fb]);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      bf16x8 vt[2];
      value_frags(st, cb, g, c16, vt);
      state_update_cb(S, cb, xh, vt, decay);
    }
    logd += glast;
  }
  store_state(ws.agg + int64_t(t) * kStateFloats, S, l);
  if (l == 0) ws.logdecay[t] = logd;
}

// ---- launch 2: start state of every tile -------------------------------------
// Block (bh, part): state elements [part * 1024, part * 1024 + 1024) of
// sequence bh in register order, 4 per thread.  S_T is written in [dk][dv].
__global__ void __launch_bounds__(kScanThreads)
falcon1a_tile_scan_kernel(const float* S0, float* S_T, int ntiles_seq, ScanWorkspace ws) {
  const int64_t bh = blockIdx.x / 4;
  const int e0 = ((blockIdx.x & 3) * kScanThreads + threadIdx.x) * 4;   // register-order index
  const int lane = (e0 >> 2) & 63, tcb = e0 >> 8;                      // tile (fb * 4 + cb)
  const int fb = tcb >> 2, cb = tcb & 3, g = lane >> 4, c16 = lane & 15;
  f32x4 s = zero4();
  if (S0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) s[r] = S0[(bh * kD + 16 * fb + 4 * g + r) * kD + 16 * cb + c16];
  }
  // aggregates are streamed kScanDepth tiles at a time, the next group's
  // loads in flight while the current group is folded in
  const int64_t t0 = bh * ntiles_seq;
  f32x4 cur[kScanDepth], nxt[kScanDepth];
  float lcur[kScanDepth], lnxt[kScanDepth];
  auto fetch = [&](int base, f32x4 (&dst)[kScanDepth], float (&ld)[kScanDepth]) {
#pragma unroll
    for (int k = 0; k < kScanDepth; ++k) {
      const int tile = base + k < ntiles_seq ? base + k : ntiles_seq - 1;
      dst[k] = *reinterpret_cast<const f32x4*>(ws.agg + (t0 + tile) * kStateFloats + e0);
      ld[k] = ws.logdecay[t0 + tile];
    }
  };
  fetch(0, cur, lcur);
  for (int base = 0; base < ntiles_seq; base += kScanDepth) {
    if (base + kScanDepth < ntiles_seq) fetch(base + kScanDepth, nxt, lnxt);
#pragma unroll
    for (int k = 0; k < kScanDepth; ++k) {
      if (base + k < ntiles_seq) {
        *reinterpret_cast<f32x4*>(ws.start + (t0 + base + k) * kStateFloats + e0) = s;
        s = s * __expf(lcur[k]) + cur[k];
      }
    }
#pragma unroll
    for (int k = 0; k < kScanDepth; ++k) {
      cur[k] = nxt[k];
      lcur[k] = lnxt[k];
    }
  }
  if (S_T) {
#pragma unroll
    for (int r = 0; r < 4; ++r) S_T[(bh * kD + 16 * fb + 4 * g + r) * kD + 16 * cb + c16] = s[r];
  }
}

// ---- launch 3: outputs from each tile's start state --------------------------
__global__ void __launch_bounds__(64)
falcon1a_tile_out_kernel(TileArgs a, ScanWorkspace ws) {
  __shared__ Stage st_;
  const int l = threadIdx.x;
  const int g = l >> 4, c16 = l & 15;
  const int t = blockIdx.x;
  const int64_t bh = t / a.ntiles_seq;
  const int tile = t % a.ntiles_seq;
  const int nchunks = (a.T + kC - 1) / kC;
  const int c0 = tile * kTileChunks;
  const int c1 = c0 + kTileChunks < nchunks ? c0 + kTileChunks : nchunks;
  const Seq sq = seq_of(a, bh);
  const bool fresh = (a.k_prev == nullptr);
  const int T = a.T;
  f32x4 S[4][4];
  {
    const float* src = ws.start + int64_t(t) * kStateFloats;
#pragma unroll
    for (int fb = 0; fb < 4; ++fb)
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) S[fb][cb] = *reinterpret_cast<const f32x4*>(src + ((fb * 4 + cb) * 64 + l) * 4);
  }
  bf16_t* o_bh = a.o + bh * T * kD;
  ChunkRegs R;
  fetch_chunk(R, sq, c0, l);
  for (int c = c0; c < c1; ++c) {
    Stage& st = opaque(st_);
    const float glast = commit_chunk(st, R, c, T, l, a.eps, a.eps_gamma, fresh);
    if (c + 1 < c1) fetch_chunk(R, sq, c + 1, l);
    const float decay = __expf(glast);
    const int t0 = c * kC;
    // decayed read mask M^T tile (sb, ib) = X_sb Q_ib^T, s <= i, as B fragments
    bf16x8 mfr[4][2];
    {
      const f32x4 gra_i = ld4(&st.graw_t[c16 * 4]);
#pragma unroll
      for (int ib = 0; ib < 4; ++ib) {
        f32x4 mt[4];
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) {
          mt[sb] = zero4();
          if (sb > ib) continue;
          f32x4 acc = mfma32(ring_frag_c(st.x, 16 * sb + c16, 0, g), ring_frag_c(st.q, 16 * ib + c16, 0, g), zero4());
          acc = mfma32(ring_frag_c(st.x, 16 * sb + c16, 1, g), ring_frag_c(st.q, 16 * ib + c16, 1, g), acc);
          const f32x4 gs = ld4(&st.graw[16 * sb + 4 * g]);
          const int i = 16 * ib + c16;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int s_ = 16 * sb + 4 * g + r;
            mt[sb][r] = s_ <= i ? __expf(gra_i[ib] - gs[r]) * acc[r] : 0.0f;
          }
        }
        mfr[ib][0] = frag_acc(mt[0], mt[1]);
        mfr[ib][1] = frag_acc(mt[2], mt[3]);
      }
    }
    bf16x8 xh[4][2];
#pragma unroll
    for (int fb = 0; fb < 4; ++fb) key_frags(st, fb, g, c16, xh[fb]);
    const f32x4 gexp_i = ld4(&st.gexp_t[c16 * 4]);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      bf16x8 vt[2];
      value_frags(st, cb, g, c16, vt);
      // O^T tiles of value block cb: e^{g_i} S^T Q^T + (Diag(eta) V)^T M^T;
      // lane holds o[t0+16ib+c16][16cb+4g+r]
      const bf16x8 s0 = frag_acc(S[0][cb], S[1][cb]);
      const bf16x8 s1 = frag_acc(S[2][cb], S[3][cb]);
#pragma unroll
      for (int ib = 0; ib < 4; ++ib) {
        const int i = 16 * ib + c16;
        f32x4 acc = mfma32(s0, ring_frag_p(st.q, i, 0, g), zero4());
        acc = mfma32(s1, ring_frag_p(st.q, i, 1, g), acc);
        acc = acc * gexp_i[ib];
        acc = mfma32(vt[0], mfr[ib][0], acc);
        if (ib >= 2) acc = mfma32(vt[1], mfr[ib][1], acc);
        const int tok = t0 + i;
        if (tok < T)
          *reinterpret_cast<uint2*>(o_bh + int64_t(tok) * kD + 16 * cb + 4 * g) =
              make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
      }
      state_update_cb(S, cb, xh, vt, decay);
    }
  }
}

int64_t scan_tiles_per_seq(const ProblemArgs& a) {
  const int64_t nchunks = (int64_t(a.T) + kC - 1) / kC;
  return (nchunks + kTileChunks - 1) / kTileChunks;
}

}  // namespace

bool chunked_scan_applies(const ProblemArgs& a) {
  return a.bf16 && a.variant == kF1A && a.dk == kD && a.dv == kD && a.C == kC && a.T > 0;
}

size_t chunked_scan_workspace_bytes(const ProblemArgs& a) {
  return ScanLayout(int64_t(a.B) * a.H * scan_tiles_per_seq(a)).total;
}

hipError_t launch_chunked_scan(const ProblemArgs& a, hipStream_t st) {
  const int64_t BH = int64_t(a.B) * a.H;
  const int64_t nts = scan_tiles_per_seq(a);
  const int64_t ntiles = BH * nts;
  if (ntiles == 0) return hipSuccess;
  const ScanLayout L(ntiles);
  char* base = static_cast<char*>(a.workspace);
  ScanWorkspace ws;
  ws.agg = reinterpret_cast<float*>(base);
  ws.start = reinterpret_cast<float*>(base + L.off_start);
  ws.logdecay = reinterpret_cast<float*>(base + L.off_logd);
  TileArgs ta;
  ta.phi_k = static_cast<const bf16_t*>(a.phi_k);
  ta.phi_q = static_cast<const bf16_t*>(a.phi_q);
  ta.v = static_cast<const bf16_t*>(a.v);
  ta.beta = a.beta;
  ta.lam = a.lam;
  ta.k_prev = static_cast<const bf16_t*>(a.k_prev);
  ta.o = static_cast<bf16_t*>(a.o);
  ta.T = a.T;
  ta.ntiles_seq = int(nts);
  ta.eps = a.eps;
  ta.eps_gamma = a.eps_gamma;
  hipLaunchKernelGGL(falcon1a_tile_agg_kernel, dim3(unsigned(ntiles)), dim3(64), 0, st, ta, ws);
  hipLaunchKernelGGL(falcon1a_tile_scan_kernel, dim3(unsigned(BH * 4)), dim3(kScanThreads), 0, st, a.S0,
                     a.S_T, int(nts), ws);
  hipLaunchKernelGGL(falcon1a_tile_out_kernel, dim3(unsigned(ntiles)), dim3(64), 0, st, ta, ws);
  return hipGetLastError();
}

}  // namespace falcon
