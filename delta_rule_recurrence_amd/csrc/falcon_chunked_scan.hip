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
//   1. every tile sweeps its chunks from S = 0 and stores its local state
//      change ("aggregate") and its total log decay;
//   2. per sequence, an element-parallel scan over the tiles forms the state
//      at each tile's start, S_{t+1} = e^{L_t} S_t + aggregate_t, streaming
//      the aggregates (this is the only sequential step, and it is a
//      per-element multiply-add);
//   3. every tile sweeps its chunks again from its true start state, writing
//      the outputs.
// A tile is one workgroup of four waves; wave w owns value block w (16
// columns) of the state and of the outputs.  Per chunk, wave 0 derives the
// gates while every wave forms its share of the raw transposes and of the read
// mask; the scaled key fragments and mask rows are exchanged through LDS.
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
constexpr int kScanThreads = 256;   // a scan block covers 256 state elements, one per thread
constexpr int kScanBlocks = 16;     // scan blocks per sequence (4096 state elements)
constexpr int kScanDepth = 32;      // tiles of aggregates in flight per scan thread
constexpr int kStateFloats = kD * kD;

constexpr int kTileThreads = 256;   // four waves per tile

// One staged chunk, the chunk's gates, and the fragments the waves exchange.
// The aggregate pass needs no queries and no read mask.
template <bool kOut>
struct TileSmem {
  uint16_t x[kC * kD];            // keys phi(k_{t0+r-1}), swizzled rows
  uint16_t q[kOut ? kC * kD : 8]; // queries phi(q_{t0+r}), swizzled rows
  uint16_t v[kC * kD];            // values v_{t0+r}, swizzled rows
  uint16_t xh[4 * 2 * 64 * 8];    // frag((Diag(e^{g_63-g}) X)^T)[fb][m]
  uint16_t mf[kOut ? 4 * 2 * 64 * 8 : 8];   // frag(M)[ib][m], M = tril0(Q X^T) o [e^{g_i-g_s}]
  float graw[kC];                 // g_s, token order
  float sxh[kC];                  // e^{g_63 - g_s}
  float eta[kC];                  // eta_s
  float graw_t[kC];               // g_i at [c16 * 4 + ib] for i = 16 ib + c16
  float gexp_t[kC];               // e^{g_i}, same order
  float glast;                    // g_63
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

// This wave's rows (16 w .. 16 w + 15) of the next chunk, held in registers
// so their loads are in flight while the current chunk is computed.
struct WaveRows {
  bf16x8 x[2], q[2], v[2];
  float beta, lam;                // wave 0: gates of token c * 64 + lane
};

__device__ __forceinline__ void fetch_rows(WaveRows& R, const Seq& sq, int c, int w, int l, bool with_q) {
  const int t0 = c * kC;
  const int T = sq.T;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = 16 * w + 8 * j + (l >> 3);
    const int kt = t0 + r - 1;
    const bf16_t* xs = kt < 0 ? (sq.k_prev ? sq.k_prev : sq.K) : sq.K + int64_t(kt < T ? kt : T - 1) * kD;
    const int tok = t0 + r < T ? t0 + r : T - 1;
    R.x[j] = *reinterpret_cast<const bf16x8*>(xs + 8 * (l & 7));
    R.v[j] = *reinterpret_cast<const bf16x8*>(sq.V + int64_t(tok) * kD + 8 * (l & 7));
    if (with_q) R.q[j] = *reinterpret_cast<const bf16x8*>(sq.Q + int64_t(tok) * kD + 8 * (l & 7));
  }
  if (w == 0) {
    const int tok = t0 + l < T ? t0 + l : T - 1;
    R.beta = sq.beta[tok];
    R.lam = sq.lam[tok];
  }
}

template <bool kOut>
__device__ __forceinline__ void commit_rows(TileSmem<kOut>& sm, const WaveRows& R, int w, int l) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = 16 * w + 8 * j + (l >> 3);
    const int off = r * kD + 8 * seg_pos(r, l & 7);
    *reinterpret_cast<bf16x8*>(sm.x + off) = R.x[j];
    *reinterpret_cast<bf16x8*>(sm.v + off) = R.v[j];
    if constexpr (kOut) *reinterpret_cast<bf16x8*>(sm.q + off) = R.q[j];
  }
}

// Fragment slot [b][m] of a 64x64 fragment array.
__device__ __forceinline__ int fslot(int b, int m, int l) { return ((b * 2 + m) * 64 + l) * 8; }

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

// One chunk of a tile for wave w (value block w).  R holds the chunk's rows on
// entry; after they are in LDS, chunk c_next (if < c_end) is fetched into R.
template <bool kOut>
__device__ __forceinline__ void tile_chunk(TileSmem<kOut>& sm, WaveRows& R, const Seq& sq, const TileArgs& a,
                                           int c, int c_next, int c_end, int w, int l, bool fresh, f32x4 (&S)[4],
                                           float& logd, bf16_t* o_bh) {
  const int g = l >> 4, c16 = l & 15;
  const int cb = w;
  const int T = a.T;
  commit_rows<kOut>(sm, R, w, l);
  const float beta = R.beta, lam = R.lam;
  __syncthreads();
  if (c_next < c_end) fetch_rows(R, sq, c_next, w, l, kOut);
  // ---- gates (wave 0); raw key block fb = w, value block cb = w, mask rows ib = w
  if (w == 0) {
    float eta, gi, gprev, glast;
    chunk_gates(sm.x, beta, lam, c * kC + l, T, a.eps, a.eps_gamma, fresh, l, eta, gi, gprev, glast);
    sm.graw[l] = gi;
    sm.sxh[l] = __expf(glast - gi);
    sm.eta[l] = eta;
    sm.graw_t[c16 * 4 + g] = gi;
    sm.gexp_t[c16 * 4 + g] = __expf(gi);
    if (l == 0) sm.glast = glast;
  }
  f32x4 dx[4], dv[4];                             // X[16sb+4g+r][16w+c16], V[16sb+4g+r][16w+c16]
  {
    const bf16x8 sel = select_frag(w & 1, g, c16);
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) {
      dx[sb] = mfma32(ring_frag_c(sm.x, 16 * sb + c16, w >> 1, g), sel, zero4());
      dv[sb] = mfma32(ring_frag_c(sm.v, 16 * sb + c16, w >> 1, g), sel, zero4());
    }
  }
  f32x4 mt[4];                                    // (Q X^T)[16w+c16][16sb+4g+r] for sb <= w
#pragma unroll
  for (int sb = 0; sb < 4; ++sb) {
    mt[sb] = zero4();
    if constexpr (kOut) {
      if (sb <= w) {
        f32x4 acc = mfma32(ring_frag_c(sm.x, 16 * sb + c16, 0, g), ring_frag_c(sm.q, 16 * w + c16, 0, g), zero4());
        mt[sb] = mfma32(ring_frag_c(sm.x, 16 * sb + c16, 1, g), ring_frag_c(sm.q, 16 * w + c16, 1, g), acc);
      }
    }
  }
  __syncthreads();                                // gates ready
  // ---- scale: Xh^T block w and mask rows w to LDS, Diag(eta) V^T block w kept
  bf16x8 vt[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    vt[m] = frag_acc(dv[2 * m] * ld4(&sm.eta[32 * m + 4 * g]), dv[2 * m + 1] * ld4(&sm.eta[32 * m + 16 + 4 * g]));
    store_frag(&sm.xh[fslot(w, m, l)],
               frag_acc(dx[2 * m] * ld4(&sm.sxh[32 * m + 4 * g]), dx[2 * m + 1] * ld4(&sm.sxh[32 * m + 16 + 4 * g])));
  }
  if constexpr (kOut) {
    const int i = 16 * w + c16;
    const float gi = sm.graw[i];
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) {
      const f32x4 gs = ld4(&sm.graw[16 * sb + 4 * g]);
#pragma unroll
      for (int r = 0; r < 4; ++r) mt[sb][r] = 16 * sb + 4 * g + r <= i ? __expf(gi - gs[r]) * mt[sb][r] : 0.0f;
    }
    store_frag(&sm.mf[fslot(w, 0, l)], frag_acc(mt[0], mt[1]));
    store_frag(&sm.mf[fslot(w, 1, l)], frag_acc(mt[2], mt[3]));
  }
  const float e63 = __expf(sm.glast);
  if (w == 0) logd += sm.glast;
  __syncthreads();                                // key fragments and mask complete
  if constexpr (kOut) {
    // O^T tiles of value block cb: e^{g_i} S^T Q^T + (Diag(eta) V)^T M^T;
    // lane holds o[t0+16ib+c16][16cb+4g+r]
    const f32x4 gexp_i = ld4(&sm.gexp_t[c16 * 4]);
    const bf16x8 s0 = frag_acc(S[0], S[1]);
    const bf16x8 s1 = frag_acc(S[2], S[3]);
    const int t0 = c * kC;
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) {
      const int i = 16 * ib + c16;
      f32x4 acc = mfma32(s0, ring_frag_p(sm.q, i, 0, g), zero4());
      acc = mfma32(s1, ring_frag_p(sm.q, i, 1, g), acc);
      acc = acc * gexp_i[ib];
      acc = mfma32(vt[0], load_frag(&sm.mf[fslot(ib, 0, l)]), acc);
      if (ib >= 2) acc = mfma32(vt[1], load_frag(&sm.mf[fslot(ib, 1, l)]), acc);
      const int tok = t0 + i;
      if (tok < T)
        *reinterpret_cast<uint2*>(o_bh + int64_t(tok) * kD + 16 * cb + 4 * g) =
            make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
    }
  }
  // S <- e^{g_63} S + (Diag(e^{g_63-g}) X)^T Diag(eta) V for value block cb
  // (the key fragments are read after the outputs, so fewer registers are live)
#pragma unroll
  for (int fb = 0; fb < 4; ++fb) {
    f32x4 acc = S[fb] * e63;
    acc = mfma32(load_frag(&sm.xh[fslot(fb, 0, l)]), vt[0], acc);
    S[fb] = mfma32(load_frag(&sm.xh[fslot(fb, 1, l)]), vt[1], acc);
  }
  __syncthreads();                                // the stage is free for the next chunk
}

// ---- launches 1 and 3: a tile's chunks, four waves --------------------------
// kOut = false: sweep from S = 0 and store the tile's aggregate and log decay.
// kOut = true: sweep from the tile's start state and write the outputs.
// Each wave fetches its rows of the next chunk while the current one is
// computed.
template <bool kOut>
__global__ void __launch_bounds__(kTileThreads) __attribute__((amdgpu_waves_per_eu(kOut ? 3 : 4)))
falcon1a_tile_kernel(TileArgs a, ScanWorkspace ws) {
  __shared__ TileSmem<kOut> sm;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;   // wave-uniform
  const int cb = w;                               // value block of this wave
  const int t = blockIdx.x;                       // tile t of sequence t / ntiles_seq
  const int64_t bh = t / a.ntiles_seq;
  const int tile = t % a.ntiles_seq;
  const int nchunks = (a.T + kC - 1) / kC;
  const int c0 = tile * kTileChunks;
  const int c1 = c0 + kTileChunks < nchunks ? c0 + kTileChunks : nchunks;
  const Seq sq = seq_of(a, bh);
  const bool fresh = (a.k_prev == nullptr);
  // S[fb]: lane holds S[16fb+4g+r][16cb+c16]
  f32x4 S[4];
#pragma unroll
  for (int fb = 0; fb < 4; ++fb)
    S[fb] = kOut ? *reinterpret_cast<const f32x4*>(ws.start + int64_t(t) * kStateFloats + ((fb * 4 + cb) * 64 + l) * 4)
                 : zero4();
  bf16_t* o_bh = a.o + bh * a.T * kD;
  float logd = 0.f;
  WaveRows R;
  fetch_rows(R, sq, c0, w, l, kOut);
  for (int c = c0; c < c1; ++c) tile_chunk<kOut>(sm, R, sq, a, c, c + 1, c1, w, l, fresh, S, logd, o_bh);
  if (!kOut) {
#pragma unroll
    for (int fb = 0; fb < 4; ++fb)
      *reinterpret_cast<f32x4*>(ws.agg + int64_t(t) * kStateFloats + ((fb * 4 + cb) * 64 + l) * 4) = S[fb];
    if (w == 0 && l == 0) ws.logdecay[t] = logd;
  }
}

// ---- launch 2: start state of every tile -------------------------------------
// Block (bh, part): state elements [part * 256, part * 256 + 256) of sequence
// bh in register order, one per thread (consecutive threads, consecutive
// addresses); up to kScanDepth tiles' aggregates are loaded before they are
// folded, so a sequence of that many tiles costs one round trip to memory.
// S_T is written in [dk][dv].
__global__ void __launch_bounds__(kScanThreads)
falcon1a_tile_scan_kernel(const float* S0, float* S_T, int ntiles_seq, ScanWorkspace ws) {
  const int64_t bh = blockIdx.x / kScanBlocks;
  const int e = (blockIdx.x % kScanBlocks) * kScanThreads + threadIdx.x;   // register-order index
  const int r = e & 3, lane = (e >> 2) & 63, tcb = e >> 8;                   // tile (fb * 4 + cb)
  const int fb = tcb >> 2, cb = tcb & 3, g = lane >> 4, c16 = lane & 15;
  const int64_t sidx = (bh * kD + 16 * fb + 4 * g + r) * kD + 16 * cb + c16;
  float s = S0 ? S0[sidx] : 0.0f;
  const int64_t t0 = bh * ntiles_seq;
  for (int base = 0; base < ntiles_seq; base += kScanDepth) {
    float ag[kScanDepth], ld[kScanDepth];
#pragma unroll
    for (int k = 0; k < kScanDepth; ++k) {
      const int tile = base + k < ntiles_seq ? base + k : ntiles_seq - 1;
      ag[k] = ws.agg[(t0 + tile) * kStateFloats + e];
      ld[k] = ws.logdecay[t0 + tile];
    }
#pragma unroll
    for (int k = 0; k < kScanDepth; ++k) {
      if (base + k < ntiles_seq) {
        ws.start[(t0 + base + k) * kStateFloats + e] = s;
        s = s * __expf(ld[k]) + ag[k];
      }
    }
  }
  if (S_T) S_T[sidx] = s;
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
  // the tiles of a sequence cover its chunks exactly; the grids and the
  // workspace hold every tile
  FALCON_HOST_CHECK(ntiles <= INT32_MAX && BH * kScanBlocks <= INT32_MAX);
  FALCON_HOST_CHECK(kScanBlocks * kScanThreads == kStateFloats);
  FALCON_HOST_CHECK(a.workspace_bytes >= L.total);
  FALCON_HOST_CHECK((nts - 1) * kTileChunks < (int64_t(a.T) + kC - 1) / kC &&
                    nts * kTileChunks >= (int64_t(a.T) + kC - 1) / kC);
  FALCON_HOST_CHECK(L.off_start >= size_t(ntiles) * kStateFloats * 4 && L.off_logd >= 2 * L.off_start &&
                    L.total >= L.off_logd + 4 * size_t(ntiles));
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
  hipLaunchKernelGGL(falcon1a_tile_kernel<false>, dim3(unsigned(ntiles)), dim3(kTileThreads), 0, st, ta, ws);
  hipLaunchKernelGGL(falcon1a_tile_scan_kernel, dim3(unsigned(BH * kScanBlocks)), dim3(kScanThreads), 0, st, a.S0,
                     a.S_T, int(nts), ws);
  hipLaunchKernelGGL(falcon1a_tile_kernel<true>, dim3(unsigned(ntiles)), dim3(kTileThreads), 0, st, ta, ws);
  return hipGetLastError();
}

}  // namespace falcon
