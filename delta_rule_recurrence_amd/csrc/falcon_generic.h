// General-shape chunked forward: the LDS layout shared by the host (tile
// choice) and the kernel, and the per-chunk-size launch, whose definition is
// in falcon_generic_kernel.h and whose instantiations are in
// falcon_chunked_generic_c16/c32/c64.hip.
#pragma once

#include "falcon_launch.h"

namespace falcon {

constexpr int kGenericThreads = 256;

struct GenericLayout {
  int C, dk, nv, ng;   // chunk, key width, value tile, gate columns (1 or nv)
  int xp, pp, sp;      // row pitches of X, Q (dk + 4), of P, G (C + 4) and of S^T (dk + 4)
  int off_x, off_q, off_p, off_g, off_r, off_s, off_eta, off_lg, off_en, off_lm, off_y, total;
  __host__ __device__ GenericLayout(int C_, int dk_, int nv_, int ng_, bool reg)
      : C(C_), dk(dk_), nv(nv_), ng(ng_), xp(dk_ + 4), pp(C_ + 4), sp(dk_ + 4) {
    off_x = 0;
    off_q = off_x + C * xp;
    off_p = off_q + C * (xp > nv ? xp : nv);   // Q, then Q S
    off_g = off_p + C * pp;
    off_r = off_g + (reg ? C * pp : 0);
    off_s = off_r + C * nv;
    off_eta = off_s + nv * sp;
    off_lg = off_eta + C * ng;
    off_en = off_lg + C * ng;
    off_lm = off_en + C;
    off_y = off_lm + C;
    total = off_y + (ng > 1 ? C * nv : 0);   // per-column rules: decay-scaled rho
  }
};

// Launch of the general kernel for chunk size C (16, 32 or 64), value tile
// nv (16, 32 or 64) and dynamic LDS bytes lds; one instantiation per file.
template <int C>
hipError_t launch_generic_c(const ProblemArgs& a, int nv, size_t lds, hipStream_t st);

}  // namespace falcon
