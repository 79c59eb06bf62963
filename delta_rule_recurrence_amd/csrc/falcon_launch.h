// Host-side launch interface between the C ABI layer and the kernels.
// Arguments reaching these functions have already been validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace falcon {

// Host-side assertions of the launchers' layout and index math.  The
// bounds-check build (FALCON_BOUNDS_CHECK, with the host sanitizers) compiles
// them in: a failed one prints the condition and aborts.  Other builds compile
// them to nothing.
#ifdef FALCON_BOUNDS_CHECK
[[noreturn]] void host_check_failed(const char* cond, const char* file, int line);
#define FALCON_HOST_CHECK(cond) ((cond) ? (void)0 : ::falcon::host_check_failed(#cond, __FILE__, __LINE__))
constexpr bool kBoundsCheck = true;
#else
#define FALCON_HOST_CHECK(cond) ((void)0)
constexpr bool kBoundsCheck = false;
#endif

struct ProblemArgs {
  int B, H, T, dk, dv;
  int variant;
  bool bf16;
  float eps, eps_gamma;
  const void* phi_k;
  const void* phi_q;
  const void* v;
  const float* beta;
  const float* lam;
  const float* S0;       // may be null (zero state)
  const void* k_prev;    // may be null (fresh start)
  void* o;
  float* S_T;            // may be null
  int C;                 // chunk size (chunked path only)
  void* workspace;
  size_t workspace_bytes;
  int spin_limit;        // polls before a bounded wait between waves gives up
  int f1_form;           // Falcon-1 bf16 fast path: 0 one launch, 1 two launches
};

// Default number of polls of a bounded wait (each poll sleeps ~64 cycles):
// about 0.1-0.2 s, far beyond any legitimate hand-over.
constexpr int kDefaultSpinLimit = 1 << 22;

struct DecodeArgs {
  int B, H, dk, dv;
  int variant;
  bool bf16;
  float eps, eps_gamma;
  const void* x;
  const void* q;
  const void* v;
  const float* beta;
  const float* lam;
  float* S;
  const uint8_t* is_first;
  void* o;
};

// Gradient buffers of the Falcon-1 backward (all float32 except dO, which has
// the io dtype).
struct BwdBuffers {
  const void* dO;
  const float* dS_T;     // may be null (no loss on the final state)
  float* dphi_k;
  float* dphi_q;
  float* dv;
  float* dbeta;
  float* dlam;
  float* dS0;            // may be null
  float* dk_prev;        // may be null; written only when k_prev is given
};

hipError_t launch_recurrent(const ProblemArgs& a, hipStream_t st);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t st);
hipError_t launch_chunked(const ProblemArgs& a, hipStream_t st);
size_t chunked_workspace_bytes(const ProblemArgs& a);
// Falcon-1 backward (dk = dv = 64): workspace size and launch.
size_t bwd_workspace_bytes(const ProblemArgs& a);
hipError_t launch_bwd(const ProblemArgs& a, const BwdBuffers& b, hipStream_t st);
// Copy S0 (or zeros when S0 is null) to S_T; used when there is no token.
hipError_t launch_state_copy(const float* S0, float* S_T, int64_t n, hipStream_t st);

}  // namespace falcon
