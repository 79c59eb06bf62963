// C ABI of the Falcon library: argument validation, status codes and
// dispatch to the kernels.  Nothing here allocates or synchronises.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>

#include <atomic>
#include <mutex>

#include "falcon.h"
#include "falcon_launch.h"

#ifdef FALCON_BOUNDS_CHECK
namespace falcon {
void host_check_failed(const char* cond, const char* file, int line) {
  fprintf(stderr, "falcon bounds check failed: %s (%s:%d)\n", cond, file, line);
  fflush(stderr);
  abort();
}
}  // namespace falcon
#endif

namespace {

// Polls a bounded wait makes before giving up (falcon_set_wait_limit).
std::atomic<int32_t> g_wait_limit{falcon::kDefaultSpinLimit};
// Form of the Falcon-1 bf16 chunked fast path (falcon_set_f1_launch_form).
std::atomic<int32_t> g_f1_form{FALCON_F1_ONE_LAUNCH};

using falcon::DecodeArgs;
using falcon::ProblemArgs;

bool supported_width(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Range {
  const void* p;
  int64_t bytes;
};

bool overlap(Range a, Range b) {
  if (!a.p || !b.p || a.bytes <= 0 || b.bytes <= 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + static_cast<uintptr_t>(b.bytes) && b0 < a0 + static_cast<uintptr_t>(a.bytes);
}

falcon_status check_problem(const falcon_problem* p) {
  if (!p) return FALCON_ERR_NULL;
  if (p->B < 0 || p->H < 0 || p->T < 0) return FALCON_ERR_SHAPE;
  if (!supported_width(p->dk) || !supported_width(p->dv)) return FALCON_ERR_SHAPE;
  if (p->variant < FALCON_1 || p->variant > FALCON_2A) return FALCON_ERR_VARIANT;
  if (p->io_dtype != FALCON_F32 && p->io_dtype != FALCON_BF16) return FALCON_ERR_DTYPE;
  if (!isfinite(p->eps) || p->eps < 0.0f) return FALCON_ERR_VALUE;
  if (!(p->eps_gamma > 0.0f && p->eps_gamma < 1.0f)) return FALCON_ERR_VALUE;
  const int64_t bh = int64_t(p->B) * p->H;
  if (bh > (int64_t(1) << 30)) return FALCON_ERR_SHAPE;
  return FALCON_OK;
}

bool per_column(int variant) { return variant == FALCON_2 || variant == FALCON_2A; }
bool is_per_column_variant(int variant) { return per_column(variant); }

// Validates the arguments shared by the two forward entry points and fills
// the launch arguments.
// `ws` is the part of a workspace the call will use (none for the recurrent
// form); it may overlap no input and no output.
falcon_status check_forward(const falcon_problem* p, const void* phi_k, const void* phi_q,
                            const void* v, const float* beta, const float* lam, const float* S0,
                            const void* k_prev, void* o, float* S_T, ProblemArgs* out,
                            Range ws = Range{nullptr, 0}) {
  falcon_status s = check_problem(p);
  if (s != FALCON_OK) return s;
  const int64_t bh = int64_t(p->B) * p->H;
  const int64_t es = p->io_dtype == FALCON_BF16 ? 2 : 4;
  const bool work = bh > 0 && p->T > 0;
  if (work && (!phi_k || !phi_q || !v || !beta || !lam || !o)) return FALCON_ERR_NULL;
  const void* ptrs[] = {phi_k, phi_q, v, beta, lam, S0, k_prev, o, S_T};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return FALCON_ERR_ALIGN;
  const int64_t nk = bh * p->T * p->dk, nv = bh * p->T * p->dv;
  const Range ro{o, nv * es};
  const Range inputs[] = {{phi_k, nk * es},
                          {phi_q, nk * es},
                          {v, nv * es},
                          {beta, (per_column(p->variant) ? nv : bh * p->T) * 4},
                          {lam, bh * p->T * 4},
                          {S0, bh * p->dk * p->dv * 4},
                          {k_prev, bh * p->dk * es},
                          {S_T, bh * p->dk * p->dv * 4}};
  for (const Range& r : inputs)
    if (overlap(ro, r)) return FALCON_ERR_ALIAS;
  // S_T may alias S0 exactly (in-place continuation) but not partially, and
  // must not overlap any other input.
  const Range rs{S_T, bh * p->dk * p->dv * 4};
  if (S_T && S0 && S_T != S0 && overlap(rs, Range{S0, rs.bytes})) return FALCON_ERR_ALIAS;
  for (int i = 0; i < 5; ++i)
    if (overlap(rs, inputs[i])) return FALCON_ERR_ALIAS;
  if (overlap(rs, inputs[6])) return FALCON_ERR_ALIAS;
  if (overlap(ws, ro) || overlap(ws, Range{S0, rs.bytes})) return FALCON_ERR_ALIAS;
  for (const Range& r : inputs)
    if (overlap(ws, r)) return FALCON_ERR_ALIAS;

  *out = ProblemArgs{};
  out->B = p->B; out->H = p->H; out->T = p->T; out->dk = p->dk; out->dv = p->dv;
  out->variant = p->variant;
  out->bf16 = p->io_dtype == FALCON_BF16;
  out->eps = p->eps; out->eps_gamma = p->eps_gamma;
  out->phi_k = phi_k; out->phi_q = phi_q; out->v = v; out->beta = beta; out->lam = lam;
  out->S0 = S0; out->k_prev = k_prev; out->o = o; out->S_T = S_T;
  out->spin_limit = g_wait_limit.load(std::memory_order_relaxed);
  out->f1_form = g_f1_form.load(std::memory_order_relaxed);
  return FALCON_OK;
}

falcon_status finish(hipError_t e) { return e == hipSuccess ? FALCON_OK : FALCON_ERR_HIP; }

// With no token to process the result is just S_T = S_0.
falcon_status empty_forward(const ProblemArgs& a, hipStream_t st) {
  const int64_t n = int64_t(a.B) * a.H * a.dk * a.dv;
  if (!a.S_T || n == 0) return FALCON_OK;
  if (a.S_T == a.S0) return FALCON_OK;
  (void)hipGetLastError();
  return finish(falcon::launch_state_copy(a.S0, a.S_T, n, st));
}

// Validates the backward's arguments and fills the launch arguments.
falcon_status check_backward(const falcon_problem* p, const void* phi_k, const void* phi_q,
                             const void* v, const float* beta, const float* lam, const float* S0,
                             const void* k_prev, const void* dO, const float* dS_T, float* dphi_k,
                             float* dphi_q, float* dv, float* dbeta, float* dlam, float* dS0,
                             float* dk_prev, ProblemArgs* out, falcon::BwdBuffers* buf) {
  falcon_status s = check_problem(p);
  if (s != FALCON_OK) return s;
  if (p->variant != FALCON_1) return FALCON_ERR_VARIANT;
  if (p->dk != 64 || p->dv != 64) return FALCON_ERR_SHAPE;
  const int64_t bh = int64_t(p->B) * p->H;
  if (bh * ((int64_t(p->T) + 31) / 32) > (int64_t(1) << 30)) return FALCON_ERR_SHAPE;   // chunk count
  const int64_t es = p->io_dtype == FALCON_BF16 ? 2 : 4;
  const bool work = bh > 0 && p->T > 0;
  if (work && (!phi_k || !phi_q || !v || !beta || !lam || !dO || !dphi_k || !dphi_q || !dv ||
               !dbeta || !dlam))
    return FALCON_ERR_NULL;
  const void* ptrs[] = {phi_k, phi_q, v, beta, lam, S0, k_prev, dO, dS_T,
                        dphi_k, dphi_q, dv, dbeta, dlam, dS0, dk_prev};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return FALCON_ERR_ALIGN;
  const int64_t nt = bh * p->T * 64, ns = bh * 64 * 64;
  const Range inputs[] = {{phi_k, nt * es}, {phi_q, nt * es}, {v, nt * es},
                          {beta, bh * p->T * 4}, {lam, bh * p->T * 4}, {S0, ns * 4},
                          {k_prev, bh * 64 * es}, {dO, nt * es}, {dS_T, ns * 4}};
  const Range outputs[] = {{dphi_k, nt * 4}, {dphi_q, nt * 4}, {dv, nt * 4},
                           {dbeta, bh * p->T * 4}, {dlam, bh * p->T * 4}, {dS0, ns * 4},
                           {k_prev ? dk_prev : nullptr, bh * 64 * 4}};
  for (int i = 0; i < 7; ++i) {
    for (const Range& r : inputs)
      if (overlap(outputs[i], r)) return FALCON_ERR_ALIAS;
    for (int j = i + 1; j < 7; ++j)
      if (overlap(outputs[i], outputs[j])) return FALCON_ERR_ALIAS;
  }
  *out = ProblemArgs{};
  out->B = p->B; out->H = p->H; out->T = p->T; out->dk = p->dk; out->dv = p->dv;
  out->variant = p->variant;
  out->bf16 = p->io_dtype == FALCON_BF16;
  out->eps = p->eps; out->eps_gamma = p->eps_gamma;
  out->phi_k = phi_k; out->phi_q = phi_q; out->v = v; out->beta = beta; out->lam = lam;
  out->S0 = S0; out->k_prev = k_prev;
  *buf = falcon::BwdBuffers{dO, dS_T, dphi_k, dphi_q, dv, dbeta, dlam, dS0, k_prev ? dk_prev : nullptr};
  return FALCON_OK;
}

// True when the backward's workspace range overlaps any input or output.
bool bwd_workspace_overlaps(const ProblemArgs& a, const falcon::BwdBuffers& b, Range ws) {
  const int64_t bh = int64_t(a.B) * a.H;
  const int64_t es = a.bf16 ? 2 : 4;
  const int64_t nt = bh * a.T * 64, ns = bh * 64 * 64;
  const Range all[] = {{a.phi_k, nt * es}, {a.phi_q, nt * es}, {a.v, nt * es},
                       {a.beta, bh * a.T * 4}, {a.lam, bh * a.T * 4}, {a.S0, ns * 4},
                       {a.k_prev, bh * 64 * es}, {b.dO, nt * es}, {b.dS_T, ns * 4},
                       {b.dphi_k, nt * 4}, {b.dphi_q, nt * 4}, {b.dv, nt * 4},
                       {b.dbeta, bh * a.T * 4}, {b.dlam, bh * a.T * 4}, {b.dS0, ns * 4},
                       {b.dk_prev, bh * 64 * 4}};
  for (const Range& r : all)
    if (overlap(ws, r)) return true;
  return false;
}

// ---- scratch of the allocation-free chunked entry point ---------------------
// One static device array per GPU the library runs on, held until the process
// ends.  In host code `scratch` only names the symbol; its device address is
// looked up once per device (hipGetSymbolAddress, with that device current)
// and only that address is ever handed to a kernel.
__device__ __align__(256) unsigned char scratch[FALCON_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch, or nullptr on failure.
void* scratch_for_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

// The forward's arguments restricted to sequences [s0, s0 + n) (sequences are
// the contiguous (b, h) slabs of every tensor), as a problem with B = 1, H = n.
ProblemArgs sequence_slice(const ProblemArgs& a, int64_t s0, int n) {
  ProblemArgs r = a;
  const int64_t es = a.bf16 ? 2 : 4;
  const int64_t tk = int64_t(a.T) * a.dk, tv = int64_t(a.T) * a.dv, st = int64_t(a.dk) * a.dv;
  const int64_t bstride = is_per_column_variant(a.variant) ? tv : a.T;
  auto off = [&](const void* p, int64_t elems, int64_t bytes) -> const void* {
    return p ? static_cast<const char*>(p) + s0 * elems * bytes : nullptr;
  };
  r.B = 1;
  r.H = n;
  r.phi_k = off(a.phi_k, tk, es);
  r.phi_q = off(a.phi_q, tk, es);
  r.v = off(a.v, tv, es);
  r.beta = static_cast<const float*>(off(a.beta, bstride, 4));
  r.lam = static_cast<const float*>(off(a.lam, a.T, 4));
  r.S0 = static_cast<const float*>(off(a.S0, st, 4));
  r.k_prev = off(a.k_prev, a.dk, es);
  r.o = const_cast<void*>(off(a.o, tv, es));
  r.S_T = static_cast<float*>(const_cast<void*>(off(a.S_T, st, 4)));
  return r;
}

}  // namespace

extern "C" {

int32_t falcon_abi_version(void) { return FALCON_ABI_VERSION; }

int32_t falcon_set_wait_limit(int32_t polls) {
  if (polls < 0) return -1;
  return g_wait_limit.exchange(polls, std::memory_order_relaxed);
}

int32_t falcon_set_f1_launch_form(int32_t form) {
  if (form != FALCON_F1_ONE_LAUNCH && form != FALCON_F1_TWO_LAUNCH) return -1;
  return g_f1_form.exchange(form, std::memory_order_relaxed);
}

const char* falcon_status_string(int32_t s) {
  switch (s) {
    case FALCON_OK: return "FALCON_OK";
    case FALCON_ERR_NULL: return "FALCON_ERR_NULL: a required pointer is NULL";
    case FALCON_ERR_SHAPE: return "FALCON_ERR_SHAPE: unsupported or negative size";
    case FALCON_ERR_DTYPE: return "FALCON_ERR_DTYPE: unknown io dtype";
    case FALCON_ERR_CHUNK: return "FALCON_ERR_CHUNK: chunk size must be 16, 32 or 64";
    case FALCON_ERR_ALIGN: return "FALCON_ERR_ALIGN: pointer not 16-byte aligned";
    case FALCON_ERR_WORKSPACE: return "FALCON_ERR_WORKSPACE: workspace missing or too small";
    case FALCON_ERR_VARIANT: return "FALCON_ERR_VARIANT: unknown variant";
    case FALCON_ERR_HIP: return "FALCON_ERR_HIP: the HIP runtime reported a launch error";
    case FALCON_ERR_VALUE: return "FALCON_ERR_VALUE: eps must be finite and >= 0, eps_gamma in (0,1)";
    case FALCON_ERR_ALIAS: return "FALCON_ERR_ALIAS: an output or the workspace overlaps another argument";
    case FALCON_ERR_SCRATCH:
      return "FALCON_ERR_SCRATCH: one sequence needs more scratch than the allocation-free entry point holds";
    default: return "unknown falcon_status";
  }
}

falcon_status falcon_fwd_recurrent(const falcon_problem* p, const void* phi_k, const void* phi_q,
                                   const void* v, const float* beta, const float* lam,
                                   const float* S0, const void* k_prev, void* o, float* S_T,
                                   hipStream_t stream) {
  ProblemArgs a;
  falcon_status s = check_forward(p, phi_k, phi_q, v, beta, lam, S0, k_prev, o, S_T, &a);
  if (s != FALCON_OK) return s;
  if (int64_t(a.B) * a.H == 0 || a.T == 0) return empty_forward(a, stream);
  (void)hipGetLastError();
  return finish(falcon::launch_recurrent(a, stream));
}

size_t falcon_workspace_bytes(const falcon_problem* p, int32_t C) {
  if (check_problem(p) != FALCON_OK) return static_cast<size_t>(-1);
  if (C != 16 && C != 32 && C != 64) return static_cast<size_t>(-1);
  ProblemArgs a{};
  a.B = p->B; a.H = p->H; a.T = p->T; a.dk = p->dk; a.dv = p->dv;
  a.variant = p->variant; a.bf16 = p->io_dtype == FALCON_BF16; a.C = C;
  return falcon::chunked_workspace_bytes(a);
}

falcon_status falcon_fwd_chunked(const falcon_problem* p, const void* phi_k, const void* phi_q,
                                 const void* v, const float* beta, const float* lam,
                                 const float* S0, const void* k_prev, void* o, float* S_T,
                                 int32_t C, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
  ProblemArgs a;
  falcon_status s = check_forward(p, phi_k, phi_q, v, beta, lam, S0, k_prev, o, S_T, &a);
  if (s != FALCON_OK) return s;
  if (C != 16 && C != 32 && C != 64) return FALCON_ERR_CHUNK;
  a.C = C;
  const size_t need = falcon::chunked_workspace_bytes(a);
  if (need > 0 && (!workspace || workspace_bytes < need)) return FALCON_ERR_WORKSPACE;
  if (workspace && !aligned16(workspace)) return FALCON_ERR_ALIGN;
  if (need > 0) {
    s = check_forward(p, phi_k, phi_q, v, beta, lam, S0, k_prev, o, S_T, &a,
                      Range{workspace, static_cast<int64_t>(need)});
    if (s != FALCON_OK) return s;
    a.C = C;
  }
  a.workspace = workspace;
  a.workspace_bytes = workspace_bytes;
  if (int64_t(a.B) * a.H == 0 || a.T == 0) return empty_forward(a, stream);
  (void)hipGetLastError();
  return finish(falcon::launch_chunked(a, stream));
}

falcon_status falcon_fwd_chunked_noalloc(const falcon_problem* p, const void* phi_k,
                                         const void* phi_q, const void* v, const float* beta,
                                         const float* lam, const float* S0, const void* k_prev,
                                         void* o, float* S_T, int32_t C, hipStream_t stream) {
  ProblemArgs a;
  falcon_status s = check_forward(p, phi_k, phi_q, v, beta, lam, S0, k_prev, o, S_T, &a);
  if (s != FALCON_OK) return s;
  if (C != 16 && C != 32 && C != 64) return FALCON_ERR_CHUNK;
  a.C = C;
  const int64_t BH = int64_t(a.B) * a.H;
  if (BH == 0 || a.T == 0) return empty_forward(a, stream);
  // sequences per launch group: as many as the scratch holds
  ProblemArgs one = sequence_slice(a, 0, 1);
  const size_t per_seq = falcon::chunked_workspace_bytes(one);
  int64_t group = BH;
  if (per_seq > 0) {
    if (per_seq > size_t(FALCON_NOALLOC_SCRATCH_BYTES)) return FALCON_ERR_SCRATCH;
    group = std::min<int64_t>(BH, int64_t(FALCON_NOALLOC_SCRATCH_BYTES / per_seq));
    while (group > 1 &&
           falcon::chunked_workspace_bytes(sequence_slice(a, 0, int(group))) > size_t(FALCON_NOALLOC_SCRATCH_BYTES))
      --group;
  }
  void* ptr = nullptr;
  if (per_seq > 0) {
    ptr = scratch_for_current_device();
    if (!ptr) return FALCON_ERR_HIP;
  }
  (void)hipGetLastError();
  // Groups run one after another on the stream, so each reuses the scratch
  // only after the previous group's kernels have finished with it.
  for (int64_t s0 = 0; s0 < BH; s0 += group) {
    ProblemArgs g = sequence_slice(a, s0, int(std::min<int64_t>(group, BH - s0)));
    g.workspace = ptr;
    g.workspace_bytes = per_seq > 0 ? size_t(FALCON_NOALLOC_SCRATCH_BYTES) : 0;
    const hipError_t e = falcon::launch_chunked(g, stream);
    if (e != hipSuccess) return FALCON_ERR_HIP;
  }
  return FALCON_OK;
}

size_t falcon_bwd_workspace_bytes(const falcon_problem* p) {
  if (check_problem(p) != FALCON_OK) return static_cast<size_t>(-1);
  if (p->variant != FALCON_1 || p->dk != 64 || p->dv != 64) return static_cast<size_t>(-1);
  ProblemArgs a{};
  a.B = p->B; a.H = p->H; a.T = p->T; a.dk = p->dk; a.dv = p->dv; a.variant = p->variant;
  return falcon::bwd_workspace_bytes(a);
}

falcon_status falcon_bwd_chunked(const falcon_problem* p, const void* phi_k, const void* phi_q,
                                 const void* v, const float* beta, const float* lam,
                                 const float* S0, const void* k_prev, const void* dO,
                                 const float* dS_T, float* dphi_k, float* dphi_q, float* dv,
                                 float* dbeta, float* dlam, float* dS0, float* dk_prev,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  ProblemArgs a;
  falcon::BwdBuffers b;
  falcon_status s = check_backward(p, phi_k, phi_q, v, beta, lam, S0, k_prev, dO, dS_T, dphi_k,
                                   dphi_q, dv, dbeta, dlam, dS0, dk_prev, &a, &b);
  if (s != FALCON_OK) return s;
  const size_t need = falcon::bwd_workspace_bytes(a);
  if (need > 0 && (!workspace || workspace_bytes < need)) return FALCON_ERR_WORKSPACE;
  if (workspace && !aligned16(workspace)) return FALCON_ERR_ALIGN;
  if (need > 0 && bwd_workspace_overlaps(a, b, Range{workspace, static_cast<int64_t>(need)}))
    return FALCON_ERR_ALIAS;
  a.workspace = workspace;
  a.workspace_bytes = workspace_bytes;
  const int64_t bh = int64_t(a.B) * a.H;
  if (bh == 0) return FALCON_OK;
  (void)hipGetLastError();
  if (a.T == 0) {
    // no token: dS0 = dS_T and the previous key reaches nothing
    hipError_t e = hipSuccess;
    if (b.dS0) e = falcon::launch_state_copy(b.dS_T, b.dS0, bh * 64 * 64, stream);
    if (e == hipSuccess && b.dk_prev) e = falcon::launch_state_copy(nullptr, b.dk_prev, bh * 64, stream);
    return finish(e);
  }
  return finish(falcon::launch_bwd(a, b, stream));
}

falcon_status falcon_decode_step(const falcon_problem* p, const void* phi_k_prev,
                                 const void* phi_q, const void* v, const float* beta,
                                 const float* lam, float* S, const uint8_t* is_first, void* o,
                                 hipStream_t stream) {
  falcon_status s = check_problem(p);
  if (s != FALCON_OK) return s;
  const int64_t bh = int64_t(p->B) * p->H;
  if (bh == 0) return FALCON_OK;
  if (!phi_k_prev || !phi_q || !v || !beta || !lam || !S || !o) return FALCON_ERR_NULL;
  const void* ptrs[] = {phi_k_prev, phi_q, v, beta, lam, S, o};
  for (const void* q : ptrs)
    if (!aligned16(q)) return FALCON_ERR_ALIGN;
  const int64_t es = p->io_dtype == FALCON_BF16 ? 2 : 4;
  const Range ro{o, bh * p->dv * es};
  const Range rs{S, bh * p->dk * p->dv * 4};
  const Range inputs[] = {{phi_k_prev, bh * p->dk * es},
                          {phi_q, bh * p->dk * es},
                          {v, bh * p->dv * es},
                          {beta, (per_column(p->variant) ? bh * p->dv : bh) * 4},
                          {lam, bh * 4},
                          {is_first, is_first ? p->B : 0}};
  for (const Range& r : inputs)
    if (overlap(ro, r) || overlap(rs, r)) return FALCON_ERR_ALIAS;
  if (overlap(ro, rs)) return FALCON_ERR_ALIAS;
  DecodeArgs a{};
  a.B = p->B; a.H = p->H; a.dk = p->dk; a.dv = p->dv; a.variant = p->variant;
  a.bf16 = p->io_dtype == FALCON_BF16;
  a.eps = p->eps; a.eps_gamma = p->eps_gamma;
  a.x = phi_k_prev; a.q = phi_q; a.v = v; a.beta = beta; a.lam = lam; a.S = S;
  a.is_first = is_first; a.o = o;
  (void)hipGetLastError();
  return finish(falcon::launch_decode(a, stream));
}

}  // extern "C"
