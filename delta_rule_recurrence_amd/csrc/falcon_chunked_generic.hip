// Chunk-parallel Falcon forward, general shapes: value-tile choice and
// dispatch to the kernel in falcon_generic_kernel.h (one instantiation file
// per chunk size, compiled in parallel), and the state copy used when there
// is no token.

#include <algorithm>

#include "falcon_device.h"
#include "falcon_generic.h"

namespace falcon {

namespace {

constexpr int kCUs = 256;   // compute units of the part the tile choice targets

size_t generic_lds_bytes(const ProblemArgs& a, int nv) {
  const GenericLayout L(a.C, a.dk, nv, is_per_column(a.variant) ? nv : 1,
                        is_regression(a.variant));
  return sizeof(float) * L.total;
}

}  // namespace

// Value tile (64, 32 or 16 columns): the widest whose LDS footprint fits,
// narrowed while the narrower tiles still give no more workgroups than there
// are compute units (each tile repeats the chunk's key products, so tiles are
// only split to occupy CUs that would otherwise idle).
int generic_tile(const ProblemArgs& a, size_t* lds_bytes) {
  int nv = std::min(a.dv, 64);
  while (nv >= 16 && generic_lds_bytes(a, nv) > 160 * 1024) nv /= 2;
  if (nv < 16) {
    *lds_bytes = 0;
    return 0;
  }
  const int64_t BH = int64_t(a.B) * a.H;
  while (nv > 16 && BH * (a.dv / (nv / 2)) <= kCUs) nv /= 2;
  *lds_bytes = generic_lds_bytes(a, nv);
  return nv;
}

hipError_t launch_chunked_generic(const ProblemArgs& a, hipStream_t st) {
  size_t lds = 0;
  const int nv = generic_tile(a, &lds);
  if (nv == 0) return hipErrorInvalidValue;
  switch (a.C) {
    case 16: return launch_generic_c<16>(a, nv, lds, st);
    case 32: return launch_generic_c<32>(a, nv, lds, st);
    case 64: return launch_generic_c<64>(a, nv, lds, st);
    default: return hipErrorInvalidValue;
  }
}

__global__ void state_copy_kernel(const float* __restrict__ src, float* __restrict__ dst,
                                  int64_t n) {
  for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < n;
       i += int64_t(gridDim.x) * blockDim.x)
    dst[i] = src ? src[i] : 0.0f;
}

hipError_t launch_state_copy(const float* S0, float* S_T, int64_t n, hipStream_t st) {
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(state_copy_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, S0,
                     S_T, n);
  return hipGetLastError();
}

}  // namespace falcon
