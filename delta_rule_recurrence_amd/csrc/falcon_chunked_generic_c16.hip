// General-shape chunked forward kernels for chunk size 16 (all variants, I/O
// dtypes and value tiles); the kernel is in falcon_generic_kernel.h.

#include "falcon_generic_kernel.h"

namespace falcon {

template hipError_t launch_generic_c<16>(const ProblemArgs& a, int nv, size_t lds, hipStream_t st);

}  // namespace falcon
