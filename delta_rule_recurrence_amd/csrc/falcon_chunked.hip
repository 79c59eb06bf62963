// Chunked-forward dispatch for bf16 I/O with dk = dv = 64 and C = 64: the
// chunk matrices and per-sequence chain for Falcon-1, the chunk-tile path for Falcon-1A,
// the per-column path for Falcon-2 / 2A; the general float32 kernel for every
// other case.
#include "falcon_device.h"
#include "falcon_launch.h"

namespace falcon {

hipError_t launch_chunked_generic(const ProblemArgs& a, hipStream_t st);
bool chunked_wy_applies(const ProblemArgs& a);
size_t chunked_wy_workspace_bytes(const ProblemArgs& a);
hipError_t launch_chunked_wy(const ProblemArgs& a, hipStream_t st);
bool chunked_scan_applies(const ProblemArgs& a);
size_t chunked_scan_workspace_bytes(const ProblemArgs& a);
hipError_t launch_chunked_scan(const ProblemArgs& a, hipStream_t st);
bool chunked_percol_applies(const ProblemArgs& a);
hipError_t launch_chunked_percol(const ProblemArgs& a, hipStream_t st);

size_t chunked_workspace_bytes(const ProblemArgs& a) {
  if (chunked_wy_applies(a)) return chunked_wy_workspace_bytes(a);
  return chunked_scan_applies(a) ? chunked_scan_workspace_bytes(a) : 0;
}

hipError_t launch_chunked(const ProblemArgs& a, hipStream_t st) {
  if (chunked_wy_applies(a)) return launch_chunked_wy(a, st);
  if (chunked_scan_applies(a)) return launch_chunked_scan(a, st);
  if (chunked_percol_applies(a)) return launch_chunked_percol(a, st);
  return launch_chunked_generic(a, st);
}

}  // namespace falcon
