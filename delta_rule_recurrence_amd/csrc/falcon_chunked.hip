// Chunked-forward dispatch: the fused MFMA kernel where it applies (Falcon-1,
// bf16 I/O, dk = dv = 64, C = 64), the chunk-tile look-back kernel for
// Falcon-1A with the same shapes, the per-column kernel for Falcon-2 / 2A
// with the same shapes, the general float32 kernel otherwise.
#include "falcon_device.h"
#include "falcon_launch.h"

namespace falcon {

hipError_t launch_chunked_generic(const ProblemArgs& a, hipStream_t st);
bool chunked_mfma_applies(const ProblemArgs& a);
hipError_t launch_chunked_mfma(const ProblemArgs& a, hipStream_t st);
bool chunked_scan_applies(const ProblemArgs& a);
size_t chunked_scan_workspace_bytes(const ProblemArgs& a);
hipError_t launch_chunked_scan(const ProblemArgs& a, hipStream_t st);
bool chunked_percol_applies(const ProblemArgs& a);
hipError_t launch_chunked_percol(const ProblemArgs& a, hipStream_t st);

size_t chunked_workspace_bytes(const ProblemArgs& a) {
  return chunked_scan_applies(a) ? chunked_scan_workspace_bytes(a) : 0;
}

hipError_t launch_chunked(const ProblemArgs& a, hipStream_t st) {
  if (chunked_mfma_applies(a)) return launch_chunked_mfma(a, st);
  if (chunked_scan_applies(a)) return launch_chunked_scan(a, st);
  if (chunked_percol_applies(a)) return launch_chunked_percol(a, st);
  return launch_chunked_generic(a, st);
}

}  // namespace falcon
