// float32 instantiation of the chunked SSD scan kernels (x, B, C, y in float32).
#include "ssd_prefill_impl.h"

namespace ssd {
hipError_t launch_scan_f32(const ScanArgs& a, int P, int N, hipStream_t stream, hipEvent_t* ev) {
  return prefill::launch_scan<float>(a, P, N, stream, ev);
}
}  // namespace ssd
