// bfloat16 instantiation of the chunked SSD scan kernels (x, B, C, y in
// bfloat16; Delta, decay, states and accumulation in float32).
#include "ssd_prefill_impl.h"

namespace ssd {
hipError_t launch_scan_bf16(const ScanArgs& a, int P, int N, hipStream_t stream, hipEvent_t* ev) {
  return prefill::launch_scan<bf16>(a, P, N, stream, ev);
}
}  // namespace ssd
