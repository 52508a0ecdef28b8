// Chunk-scan kernels for bf16 inputs, M = 256 slots, chunks of 32 (one compilation unit per
// type and M so the instantiations build in parallel).
#include "rsm_scan.h"

namespace rsm {
int scan_bf16_m256(int C, int DT, const ScanArgs& a) { return dispatch_c<bf16_t, 256>(C, DT, a); }
}  // namespace rsm
