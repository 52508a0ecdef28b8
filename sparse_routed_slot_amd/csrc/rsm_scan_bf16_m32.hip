// Chunk-scan kernels for bf16 inputs, M = 32 slots (one compilation unit per type and M so the
// instantiations build in parallel).
#include "rsm_scan.h"

namespace rsm {
int scan_bf16_m32(int C, int DT, const ScanArgs& a) { return dispatch_c<bf16_t, 32>(C, DT, a); }
}  // namespace rsm
