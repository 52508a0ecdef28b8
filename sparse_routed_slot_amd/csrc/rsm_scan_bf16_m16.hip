// Chunk-scan kernels for bf16 inputs, M = 16 slots (one compilation unit per type and M so the
// instantiations build in parallel).
#include "rsm_scan.h"

namespace rsm {
int scan_bf16_m16(int C, int DT, const ScanArgs& a) { return dispatch_c<bf16_t, 16>(C, DT, a); }
}  // namespace rsm
