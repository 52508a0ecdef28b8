// Chunk-scan kernels for f32 inputs, M = 32 slots (one compilation unit per type and M so the
// instantiations build in parallel).
#include "rsm_scan.h"

namespace rsm {
int scan_f32_m32(int C, int DT, const ScanArgs& a) { return dispatch_c<float, 32>(C, DT, a); }
}  // namespace rsm
