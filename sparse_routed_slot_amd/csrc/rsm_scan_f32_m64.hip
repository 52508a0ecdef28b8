// Chunk-scan kernels for f32 inputs, M = 64 slots (one compilation unit per type and M so the
// instantiations build in parallel).
#include "rsm_scan.h"

namespace rsm {
int scan_f32_m64(int C, int DT, const ScanArgs& a) { return dispatch_c<float, 64>(C, DT, a); }
}  // namespace rsm
