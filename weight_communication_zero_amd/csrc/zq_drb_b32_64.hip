// zq_drb_b32_64.hip -- batched (segment-table) dequantize-reduce(-requant)
// kernels for blocks of 32 and 64 elements (see zq_dr_kernels.h).
#include "zq_dr_kernels.h"

namespace zq {

ZQ_DRB_LAUNCHER(32)
ZQ_DRB_LAUNCHER(64)

}  // namespace zq
