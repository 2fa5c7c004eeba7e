// zq_drb_b128_256.hip -- batched (segment-table) dequantize-reduce(-requant)
// kernels for blocks of 128 and 256 elements (see zq_dr_kernels.h).
#include "zq_dr_kernels.h"

namespace zq {

ZQ_DRB_LAUNCHER(128)
ZQ_DRB_LAUNCHER(256)

}  // namespace zq
