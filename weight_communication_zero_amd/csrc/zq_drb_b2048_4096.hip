// zq_drb_b2048_4096.hip -- batched (segment-table) dequantize-reduce(-requant)
// kernels for blocks of 2048 and 4096 elements (see zq_dr_kernels.h).
#include "zq_dr_kernels.h"

namespace zq {

ZQ_DRB_LAUNCHER(2048)
ZQ_DRB_LAUNCHER(4096)

}  // namespace zq
