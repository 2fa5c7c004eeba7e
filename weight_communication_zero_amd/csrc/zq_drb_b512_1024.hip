// zq_drb_b512_1024.hip -- batched (segment-table) dequantize-reduce(-requant)
// kernels for blocks of 512 and 1024 elements (see zq_dr_kernels.h).
#include "zq_dr_kernels.h"

namespace zq {

ZQ_DRB_LAUNCHER(512)
ZQ_DRB_LAUNCHER(1024)

}  // namespace zq
