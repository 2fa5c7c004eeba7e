// zq_dr_b2048_4096.hip -- dequantize-reduce(-requant) kernels for blocks of
// 2048 and 4096 elements (see zq_dr_kernels.h).
#include "zq_dr_kernels.h"

namespace zq {

ZQ_DR_LAUNCHER(2048)
ZQ_DR_LAUNCHER(4096)

}  // namespace zq
