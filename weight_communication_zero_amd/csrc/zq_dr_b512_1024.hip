// zq_dr_b512_1024.hip -- dequantize-reduce(-requant) kernels for blocks of
// 512 and 1024 elements (see zq_dr_kernels.h).
#include "zq_dr_kernels.h"

namespace zq {

ZQ_DR_LAUNCHER(512)
ZQ_DR_LAUNCHER(1024)

}  // namespace zq
