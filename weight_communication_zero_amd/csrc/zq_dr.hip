// zq_dr.hip -- entry of the dequantize-reduce(-requant) launch: picks the
// launcher of the block size.  The kernels live in zq_dr_kernels.h; each
// block size's instantiations are compiled in zq_dr_b*.hip.
#include "zq_dr_launch.h"

namespace zq {

hipError_t launch_dequant_reduce(const DrParams& p, uint32_t block, hipStream_t st) {
    switch (block) {
        case 32: return launch_dr_b32(p, st);
        case 64: return launch_dr_b64(p, st);
        case 128: return launch_dr_b128(p, st);
        case 256: return launch_dr_b256(p, st);
        case 512: return launch_dr_b512(p, st);
        case 1024: return launch_dr_b1024(p, st);
        case 2048: return launch_dr_b2048(p, st);
        case 4096: return launch_dr_b4096(p, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace zq
