// zq_dr.hip -- entries of the dequantize-reduce(-requant) launches, single and
// batched: each picks the launcher of the block size.  The kernels live in
// zq_dr_kernels.h; each block size's instantiations are compiled in
// zq_dr_b*.hip (single calls) and zq_drb_b*.hip (batched calls).
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

hipError_t launch_dequant_reduce_batched(const DrSegment* segs, uint32_t n_seg,
                                         const DrBatchArgs& a, uint32_t block, hipStream_t st) {
    switch (block) {
        case 32: return launch_drb_b32(segs, n_seg, a, st);
        case 64: return launch_drb_b64(segs, n_seg, a, st);
        case 128: return launch_drb_b128(segs, n_seg, a, st);
        case 256: return launch_drb_b256(segs, n_seg, a, st);
        case 512: return launch_drb_b512(segs, n_seg, a, st);
        case 1024: return launch_drb_b1024(segs, n_seg, a, st);
        case 2048: return launch_drb_b2048(segs, n_seg, a, st);
        case 4096: return launch_drb_b4096(segs, n_seg, a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace zq
