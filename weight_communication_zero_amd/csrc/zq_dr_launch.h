// zq_dr_launch.h -- the reduce kernels of one block size each, compiled in
// their own translation units (zq_dr_b*.hip) so the instantiations build in
// parallel; launch_dequant_reduce (zq_dr.hip) picks one.
#pragma once

#include "zq_launch.h"

namespace zq {

hipError_t launch_dr_b32(const DrParams& p, hipStream_t st);
hipError_t launch_dr_b64(const DrParams& p, hipStream_t st);
hipError_t launch_dr_b128(const DrParams& p, hipStream_t st);
hipError_t launch_dr_b256(const DrParams& p, hipStream_t st);
hipError_t launch_dr_b512(const DrParams& p, hipStream_t st);
hipError_t launch_dr_b1024(const DrParams& p, hipStream_t st);
hipError_t launch_dr_b2048(const DrParams& p, hipStream_t st);
hipError_t launch_dr_b4096(const DrParams& p, hipStream_t st);

#define ZQ_DRB_DECL(BLK)                                                                  \
    hipError_t launch_drb_b##BLK(const DrSegment* segs, uint32_t n_seg, const DrBatchArgs& a, \
                                 hipStream_t st);
ZQ_DRB_DECL(32)
ZQ_DRB_DECL(64)
ZQ_DRB_DECL(128)
ZQ_DRB_DECL(256)
ZQ_DRB_DECL(512)
ZQ_DRB_DECL(1024)
ZQ_DRB_DECL(2048)
ZQ_DRB_DECL(4096)
#undef ZQ_DRB_DECL

}  // namespace zq
