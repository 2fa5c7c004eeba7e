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

}  // namespace zq
