// zq_launch.h -- internal launchers behind the C ABI (host side).  Each one
// assumes its arguments were validated by the ABI layer and only enqueues
// kernels on the given stream.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace zq {

constexpr uint32_t kMaxPeers = 16;

// Upper bound on workgroups per launch (grid-stride beyond it).  256 CUs
// times 16 workgroups of 4 waves keeps every SIMD at full occupancy.
#ifndef ZQ_MAX_WORKGROUPS
#define ZQ_MAX_WORKGROUPS 4096
#endif

inline uint32_t grid_for_tiles(size_t tiles, size_t waves_per_wg) {
    size_t wgs = (tiles + waves_per_wg - 1) / waves_per_wg;
    if (wgs > ZQ_MAX_WORKGROUPS)
        wgs = ZQ_MAX_WORKGROUPS;
    if (wgs == 0)
        wgs = 1;
    return (uint32_t)wgs;
}

hipError_t launch_quantize_ef_int4(const void* g, bool g_bf16, float* ef, size_t n, uint32_t block,
                                   float beta_e, float beta_r, uint8_t* codes, float* scales,
                                   hipStream_t stream);

struct DrParams {
    const uint8_t* codes[kMaxPeers];
    const float* scales[kMaxPeers];
    uint32_t P;
    size_t n;
    float alpha;
    float* out;
    uint8_t* rq_codes;
    float* rq_scales;
    float* rq_ef;
    float rq_beta_e;
    float rq_beta_r;
};

hipError_t launch_dequant_reduce(const DrParams& p, uint32_t block, hipStream_t stream);

hipError_t launch_quant_int8(const void* w, bool w_bf16, size_t n, uint32_t block, int8_t* codes,
                             float* scales, hipStream_t stream);

hipError_t launch_dequant_int8(const int8_t* codes, const float* scales, size_t n, uint32_t block,
                               void* out, bool out_bf16, hipStream_t stream);

hipError_t launch_sr_accumulate(uint16_t* dst, uint16_t* src, size_t n, uint64_t seed,
                                uint64_t counter_base, bool zero_src, hipStream_t stream);

}  // namespace zq
