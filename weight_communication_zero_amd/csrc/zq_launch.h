// zq_launch.h -- internal launchers behind the C ABI (host side).  Each one
// assumes its arguments were validated by the ABI layer and only enqueues
// kernels on the given stream.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace zq {

constexpr uint32_t kMaxPeers = 16;

// Element types of the 16- and 32-bit data streams (the values of zq_dtype).
enum ElemType : int { kF32 = 0, kBF16 = 1, kF16 = 2 };

// Launch geometry of a kernel: threads per workgroup (64..256) and the most
// workgroups one launch may have; a larger job walks its tiles with a grid
// stride.  Measured on MI355X: the streaming kernels run best with one tile
// per wave in 1-wave workgroups (the dispatcher keeps every CU fed and a
// wave never waits on a sibling), the reduces with one tile per wave in
// 4-wave workgroups, and the ALU-heavy reduce+requant without EF persistent
// (4096 workgroups of 4 waves walking many tiles).
struct Geometry {
    uint32_t threads;
    uint32_t max_wgs;
};

#ifndef ZQ_STREAM_THREADS
#define ZQ_STREAM_THREADS 64
#endif
#ifndef ZQ_REDUCE_THREADS
#define ZQ_REDUCE_THREADS 256
#endif
#ifndef ZQ_RQ_THREADS
#define ZQ_RQ_THREADS 256
#endif
#ifndef ZQ_RQ_MAX_WGS
#define ZQ_RQ_MAX_WGS 4096
#endif

constexpr Geometry kGeomStream{ZQ_STREAM_THREADS, 1u << 24};          // EF quantize, int8, SR
constexpr Geometry kGeomReduce{ZQ_REDUCE_THREADS, 1u << 22};          // dequant-reduce into fp32
constexpr Geometry kGeomReduceRequant{ZQ_RQ_THREADS, ZQ_RQ_MAX_WGS};  // dequant-reduce-requant

inline dim3 grid_for_tiles(size_t tiles, Geometry g) {
    const size_t per_wg = g.threads / 64;
    size_t wgs = (tiles + per_wg - 1) / per_wg;
    if (wgs > g.max_wgs)
        wgs = g.max_wgs;
    if (wgs == 0)
        wgs = 1;
    return dim3((uint32_t)wgs);
}

// g_type, w_type, out_type: an ElemType (kF32, kBF16, kF16).
hipError_t launch_quantize_ef_int4(const void* g, int g_type, float* ef, size_t n, uint32_t block,
                                   float beta_e, float beta_r, uint8_t* codes, float* scales,
                                   hipStream_t stream);

// Partition permutation of the EF quantizer's outputs (codes and scales of
// partition p go to slot slot[p]).
constexpr uint32_t kMaxParts = 256;
struct PartPerm {
    uint64_t part_len;
    uint32_t n_part;
    uint32_t slot[kMaxParts];
};

hipError_t launch_quantize_ef_int4_permuted(const void* g, int g_type, float* ef, size_t n,
                                            uint32_t block, float beta_e, float beta_r,
                                            uint8_t* codes, float* scales, const PartPerm& perm,
                                            hipStream_t stream);

// One tensor of a batched EF quantize (validated by the ABI layer).
struct EfqSegment {
    const void* g;
    float* ef;
    uint8_t* codes;
    float* scales;
    uint64_t n;
};

hipError_t launch_quantize_ef_int4_batched(const EfqSegment* segs, uint32_t n_seg, int g_type,
                                           bool with_ef, uint32_t block, float beta_e,
                                           float beta_r, hipStream_t stream);

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

    __device__ const uint8_t* codes_of(uint32_t q) const { return codes[q]; }
    __device__ const float* scales_of(uint32_t q) const { return scales[q]; }
};

hipError_t launch_dequant_reduce(const DrParams& p, uint32_t block, hipStream_t stream);

// One tensor of a batched dequantize-reduce (validated by the ABI layer):
// peer q's chunk of n elements has its codes at codes + q * codes_stride
// bytes and its scales at scales + q * scales_stride floats.
struct DrSegment {
    const uint8_t* codes;
    const float* scales;
    uint64_t codes_stride;
    uint64_t scales_stride;
    uint64_t n;
    float* out;
    uint8_t* rq_codes;
    float* rq_scales;
    float* rq_ef;
};

// Settings shared by every segment of a batch.
struct DrBatchArgs {
    uint32_t P;
    float alpha;
    float rq_beta_e;
    float rq_beta_r;
    bool out, rq, rq_ef;
};

hipError_t launch_dequant_reduce_batched(const DrSegment* segs, uint32_t n_seg,
                                         const DrBatchArgs& a, uint32_t block, hipStream_t stream);

hipError_t launch_quant_int8(const void* w, int w_type, size_t n, uint32_t block, int8_t* codes,
                             float* scales, hipStream_t stream);

hipError_t launch_dequant_int8(const int8_t* codes, const float* scales, size_t n, uint32_t block,
                               void* out, int out_type, hipStream_t stream);

hipError_t launch_sr_accumulate(uint16_t* dst, uint16_t* src, size_t n, uint64_t seed,
                                uint64_t counter_base, bool zero_src, hipStream_t stream);

// One segment of a batched SR accumulation (validated by the ABI layer).
struct SrSegment {
    uint16_t* dst;
    uint16_t* src;
    uint64_t n;
    uint64_t off;
    uint64_t len;
    uint64_t seed;
    uint64_t cbase;
};

hipError_t launch_sr_accumulate_batched(const SrSegment* segs, uint32_t n_seg, bool zero_src,
                                        hipStream_t stream);

}  // namespace zq
