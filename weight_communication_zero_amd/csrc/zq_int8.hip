// zq_int8.hip -- qwZ: block int8 weight quantization before the forward
// all-gather, and dequantization after it ("ZeROPlusPlus.md" notes, section
// 1.2: fp16 weights sent as int8, every block of parameters quantized
// independently for accuracy).
//   s = absmax(w over the block) / 127;  k = clamp(rne(w / s), +-127)
//   w' = k * s   (fp32, or rounded to nearest even bf16 or fp16)
// The weights come as fp32, bf16 or fp16 (the pages' qwZ input), widened to
// fp32 exactly.
//
// Quantize reads 2 (bf16, fp16) or 4 (fp32) B/elem and writes 1 B + 4/B B;
// dequantize the reverse.  In sub-vector u lane l owns the 8 elements
// starting at u*512 + 8l: a 16-byte 16-bit load, an 8-byte code store.  A
// block of B <= 512 elements is B/8 adjacent lanes; a larger block spans
// B/512 sub-vectors of the whole wave.  No LDS.
#include "zq_device.h"
#include "zq_launch.h"

namespace zq {
namespace {

template <int B>
struct Q8Geom {
    static constexpr int VEC = 8;
    static constexpr int SUB = kWave * VEC;
    static constexpr int LPB = B <= SUB ? B / VEC : kWave;
    static constexpr int SPB = B <= SUB ? 1 : B / SUB;
    static constexpr int U = SPB > 2 ? SPB : 2;
    static constexpr int TILE = SUB * U;
    static constexpr int BPT = TILE / B;
};

template <int IN, int B, bool MASK>
__device__ __forceinline__ void q8_tile(const void* __restrict__ wv, size_t n,
                                        int8_t* __restrict__ codes, float* __restrict__ scales,
                                        size_t tile) {
    using G = Q8Geom<B>;
    const int lane = lane_id();
    const size_t base = tile * (size_t)G::TILE;
    float x[G::U][8];

#pragma unroll
    for (int u = 0; u < G::U; ++u) {
        const size_t i0 = base + (size_t)u * G::SUB + (size_t)lane * 8;
        if constexpr (!MASK) {
            if constexpr (IN != kF32) {
                u4 w = ld_stream((const u4*)((const uint16_t*)wv + i0));
                x[u][0] = half_lo<IN>(w.x); x[u][1] = half_hi<IN>(w.x);
                x[u][2] = half_lo<IN>(w.y); x[u][3] = half_hi<IN>(w.y);
                x[u][4] = half_lo<IN>(w.z); x[u][5] = half_hi<IN>(w.z);
                x[u][6] = half_lo<IN>(w.w); x[u][7] = half_hi<IN>(w.w);
            } else {
                f4 a = ld_stream((const f4*)((const float*)wv + i0));
                f4 b = ld_stream((const f4*)((const float*)wv + i0 + 4));
                x[u][0] = a.x; x[u][1] = a.y; x[u][2] = a.z; x[u][3] = a.w;
                x[u][4] = b.x; x[u][5] = b.y; x[u][6] = b.z; x[u][7] = b.w;
            }
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const bool in = i0 + j < n;
                if constexpr (IN != kF32)
                    x[u][j] = in ? half_lo<IN>(((const uint16_t*)wv)[i0 + j]) : 0.0f;
                else
                    x[u][j] = in ? ((const float*)wv)[i0 + j] : 0.0f;
            }
        }
    }

    BlockScale bs[G::SPB == 1 ? G::U : G::BPT];
    if constexpr (G::SPB == 1) {
#pragma unroll
        for (int u = 0; u < G::U; ++u) {
            uint32_t m = 0;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                m = max(m, absbits(x[u][j]));
            bs[u] = block_scale<127>(group_max<G::LPB>(m));
        }
    } else {
#pragma unroll
        for (int b = 0; b < G::BPT; ++b) {
            uint32_t m = 0;
#pragma unroll
            for (int u = b * G::SPB; u < (b + 1) * G::SPB; ++u)
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    m = max(m, absbits(x[u][j]));
            bs[b] = block_scale<127>(group_max<kWave>(m));
        }
    }

    if constexpr (G::SPB == 1) {
        if (lane % G::LPB == 0) {
#pragma unroll
            for (int u = 0; u < G::U; ++u) {
                const size_t i0 = base + (size_t)u * G::SUB + (size_t)lane * 8;
                if (!MASK || i0 < n)
                    scales[i0 / B] = bs[u].s;
            }
        }
    } else {
        if (lane == 0) {
#pragma unroll
            for (int b = 0; b < G::BPT; ++b) {
                const size_t i0 = base + (size_t)b * B;
                if (!MASK || i0 < n)
                    scales[i0 / B] = bs[b].s;
            }
        }
    }

    float kf[G::U][8];
    bool redo = false;
#pragma unroll
    for (int u = 0; u < G::U; ++u)
#pragma unroll
        for (int j = 0; j < 8; ++j)
            kf[u][j] = code_fast<127>(x[u][j], bs[G::SPB == 1 ? u : u / G::SPB], redo);
    if (redo) {
#pragma unroll
        for (int u = 0; u < G::U; ++u)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                kf[u][j] = code_fix<127>(x[u][j], bs[G::SPB == 1 ? u : u / G::SPB], kf[u][j]);
    }

#pragma unroll
    for (int u = 0; u < G::U; ++u) {
        const size_t i0 = base + (size_t)u * G::SUB + (size_t)lane * 8;
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            lo |= ((uint32_t)code_clamp<127>(kf[u][j]) & 0xFFu) << (8 * j);
            hi |= ((uint32_t)code_clamp<127>(kf[u][j + 4]) & 0xFFu) << (8 * j);
        }
        if constexpr (!MASK) {
            u2 v = {lo, hi};
            st_stream(v, (u2*)(codes + i0));
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (i0 + j < n)
                    codes[i0 + j] = (int8_t)((j < 4 ? lo : hi) >> (8 * (j & 3)));
        }
    }
}

// Full tiles without bounds checks; the ragged last tile goes, in the same
// launch, to the one wave whose loop stops exactly at it (the two paths are
// never live at once, so the masked one costs the loop no registers).
template <int IN, int B>
__global__ __launch_bounds__(kBlockThreads) void q8_kernel(const void* __restrict__ w, size_t n,
                                                           int8_t* __restrict__ codes,
                                                           float* __restrict__ scales) {
    using G = Q8Geom<B>;
    const size_t nfull = n / G::TILE;
    size_t t = stream_wave_id<kGeomStream.threads>();
    for (; t < nfull; t += wave_count())
        q8_tile<IN, B, false>(w, n, codes, scales, t);
    if (t == nfull && n % G::TILE)
        q8_tile<IN, B, true>(w, n, codes, scales, t);
}

// Dequantize: lane l of sub-vector u owns 8 codes (one 8-byte load) that lie
// in a single block (B >= 32), so each lane needs one scale and no exchange.
#ifndef ZQ_DQ_U
#define ZQ_DQ_U 2
#endif
constexpr int kDqU = ZQ_DQ_U;
constexpr int kDqSub = kWave * 8;
constexpr int kDqTile = kDqSub * kDqU;

template <int OUT, bool MASK>
__device__ __forceinline__ void dq8_tile(const int8_t* __restrict__ codes,
                                         const float* __restrict__ scales, size_t n,
                                         uint32_t log2b, void* __restrict__ out, size_t tile) {
    const int lane = lane_id();
    const size_t base = tile * (size_t)kDqTile;
    u2 cw[kDqU];
    float s[kDqU];
#pragma unroll
    for (int u = 0; u < kDqU; ++u) {
        const size_t i0 = base + (size_t)u * kDqSub + (size_t)lane * 8;
        if constexpr (!MASK) {
            cw[u] = ld_stream((const u2*)(codes + i0));
            s[u] = scales[i0 >> log2b];
        } else {
            uint32_t lo = 0, hi = 0;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (i0 + j < n) {
                    const uint32_t b = (uint8_t)codes[i0 + j];
                    if (j < 4)
                        lo |= b << (8 * j);
                    else
                        hi |= b << (8 * (j - 4));
                }
            cw[u] = u2{lo, hi};
            s[u] = i0 < n ? scales[i0 >> log2b] : 0.0f;
        }
    }
#pragma unroll
    for (int u = 0; u < kDqU; ++u) {
        const size_t i0 = base + (size_t)u * kDqSub + (size_t)lane * 8;
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t w = j < 4 ? cw[u].x : cw[u].y;
            v[j] = (float)((int32_t)(w << (24 - 8 * (j & 3))) >> 24) * s[u];
        }
        if constexpr (OUT != kF32) {
            if constexpr (!MASK) {
                u4 o = {pack_half_rne<OUT>(v[0], v[1]), pack_half_rne<OUT>(v[2], v[3]),
                        pack_half_rne<OUT>(v[4], v[5]), pack_half_rne<OUT>(v[6], v[7])};
                st_stream(o, (u4*)((uint16_t*)out + i0));
            } else {
#pragma unroll
                for (int j = 0; j < 8; j += 2) {
                    const uint32_t pr = pack_half_rne<OUT>(v[j], v[j + 1]);
                    if (i0 + j < n)
                        ((uint16_t*)out)[i0 + j] = (uint16_t)pr;
                    if (i0 + j + 1 < n)
                        ((uint16_t*)out)[i0 + j + 1] = (uint16_t)(pr >> 16);
                }
            }
        } else {
            if constexpr (!MASK) {
                f4 a = {v[0], v[1], v[2], v[3]};
                f4 b = {v[4], v[5], v[6], v[7]};
                st_stream(a, (f4*)((float*)out + i0));
                st_stream(b, (f4*)((float*)out + i0 + 4));
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (i0 + j < n)
                        ((float*)out)[i0 + j] = v[j];
            }
        }
    }
}

template <int OUT>
__global__ __launch_bounds__(kBlockThreads) void dq8_kernel(const int8_t* __restrict__ codes,
                                                            const float* __restrict__ scales,
                                                            size_t n, uint32_t log2b,
                                                            void* __restrict__ out) {
    const size_t nfull = n / kDqTile;
    size_t t = stream_wave_id<kGeomStream.threads>();
    for (; t < nfull; t += wave_count())
        dq8_tile<OUT, false>(codes, scales, n, log2b, out, t);
    if (t == nfull && n % kDqTile)
        dq8_tile<OUT, true>(codes, scales, n, log2b, out, t);
}

template <int IN, int B>
hipError_t launch_q8_b(const void* w, size_t n, int8_t* codes, float* scales, hipStream_t st) {
    using G = Q8Geom<B>;
    const size_t ntiles = (n + G::TILE - 1) / G::TILE;
    void* args[] = {(void*)&w, (void*)&n, (void*)&codes, (void*)&scales};
    return hipLaunchKernel((const void*)&q8_kernel<IN, B>, grid_for_tiles(ntiles, kGeomStream),
                           dim3(kGeomStream.threads), args, 0, st);
}

template <int IN>
hipError_t launch_q8_t(const void* w, size_t n, uint32_t block, int8_t* codes, float* scales,
                       hipStream_t st) {
    switch (block) {
        case 32: return launch_q8_b<IN, 32>(w, n, codes, scales, st);
        case 64: return launch_q8_b<IN, 64>(w, n, codes, scales, st);
        case 128: return launch_q8_b<IN, 128>(w, n, codes, scales, st);
        case 256: return launch_q8_b<IN, 256>(w, n, codes, scales, st);
        case 512: return launch_q8_b<IN, 512>(w, n, codes, scales, st);
        case 1024: return launch_q8_b<IN, 1024>(w, n, codes, scales, st);
        case 2048: return launch_q8_b<IN, 2048>(w, n, codes, scales, st);
        case 4096: return launch_q8_b<IN, 4096>(w, n, codes, scales, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_quant_int8(const void* w, int w_type, size_t n, uint32_t block, int8_t* codes,
                             float* scales, hipStream_t stream) {
    switch (w_type) {
        case kF32: return launch_q8_t<kF32>(w, n, block, codes, scales, stream);
        case kBF16: return launch_q8_t<kBF16>(w, n, block, codes, scales, stream);
        case kF16: return launch_q8_t<kF16>(w, n, block, codes, scales, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_dequant_int8(const int8_t* codes, const float* scales, size_t n, uint32_t block,
                               void* out, int out_type, hipStream_t stream) {
    uint32_t log2b = 0;
    while ((1u << log2b) < block)
        ++log2b;
    const size_t ntiles = (n + kDqTile - 1) / kDqTile;
    void* args[] = {(void*)&codes, (void*)&scales, (void*)&n, (void*)&log2b, (void*)&out};
    const void* fn = out_type == kBF16  ? (const void*)&dq8_kernel<kBF16>
                     : out_type == kF16 ? (const void*)&dq8_kernel<kF16>
                     : out_type == kF32 ? (const void*)&dq8_kernel<kF32>
                                        : nullptr;
    if (!fn)
        return hipErrorInvalidValue;
    return hipLaunchKernel(fn, grid_for_tiles(ntiles, kGeomStream), dim3(kGeomStream.threads), args,
                           0, stream);
}

}  // namespace zq
