// zq_efq.hip -- block int4 gradient quantization with LoCo error feedback.
//
// Definition ("Merge LoCo with Zero++", Overview: error feedback applied to
// the 4-bit gradients before communication; review thread: one EF buffer per
// parameter.  "ZeROPlusPlus.md" notes, section 1.2: qgZ block int4):
//   c = g + e;  s = absmax(c over the block) / 7;  k = clamp(rne(c / s), +-7)
//   e' = beta_e * e + beta_r * (c - k s)          (every step rounded in fp32)
//
// g is fp32, bf16 or fp16 (the LoCo kernel's half loads), widened to fp32
// exactly.  One pass over HBM: read g (4 or 2 B/elem) and e (4 B), write e (4 B),
// codes (0.5 B) and one fp32 scale per block.  Layout on the wave: a wave
// owns a tile of U sub-vectors of 256 elements; in sub-vector u lane l holds
// the 4 consecutive elements starting at u*256 + 4l, so every load and store
// instruction of the wave covers one contiguous span (1 KB of fp32).  A block
// of B <= 256 elements is B/4 adjacent lanes of one sub-vector (absmax by a
// DPP butterfly inside the lane group); a larger block is B/256 whole
// sub-vectors (in-lane max first, then the full-wave butterfly).  No LDS.
#include "zq_device.h"
#include "zq_launch.h"

#ifndef ZQ_EFQ_U
#define ZQ_EFQ_U 2  // sub-vectors of 256 elements per wave tile
#endif

namespace zq {
namespace {

template <int B>
struct EfqGeom {
    static constexpr int VEC = 4;
    static constexpr int SUB = kWave * VEC;
    static constexpr int LPB = B <= SUB ? B / VEC : kWave;
    static constexpr int SPB = B <= SUB ? 1 : B / SUB;
    static constexpr int U = SPB > ZQ_EFQ_U ? SPB : ZQ_EFQ_U;
    static constexpr int TILE = SUB * U;
    static constexpr int BPT = TILE / B;
};

// Where the codes and scales of element i go: the same place (plain
// quantize), or the slot of its partition (permuted quantize).  A tile lies
// in at most two partitions (partitions are at least a tile long), so the
// map is the offset of the tile's first partition below `bnd` and of the
// next one from `bnd` on.
struct IdentityMap {
    __device__ __forceinline__ size_t operator()(size_t i) const { return i; }
};

struct PermMap {
    size_t bnd;
    size_t d0, d1;  // added modulo 2^64 (a slot may lie before its partition)
    __device__ __forceinline__ size_t operator()(size_t i) const { return i + (i < bnd ? d0 : d1); }
};

__device__ __forceinline__ PermMap perm_map(const PartPerm& pp, size_t base) {
    const uint32_t p0 = __builtin_amdgcn_readfirstlane((uint32_t)(base / pp.part_len));
    PermMap m;
    m.bnd = (size_t)(p0 + 1) * pp.part_len;
    m.d0 = ((size_t)pp.slot[p0] - p0) * pp.part_len;
    m.d1 = p0 + 1 < pp.n_part ? ((size_t)pp.slot[p0 + 1] - (p0 + 1)) * pp.part_len : 0;
    return m;
}

template <int IN, bool EF, int B, bool MASK, class Map = IdentityMap>
__device__ __forceinline__ void efq_tile(const void* __restrict__ gv, float* __restrict__ ef,
                                         size_t n, float beta_e, float beta_r,
                                         uint8_t* __restrict__ codes, float* __restrict__ scales,
                                         size_t tile, const Map& out = Map()) {
    using G = EfqGeom<B>;
    const int lane = lane_id();
    const size_t base = tile * (size_t)G::TILE;

    float c[G::U][4];
    float e[G::U][4];

#pragma unroll
    for (int u = 0; u < G::U; ++u) {
        const size_t i0 = base + (size_t)u * G::SUB + (size_t)lane * 4;
        float gv4[4];
        if constexpr (!MASK) {
            if constexpr (IN != kF32) {
                u2 w = ld_stream((const u2*)((const uint16_t*)gv + i0));
                gv4[0] = half_lo<IN>(w.x);
                gv4[1] = half_hi<IN>(w.x);
                gv4[2] = half_lo<IN>(w.y);
                gv4[3] = half_hi<IN>(w.y);
            } else {
                f4 w = ld_stream((const f4*)((const float*)gv + i0));
                gv4[0] = w.x;
                gv4[1] = w.y;
                gv4[2] = w.z;
                gv4[3] = w.w;
            }
            if constexpr (EF) {
                f4 v = ld_stream((const f4*)(ef + i0));
                e[u][0] = v.x;
                e[u][1] = v.y;
                e[u][2] = v.z;
                e[u][3] = v.w;
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bool in = i0 + j < n;
                if constexpr (IN != kF32)
                    gv4[j] = in ? half_lo<IN>(((const uint16_t*)gv)[i0 + j]) : 0.0f;
                else
                    gv4[j] = in ? ((const float*)gv)[i0 + j] : 0.0f;
                if constexpr (EF)
                    e[u][j] = in ? ef[i0 + j] : 0.0f;
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
            c[u][j] = EF ? gv4[j] + e[u][j] : gv4[j];
    }

    // Block absmax and scale.
    BlockScale bs[G::SPB == 1 ? G::U : G::BPT];
    if constexpr (G::SPB == 1) {
#pragma unroll
        for (int u = 0; u < G::U; ++u) {
            uint32_t m = max(max(absbits(c[u][0]), absbits(c[u][1])),
                             max(absbits(c[u][2]), absbits(c[u][3])));
            bs[u] = block_scale<7>(group_max<G::LPB>(m));
        }
    } else {
#pragma unroll
        for (int b = 0; b < G::BPT; ++b) {
            uint32_t m = 0;
#pragma unroll
            for (int u = b * G::SPB; u < (b + 1) * G::SPB; ++u)
                m = max(m, max(max(absbits(c[u][0]), absbits(c[u][1])),
                               max(absbits(c[u][2]), absbits(c[u][3]))));
            bs[b] = block_scale<7>(group_max<kWave>(m));
        }
    }

    // Scales: one writer lane per block.
    if constexpr (G::SPB == 1) {
        if (lane % G::LPB == 0) {
#pragma unroll
            for (int u = 0; u < G::U; ++u) {
                const size_t i0 = base + (size_t)u * G::SUB + (size_t)lane * 4;
                if (!MASK || i0 < n)
                    scales[out(i0) / B] = bs[u].s;
            }
        }
    } else {
        if (lane == 0) {
#pragma unroll
            for (int b = 0; b < G::BPT; ++b) {
                const size_t i0 = base + (size_t)b * B;
                if (!MASK || i0 < n)
                    scales[out(i0) / B] = bs[b].s;
            }
        }
    }

    // Codes: fast reciprocal path for the whole tile, one rare fix-up branch.
    float kf[G::U][4];
    bool redo = false;
#pragma unroll
    for (int u = 0; u < G::U; ++u)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            kf[u][j] = code_fast<7>(c[u][j], bs[G::SPB == 1 ? u : u / G::SPB], redo);
    if (redo) {
#pragma unroll
        for (int u = 0; u < G::U; ++u)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                kf[u][j] = code_fix<7>(c[u][j], bs[G::SPB == 1 ? u : u / G::SPB], kf[u][j]);
    }

    // Residual, EF update, packing, stores.
#pragma unroll
    for (int u = 0; u < G::U; ++u) {
        const BlockScale& sc = bs[G::SPB == 1 ? u : u / G::SPB];
        const size_t i0 = base + (size_t)u * G::SUB + (size_t)lane * 4;
        uint32_t packed = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int k = code_clamp<7>(kf[u][j]);
            packed |= ((uint32_t)k & 0xFu) << (4 * j);
            if constexpr (EF)
                e[u][j] = ef_update(c[u][j], k, sc.s, e[u][j], beta_e, beta_r);
        }
        const size_t o0 = out(i0);
        if constexpr (!MASK) {
            st_stream((uint16_t)packed, (uint16_t*)(codes + o0 / 2));
            if constexpr (EF) {
                f4 v = {e[u][0], e[u][1], e[u][2], e[u][3]};
                st_stream(v, (f4*)(ef + i0));
            }
        } else {
            if (i0 < n)
                codes[o0 / 2] = (uint8_t)(packed & 0xFFu);
            if (i0 + 2 < n)
                codes[o0 / 2 + 1] = (uint8_t)(packed >> 8);
            if constexpr (EF) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (i0 + j < n)
                        ef[i0 + j] = e[u][j];
            }
        }
    }
}

// Full tiles without bounds checks; the ragged last tile (when n is not a
// multiple of the tile) goes, in the same launch, to the one wave whose loop
// stops exactly at it.  The two paths run one after the other, so their
// registers are not live at once.
template <int IN, bool EF, int B>
__global__ __launch_bounds__(kBlockThreads) void efq_kernel(const void* __restrict__ g,
                                                            float* __restrict__ ef, size_t n,
                                                            float beta_e, float beta_r,
                                                            uint8_t* __restrict__ codes,
                                                            float* __restrict__ scales) {
    using G = EfqGeom<B>;
    const size_t nfull = n / G::TILE;
    size_t t = stream_wave_id<kGeomStream.threads>();
    for (; t < nfull; t += wave_count())
        efq_tile<IN, EF, B, false>(g, ef, n, beta_e, beta_r, codes, scales, t);
    if (t == nfull && n % G::TILE)
        efq_tile<IN, EF, B, true>(g, ef, n, beta_e, beta_r, codes, scales, t);
}

template <int IN, bool EF, int B>
hipError_t launch_b(const void* g, float* ef, size_t n, float beta_e, float beta_r,
                    uint8_t* codes, float* scales, hipStream_t stream) {
    using G = EfqGeom<B>;
    const size_t ntiles = (n + G::TILE - 1) / G::TILE;
    void* args[] = {(void*)&g, (void*)&ef, (void*)&n, (void*)&beta_e, (void*)&beta_r,
                    (void*)&codes, (void*)&scales};
    return hipLaunchKernel((const void*)&efq_kernel<IN, EF, B>,
                           grid_for_tiles(ntiles, kGeomStream), dim3(kGeomStream.threads), args, 0,
                           stream);
}

template <int IN, bool EF, int B>
__global__ __launch_bounds__(kBlockThreads) void efq_perm_kernel(const void* __restrict__ g,
                                                                 float* __restrict__ ef, size_t n,
                                                                 float beta_e, float beta_r,
                                                                 uint8_t* __restrict__ codes,
                                                                 float* __restrict__ scales,
                                                                 PartPerm perm) {
    using G = EfqGeom<B>;
    const size_t nfull = n / G::TILE;
    size_t t = stream_wave_id<kGeomStream.threads>();
    for (; t < nfull; t += wave_count())
        efq_tile<IN, EF, B, false>(g, ef, n, beta_e, beta_r, codes, scales, t,
                                     perm_map(perm, t * G::TILE));
    if (t == nfull && n % G::TILE)
        efq_tile<IN, EF, B, true>(g, ef, n, beta_e, beta_r, codes, scales, t,
                                    perm_map(perm, t * G::TILE));
}

template <int IN, bool EF, int B>
hipError_t launch_perm_b(const void* g, float* ef, size_t n, float beta_e, float beta_r,
                         uint8_t* codes, float* scales, const PartPerm& perm, hipStream_t stream) {
    using G = EfqGeom<B>;
    const size_t ntiles = (n + G::TILE - 1) / G::TILE;
    PartPerm arg = perm;
    void* args[] = {(void*)&g, (void*)&ef, (void*)&n, (void*)&beta_e, (void*)&beta_r,
                    (void*)&codes, (void*)&scales, (void*)&arg};
    return hipLaunchKernel((const void*)&efq_perm_kernel<IN, EF, B>,
                           grid_for_tiles(ntiles, kGeomStream), dim3(kGeomStream.threads), args, 0,
                           stream);
}

template <int IN, bool EF>
hipError_t launch_perm_t(const void* g, float* ef, size_t n, uint32_t block, float be, float br,
                         uint8_t* codes, float* scales, const PartPerm& pp, hipStream_t st) {
    switch (block) {
        case 32: return launch_perm_b<IN, EF, 32>(g, ef, n, be, br, codes, scales, pp, st);
        case 64: return launch_perm_b<IN, EF, 64>(g, ef, n, be, br, codes, scales, pp, st);
        case 128: return launch_perm_b<IN, EF, 128>(g, ef, n, be, br, codes, scales, pp, st);
        case 256: return launch_perm_b<IN, EF, 256>(g, ef, n, be, br, codes, scales, pp, st);
        case 512: return launch_perm_b<IN, EF, 512>(g, ef, n, be, br, codes, scales, pp, st);
        case 1024: return launch_perm_b<IN, EF, 1024>(g, ef, n, be, br, codes, scales, pp, st);
        case 2048: return launch_perm_b<IN, EF, 2048>(g, ef, n, be, br, codes, scales, pp, st);
        case 4096: return launch_perm_b<IN, EF, 4096>(g, ef, n, be, br, codes, scales, pp, st);
        default: return hipErrorInvalidValue;
    }
}

// Batched segments.  One launch runs every tile of up to kEfqSegs segments:
// first all full tiles (a wave finds its segment from the cumulative
// full-tile counts in the kernel arguments, held one per lane: SegmentFinder),
// then the ragged last tiles, the k-th of which belongs to segment
// tail_seg[k].  80 segments (3.6 KB of kernel arguments) take the 7.5B
// model's 327 tensors in 5 launches.
#ifndef ZQ_EFQ_SEGS
#define ZQ_EFQ_SEGS 80
#endif
constexpr int kEfqSegs = ZQ_EFQ_SEGS;

struct EfqBatch {
    EfqSegment seg[kEfqSegs];
    uint32_t tile_end[kEfqSegs];  // cumulative full tiles through segment s
    uint8_t tail_seg[kEfqSegs];   // segment of the k-th ragged last tile
    uint32_t nseg;
    uint32_t full;   // full tiles of all segments
    uint32_t total;  // full + ragged tiles
    float beta_e, beta_r;
};
static_assert(kEfqSegs <= 256, "tail_seg holds 8-bit segment indices");

template <int IN, bool EF, int B>
__global__ __launch_bounds__(kBlockThreads) void efq_batched_kernel(EfqBatch b) {
    using G = EfqGeom<B>;
    const SegmentFinder<kEfqSegs> find(b.tile_end, b.nseg);
    size_t ts = stream_wave_id<kGeomStream.threads>();
    for (; ts < b.full; ts += wave_count()) {
        const uint32_t t = (uint32_t)ts;
        const uint32_t s = find(t);
        const EfqSegment& g = b.seg[s];
        const size_t local = t - (s ? b.tile_end[s - 1] : 0u);
        efq_tile<IN, EF, B, false>(g.g, g.ef, g.n, b.beta_e, b.beta_r, g.codes, g.scales, local);
    }
    for (; ts < b.total; ts += wave_count()) {
        const EfqSegment& g = b.seg[b.tail_seg[ts - b.full]];
        efq_tile<IN, EF, B, true>(g.g, g.ef, g.n, b.beta_e, b.beta_r, g.codes, g.scales,
                                    g.n / G::TILE);
    }
}

template <int IN, bool EF, int B>
hipError_t launch_batched_b(const EfqSegment* segs, uint32_t n_seg, float be, float br,
                            hipStream_t stream) {
    using G = EfqGeom<B>;
    uint32_t i = 0;
    while (i < n_seg) {
        EfqBatch bt = {};
        bt.beta_e = be;
        bt.beta_r = br;
        uint64_t full = 0, tails = 0;
        // A launch takes segments while its tile count (32-bit in the kernel's
        // table) stays below 2^32; one segment (at most 2^40 elements) has
        // fewer than 2^32 tiles.
        static_assert(G::TILE >= 512, "2^40-element segments need tiles of >= 512");
        while (i < n_seg && bt.nseg < (uint32_t)kEfqSegs) {
            const EfqSegment& g = segs[i];
            const uint64_t f = g.n / G::TILE, r = g.n % G::TILE ? 1 : 0;
            if (full + tails + f + r > UINT32_MAX)
                break;  // the next launch starts with this segment
            ++i;
            if (f + r == 0)
                continue;
            if (r)
                bt.tail_seg[tails++] = (uint8_t)bt.nseg;
            bt.seg[bt.nseg] = g;
            full += f;
            bt.tile_end[bt.nseg++] = (uint32_t)full;
        }
        if (bt.nseg == 0)
            continue;
        const uint64_t tiles = full + tails;
        bt.full = (uint32_t)full;
        bt.total = (uint32_t)tiles;
        void* args[] = {(void*)&bt};
        const hipError_t e =
            hipLaunchKernel((const void*)&efq_batched_kernel<IN, EF, B>,
                            grid_for_tiles(tiles, kGeomStream), dim3(kGeomStream.threads), args, 0,
                            stream);
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

template <int IN, bool EF>
hipError_t launch_batched_t(const EfqSegment* segs, uint32_t n_seg, uint32_t block, float be,
                            float br, hipStream_t st) {
    switch (block) {
        case 32: return launch_batched_b<IN, EF, 32>(segs, n_seg, be, br, st);
        case 64: return launch_batched_b<IN, EF, 64>(segs, n_seg, be, br, st);
        case 128: return launch_batched_b<IN, EF, 128>(segs, n_seg, be, br, st);
        case 256: return launch_batched_b<IN, EF, 256>(segs, n_seg, be, br, st);
        case 512: return launch_batched_b<IN, EF, 512>(segs, n_seg, be, br, st);
        case 1024: return launch_batched_b<IN, EF, 1024>(segs, n_seg, be, br, st);
        case 2048: return launch_batched_b<IN, EF, 2048>(segs, n_seg, be, br, st);
        case 4096: return launch_batched_b<IN, EF, 4096>(segs, n_seg, be, br, st);
        default: return hipErrorInvalidValue;
    }
}

template <int IN, bool EF>
hipError_t launch_t(const void* g, float* ef, size_t n, uint32_t block, float be, float br,
                    uint8_t* codes, float* scales, hipStream_t st) {
    switch (block) {
        case 32: return launch_b<IN, EF, 32>(g, ef, n, be, br, codes, scales, st);
        case 64: return launch_b<IN, EF, 64>(g, ef, n, be, br, codes, scales, st);
        case 128: return launch_b<IN, EF, 128>(g, ef, n, be, br, codes, scales, st);
        case 256: return launch_b<IN, EF, 256>(g, ef, n, be, br, codes, scales, st);
        case 512: return launch_b<IN, EF, 512>(g, ef, n, be, br, codes, scales, st);
        case 1024: return launch_b<IN, EF, 1024>(g, ef, n, be, br, codes, scales, st);
        case 2048: return launch_b<IN, EF, 2048>(g, ef, n, be, br, codes, scales, st);
        case 4096: return launch_b<IN, EF, 4096>(g, ef, n, be, br, codes, scales, st);
        default: return hipErrorInvalidValue;
    }
}

template <bool EF>
hipError_t launch_typed(const void* g, int g_type, float* ef, size_t n, uint32_t block, float be,
                        float br, uint8_t* codes, float* scales, hipStream_t st) {
    switch (g_type) {
        case kF32: return launch_t<kF32, EF>(g, ef, n, block, be, br, codes, scales, st);
        case kBF16: return launch_t<kBF16, EF>(g, ef, n, block, be, br, codes, scales, st);
        case kF16: return launch_t<kF16, EF>(g, ef, n, block, be, br, codes, scales, st);
        default: return hipErrorInvalidValue;
    }
}

template <bool EF>
hipError_t launch_batched_typed(const EfqSegment* segs, uint32_t n_seg, int g_type, uint32_t block,
                                float be, float br, hipStream_t st) {
    switch (g_type) {
        case kF32: return launch_batched_t<kF32, EF>(segs, n_seg, block, be, br, st);
        case kBF16: return launch_batched_t<kBF16, EF>(segs, n_seg, block, be, br, st);
        case kF16: return launch_batched_t<kF16, EF>(segs, n_seg, block, be, br, st);
        default: return hipErrorInvalidValue;
    }
}

template <bool EF>
hipError_t launch_perm_typed(const void* g, int g_type, float* ef, size_t n, uint32_t block,
                             float be, float br, uint8_t* codes, float* scales,
                             const PartPerm& perm, hipStream_t st) {
    switch (g_type) {
        case kF32: return launch_perm_t<kF32, EF>(g, ef, n, block, be, br, codes, scales, perm, st);
        case kBF16:
            return launch_perm_t<kBF16, EF>(g, ef, n, block, be, br, codes, scales, perm, st);
        case kF16: return launch_perm_t<kF16, EF>(g, ef, n, block, be, br, codes, scales, perm, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_quantize_ef_int4(const void* g, int g_type, float* ef, size_t n, uint32_t block,
                                   float beta_e, float beta_r, uint8_t* codes, float* scales,
                                   hipStream_t stream) {
    return ef ? launch_typed<true>(g, g_type, ef, n, block, beta_e, beta_r, codes, scales, stream)
              : launch_typed<false>(g, g_type, ef, n, block, beta_e, beta_r, codes, scales, stream);
}

hipError_t launch_quantize_ef_int4_batched(const EfqSegment* segs, uint32_t n_seg, int g_type,
                                           bool with_ef, uint32_t block, float beta_e,
                                           float beta_r, hipStream_t stream) {
    return with_ef ? launch_batched_typed<true>(segs, n_seg, g_type, block, beta_e, beta_r, stream)
                   : launch_batched_typed<false>(segs, n_seg, g_type, block, beta_e, beta_r, stream);
}

hipError_t launch_quantize_ef_int4_permuted(const void* g, int g_type, float* ef, size_t n,
                                            uint32_t block, float beta_e, float beta_r,
                                            uint8_t* codes, float* scales, const PartPerm& perm,
                                            hipStream_t stream) {
    return ef ? launch_perm_typed<true>(g, g_type, ef, n, block, beta_e, beta_r, codes, scales,
                                        perm, stream)
              : launch_perm_typed<false>(g, g_type, ef, n, block, beta_e, beta_r, codes, scales,
                                         perm, stream);
}

}  // namespace zq
