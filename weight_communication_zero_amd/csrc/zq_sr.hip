// zq_sr.hip -- bf16 gradient accumulation with stochastic rounding.
//
// Definition ("Zero 2 #593", review of llmc/cuda_utils.cuh: the accumulation
// adds the two bf16 values in fp32 and rounds the sum stochastically so it
// stays correct in expectation; review of llmc/zero.cuh: zeroing the reduced
// buffer can be folded into the same kernel):
//   x = float(dst) + float(src);  dst = SR_bf16(x, r16(seed, counter_base + i))
// r16 comes from Philox-4x32-10 at counter (q >> 3): one call gives the
// eight 16-bit numbers of indices 8c .. 8c+7.
//
// 6 B/elem (8 with zero_src).  In sub-vector u lane l owns the 8 elements
// starting at u*512 + 8l: one 16-byte load of dst and of src, one Philox
// call (two when counter_base is not a multiple of 8), one 16-byte store.
#include "zq_device.h"
#include "zq_launch.h"

namespace zq {
namespace {

#ifndef ZQ_SR_U
#define ZQ_SR_U 2
#endif
constexpr int kSrU = ZQ_SR_U;
constexpr int kSrSub = kWave * 8;
constexpr int kSrTile = kSrSub * kSrU;

// The random numbers of the 8 indices q0 .. q0+7 where q0 = 8*c + PHASE.
template <int PHASE>
__device__ __forceinline__ void r16x8(uint64_t c, uint32_t k0, uint32_t k1, uint32_t r[8]) {
    const Philox4 a = philox4x32_10((uint32_t)c, (uint32_t)(c >> 32), 0u, 0u, k0, k1);
    Philox4 b = a;
    if constexpr (PHASE != 0) {
        const uint64_t c1 = c + 1;
        b = philox4x32_10((uint32_t)c1, (uint32_t)(c1 >> 32), 0u, 0u, k0, k1);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int qq = PHASE + j;
        const uint32_t word = qq < 8 ? a.w[(qq & 7) >> 1] : b.w[(qq & 7) >> 1];
        r[j] = (qq & 1) ? (word >> 16) : (word & 0xFFFFu);
    }
}

template <int PHASE, bool ZERO, bool MASK>
__device__ __forceinline__ void sr_tile(uint16_t* __restrict__ dst, uint16_t* __restrict__ src,
                                        size_t n, uint32_t k0, uint32_t k1, uint64_t cbase8,
                                        size_t tile) {
    const int lane = lane_id();
    const size_t base = tile * (size_t)kSrTile;
    u4 d[kSrU], s[kSrU];
#pragma unroll
    for (int u = 0; u < kSrU; ++u) {
        const size_t i0 = base + (size_t)u * kSrSub + (size_t)lane * 8;
        if constexpr (!MASK) {
            d[u] = ld_stream((const u4*)(dst + i0));
            s[u] = ld_stream((const u4*)(src + i0));
        } else {
            uint32_t dv[4] = {0, 0, 0, 0}, sv[4] = {0, 0, 0, 0};
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (i0 + j < n) {
                    dv[j >> 1] |= (uint32_t)dst[i0 + j] << (16 * (j & 1));
                    sv[j >> 1] |= (uint32_t)src[i0 + j] << (16 * (j & 1));
                }
            d[u] = u4{dv[0], dv[1], dv[2], dv[3]};
            s[u] = u4{sv[0], sv[1], sv[2], sv[3]};
        }
    }
#pragma unroll
    for (int u = 0; u < kSrU; ++u) {
        const size_t i0 = base + (size_t)u * kSrSub + (size_t)lane * 8;
        uint32_t r[8];
        r16x8<PHASE>(cbase8 + (i0 >> 3), k0, k1, r);
        const uint32_t dw[4] = {d[u].x, d[u].y, d[u].z, d[u].w};
        const uint32_t sw[4] = {s[u].x, s[u].y, s[u].z, s[u].w};
        uint32_t o[4];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            const float x0 = bf16lo(dw[h]) + bf16lo(sw[h]);
            const float x1 = bf16hi(dw[h]) + bf16hi(sw[h]);
            o[h] = sr_bf16(x0, r[2 * h]) | (sr_bf16(x1, r[2 * h + 1]) << 16);
        }
        if constexpr (!MASK) {
            st_stream(u4{o[0], o[1], o[2], o[3]}, (u4*)(dst + i0));
            if constexpr (ZERO)
                st_stream(u4{0u, 0u, 0u, 0u}, (u4*)(src + i0));
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (i0 + j < n) {
                    dst[i0 + j] = (uint16_t)(o[j >> 1] >> (16 * (j & 1)));
                    if constexpr (ZERO)
                        src[i0 + j] = 0;
                }
        }
    }
}

// Full tiles and the ragged last tile in one launch: the tile past the last
// full one (when n is not a multiple of the tile) takes the masked path.
template <int PHASE, bool ZERO>
__global__ __launch_bounds__(kBlockThreads) void sr_kernel(uint16_t* __restrict__ dst,
                                                           uint16_t* __restrict__ src, size_t n,
                                                           uint32_t k0, uint32_t k1,
                                                           uint64_t cbase8) {
    const size_t nfull = n / kSrTile;
    const size_t ntiles = nfull + (n % kSrTile ? 1 : 0);
    for (size_t t = stream_wave_id<kGeomStream.threads>(); t < ntiles; t += wave_count()) {
        if (t < nfull)
            sr_tile<PHASE, ZERO, false>(dst, src, n, k0, k1, cbase8, t);
        else
            sr_tile<PHASE, ZERO, true>(dst, src, n, k0, k1, cbase8, t);
    }
}

template <int PHASE>
const void* sr_fn(bool zero) {
    return zero ? (const void*)&sr_kernel<PHASE, true> : (const void*)&sr_kernel<PHASE, false>;
}

const void* sr_pick(uint64_t counter_base, bool zero) {
    switch (counter_base & 7u) {
        case 0: return sr_fn<0>(zero);
        case 1: return sr_fn<1>(zero);
        case 2: return sr_fn<2>(zero);
        case 3: return sr_fn<3>(zero);
        case 4: return sr_fn<4>(zero);
        case 5: return sr_fn<5>(zero);
        case 6: return sr_fn<6>(zero);
        default: return sr_fn<7>(zero);
    }
}

// ---------------------------------------------------------------------------
// Batched segments: one launch runs the SR tiles of up to kSegsPerLaunch
// segments and, with zero_src, the tiles that clear the rest of each
// segment's source buffer.  The table (with cumulative tile counts) travels
// in the kernel arguments; a wave finds its segment from the cumulative
// counts, held one per lane (SegmentFinder).  Fewer launches pay: GPT-2's
// 148 tensors took 91 / 75.5 / 71 us with 16 / 32 / 50 segments per launch
// (MI355X, with the earlier per-entry scalar search); 50 keeps the table
// (3.2 KB) inside the 4 KB kernel-argument space.
#ifndef ZQ_SR_SEGS
#define ZQ_SR_SEGS 50
#endif
constexpr int kSegsPerLaunch = ZQ_SR_SEGS;

struct SrBatch {
    SrSegment seg[kSegsPerLaunch];
    uint32_t tile_end[kSegsPerLaunch];  // cumulative tiles (SR + zeroing) through segment s;
                                        // unused entries hold UINT32_MAX
    uint32_t sr_tiles[kSegsPerLaunch];  // SR tiles of segment s; the rest clear its buffer
    uint32_t total;                     // tiles of this launch (< 2^32 by construction)
    uint32_t zero;
};

template <int PHASE>
__device__ __forceinline__ void sr_group(const SrSegment& g, uint64_t e0, bool zero) {
    uint16_t* dst = g.dst;
    uint16_t* src = g.src + g.off;
    const uint32_t k0 = (uint32_t)g.seed, k1 = (uint32_t)(g.seed >> 32);
    uint32_t r[8];
    r16x8<PHASE>((g.cbase >> 3) + (e0 >> 3), k0, k1, r);
    if (e0 + 8 <= g.n) {
        const u4 d = ld_stream((const u4*)(dst + e0));
        const u4 s = ld_stream((const u4*)(src + e0));
        const uint32_t dw[4] = {d.x, d.y, d.z, d.w};
        const uint32_t sw[4] = {s.x, s.y, s.z, s.w};
        uint32_t o[4];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            const float x0 = bf16lo(dw[h]) + bf16lo(sw[h]);
            const float x1 = bf16hi(dw[h]) + bf16hi(sw[h]);
            o[h] = sr_bf16(x0, r[2 * h]) | (sr_bf16(x1, r[2 * h + 1]) << 16);
        }
        st_stream(u4{o[0], o[1], o[2], o[3]}, (u4*)(dst + e0));
        if (zero)
            st_stream(u4{0u, 0u, 0u, 0u}, (u4*)(src + e0));
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (e0 + j < g.n) {
                const float x = bf16lo(dst[e0 + j]) + bf16lo(src[e0 + j]);
                dst[e0 + j] = (uint16_t)sr_bf16(x, r[j]);
                if (zero)
                    src[e0 + j] = 0;
            }
        }
    }
}

// The counter phase (cbase & 7) is uniform per segment: one switch picks the
// specialised random-number layout.
__device__ __forceinline__ void sr_seg_tile(const SrSegment& g, uint64_t local, bool zero) {
    const int lane = lane_id();
    const uint32_t phase = __builtin_amdgcn_readfirstlane((uint32_t)(g.cbase & 7u));
#pragma unroll
    for (int u = 0; u < kSrU; ++u) {
        const uint64_t e0 = local * kSrTile + (uint64_t)u * kSrSub + (uint64_t)lane * 8;
        if (e0 >= g.n)
            continue;
        switch (phase) {
            case 0: sr_group<0>(g, e0, zero); break;
            case 1: sr_group<1>(g, e0, zero); break;
            case 2: sr_group<2>(g, e0, zero); break;
            case 3: sr_group<3>(g, e0, zero); break;
            case 4: sr_group<4>(g, e0, zero); break;
            case 5: sr_group<5>(g, e0, zero); break;
            case 6: sr_group<6>(g, e0, zero); break;
            default: sr_group<7>(g, e0, zero); break;
        }
    }
}

// Clear the part of the source buffer outside the read slice: position c of
// the complement (length len - n) is buffer element c (before the slice) or
// c + n (after it).
__device__ __forceinline__ void zero_seg_tile(const SrSegment& g, uint64_t local) {
    const int lane = lane_id();
    const uint64_t z = g.len - g.n;
#pragma unroll
    for (int u = 0; u < kSrU; ++u) {
        const uint64_t c0 = local * kSrTile + (uint64_t)u * kSrSub + (uint64_t)lane * 8;
        if (c0 >= z)
            continue;
        const uint64_t p0 = c0 < g.off ? c0 : c0 + g.n;
        const bool one_side = c0 + 8 <= g.off || c0 >= g.off;
        if (c0 + 8 <= z && one_side && (p0 & 7u) == 0) {
            st_stream(u4{0u, 0u, 0u, 0u}, (u4*)(g.src + p0));
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint64_t c = c0 + j;
                if (c < z)
                    g.src[c < g.off ? c : c + g.n] = 0;
            }
        }
    }
}

__global__ __launch_bounds__(kBlockThreads) void sr_batched_kernel(SrBatch b) {
    // Segment of tile t: the number of cumulative counts it has passed (a
    // scalar compare per entry measured 6 % slower on GPT-2's 148 tensors).
    const SegmentFinder<kSegsPerLaunch> find(b.tile_end, (uint32_t)kSegsPerLaunch);
    for (size_t ts = stream_wave_id<kGeomStream.threads>(); ts < b.total; ts += wave_count()) {
        const uint32_t t = (uint32_t)ts;
        const uint32_t s = find(t);
        const uint32_t local = t - (s ? b.tile_end[s - 1] : 0u);
        if (local < b.sr_tiles[s])
            sr_seg_tile(b.seg[s], local, b.zero != 0);
        else
            zero_seg_tile(b.seg[s], local - b.sr_tiles[s]);
    }
}

}  // namespace

hipError_t launch_sr_accumulate(uint16_t* dst, uint16_t* src, size_t n, uint64_t seed,
                                uint64_t counter_base, bool zero_src, hipStream_t stream) {
    uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
    uint64_t cbase8 = counter_base >> 3;
    const size_t ntiles = (n + kSrTile - 1) / kSrTile;
    void* args[] = {(void*)&dst, (void*)&src, (void*)&n, (void*)&k0, (void*)&k1, (void*)&cbase8};
    return hipLaunchKernel(sr_pick(counter_base, zero_src), grid_for_tiles(ntiles, kGeomStream),
                           dim3(kGeomStream.threads), args, 0, stream);
}

hipError_t launch_sr_accumulate_batched(const SrSegment* segs, uint32_t n_seg, bool zero_src,
                                        hipStream_t stream) {
    // Segments are at most 2^40 elements (checked by the ABI layer), so one
    // has at most 2^31 tiles; a launch takes segments while its tile count
    // (32-bit in the kernel's table) stays below 2^32.
    uint32_t i = 0;
    while (i < n_seg) {
        SrBatch b = {};
        b.zero = zero_src ? 1u : 0u;
        uint32_t nseg = 0;
        uint64_t tiles = 0;
        while (i < n_seg && nseg < (uint32_t)kSegsPerLaunch) {
            const SrSegment& g = segs[i];
            const uint64_t sr = (g.n + kSrTile - 1) / kSrTile;
            const uint64_t zt = zero_src ? (g.len - g.n + kSrTile - 1) / kSrTile : 0;
            if (tiles + sr + zt > UINT32_MAX)
                break;  // the next launch starts with this segment
            ++i;
            if (sr + zt == 0)
                continue;
            b.seg[nseg] = g;
            b.sr_tiles[nseg] = (uint32_t)sr;
            tiles += sr + zt;
            b.tile_end[nseg] = (uint32_t)tiles;
            ++nseg;
        }
        if (nseg == 0)
            continue;
        for (uint32_t k = nseg; k < (uint32_t)kSegsPerLaunch; ++k)
            b.tile_end[k] = UINT32_MAX;
        b.total = (uint32_t)tiles;
        void* args[] = {(void*)&b};
        const hipError_t e = hipLaunchKernel((const void*)&sr_batched_kernel,
                                             grid_for_tiles(tiles, kGeomStream),
                                             dim3(kGeomStream.threads), args, 0, stream);
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

}  // namespace zq
