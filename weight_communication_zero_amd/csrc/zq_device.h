// zq_device.h -- device helpers shared by the libzq kernels (gfx950, wave64).
//
// Everything here is register-level: 16-byte vector types, DPP / permlane
// cross-lane maxima, bf16 conversion, the int4/int8 block quantizer step and
// Philox-4x32-10.  Nothing here allocates or touches LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "zq_launch.h"

namespace zq {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));

// Streaming memory hints: data read or written once goes through the cache
// hierarchy with the nontemporal bit (global_load/store ... nt), so it does
// not evict what other waves still need.  Build-time switches for tuning.
#ifndef ZQ_NT_LOAD
#define ZQ_NT_LOAD 1
#endif
#ifndef ZQ_NT_STORE
#define ZQ_NT_STORE 1
#endif

template <typename T>
__device__ __forceinline__ T ld_stream(const T* p) {
    if constexpr (ZQ_NT_LOAD)
        return __builtin_nontemporal_load(p);
    else
        return *p;
}

template <typename T>
__device__ __forceinline__ void st_stream(T v, T* p) {
    if constexpr (ZQ_NT_STORE)
        __builtin_nontemporal_store(v, p);
    else
        *p = v;
}

constexpr int kWave = 64;
// Workgroups hold 1 to 4 waves (chosen per kernel at launch); kernels are
// compiled for the largest.
constexpr int kBlockThreads = 256;

__device__ __forceinline__ uint32_t fbits(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ __forceinline__ float bitsf(uint32_t u) { return __builtin_bit_cast(float, u); }

// bf16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float bf16lo(uint32_t w) { return bitsf(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return bitsf(w & 0xFFFF0000u); }

// IEEE binary16 bit pattern -> fp32 (exact, subnormals included:
// v_cvt_f32_f16, the high half through the operand word select).
__device__ __forceinline__ float f16lo(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)w);
}
__device__ __forceinline__ float f16hi(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// Low / high 16-bit element of a word of bf16 or fp16 values, as fp32.
template <int T>
__device__ __forceinline__ float half_lo(uint32_t w) {
    static_assert(T == kBF16 || T == kF16, "16-bit element types only");
    if constexpr (T == kBF16)
        return bf16lo(w);
    else
        return f16lo(w);
}
template <int T>
__device__ __forceinline__ float half_hi(uint32_t w) {
    static_assert(T == kBF16 || T == kF16, "16-bit element types only");
    if constexpr (T == kBF16)
        return bf16hi(w);
    else
        return f16hi(w);
}

// Two fp32 -> packed bf16 pair, round to nearest even (gfx950 v_cvt_pk_bf16_f32).
// Only used on finite values.
__device__ __forceinline__ uint32_t pack_bf16_rne(float lo, float hi) {
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    bf2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// Two fp32 -> packed IEEE binary16 pair, round to nearest even (the MODE
// register's default rounding; not the round-toward-zero pkrtz form);
// magnitudes from 65520 up become infinity, small ones fp16 subnormals.
__device__ __forceinline__ uint32_t pack_f16_rne(float lo, float hi) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    h2 v = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

template <int T>
__device__ __forceinline__ uint32_t pack_half_rne(float lo, float hi) {
    static_assert(T == kBF16 || T == kF16, "16-bit element types only");
    if constexpr (T == kBF16)
        return pack_bf16_rne(lo, hi);
    else
        return pack_f16_rne(lo, hi);
}

// |x| as an unsigned bit pattern: for non-NaN values its unsigned order is
// the order of the magnitudes, so a max over these bits is the exact absmax.
__device__ __forceinline__ uint32_t absbits(float x) { return fbits(x) & 0x7FFFFFFFu; }

// ---------------------------------------------------------------------------
// Maximum over aligned groups of G consecutive lanes (G a power of two <= 64);
// every lane of the group receives the group maximum.  Butterfly on DPP:
// quad_perm swaps (xor 1, xor 2), row half-mirror (pairs quads within 8),
// row mirror (pairs half-rows within 16), ds_swizzle xor 16 (within 32), and
// gfx950's v_permlane32_swap (exchanges the two 32-lane halves).
// The DPP steps are written with bound_ctrl and an identity (0) old value,
// so the compiler fuses each move into the maximum (v_max_u32_dpp).
template <int G>
__device__ __forceinline__ uint32_t group_max(uint32_t v) {
    if constexpr (G >= 2)
        v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, true));
    if constexpr (G >= 4)
        v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, true));
    if constexpr (G >= 8)
        v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, true));
    if constexpr (G >= 16)
        v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, true));
    if constexpr (G >= 32)
        v = max(v, (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F));
    if constexpr (G >= 64) {
        auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        v = max((uint32_t)r[0], (uint32_t)r[1]);
    }
    return v;
}

// ---------------------------------------------------------------------------
// Block scale of the symmetric quantizer: s = fl(a / qmax) by IEEE division.
//
// The per-element quotient fl(x / s) matters only through round-half-even to
// an integer, so it is first formed as y = x * rcp(s) (v_rcp_f32, relative
// error <= 2^-23).  With |x / s| <= qmax + 1/2, y differs from the exact
// ratio by at most 1.5 (qmax + 1/2) 2^-23 and the IEEE quotient by at most
// half an ulp of it: together < 2^-19.2 for qmax = 7 and < 2^-15.2 for
// qmax = 127.  Whenever y is farther than `band` (2^-17 resp. 2^-14) from a
// half-integer, y and the IEEE quotient lie on the same side of every
// rounding boundary and round to the same integer.  Elements inside the band
// -- and every element of a block whose scale is subnormal, where the
// reciprocal is not well scaled -- take the IEEE quotient instead.  A zero
// scale has reciprocal 0 and gives code 0.
struct BlockScale {
    float s;
    float inv;
    bool exact;
};

template <int QMAX>
__device__ __forceinline__ BlockScale block_scale(uint32_t amax_bits) {
    BlockScale b;
    b.s = bitsf(amax_bits) / (float)QMAX;
    b.exact = (b.s != 0.0f) && (b.s < 0x1p-126f);
    b.inv = (b.s == 0.0f) ? 0.0f : __builtin_amdgcn_rcpf(b.s);
    return b;
}

template <int QMAX>
__device__ __forceinline__ constexpr float tie_band() {
    static_assert(QMAX == 7 || QMAX == 127, "band derived for qmax 7 and 127 only");
    return QMAX == 7 ? 0.5f - 0x1p-17f : 0.5f - 0x1p-14f;
}

// Fast code (before clamping); sets `redo` when the IEEE quotient must decide.
template <int QMAX>
__device__ __forceinline__ float code_fast(float x, const BlockScale& b, bool& redo) {
    const float y = x * b.inv;
    const float k = rintf(y);
    redo |= b.exact | (__builtin_fabsf(y - k) > tie_band<QMAX>());
    return k;
}

// Rare path: recompute with the IEEE quotient where the fast code is unsafe.
// The clamp to [-qmax, qmax] is only reachable here: with s = fl(a / qmax)
// every |x| <= a gives |x / s| <= qmax (1 + 2^-24) and |x * rcp(s)| <=
// qmax (1 + 2^-22), both below qmax + 1/2, so outside a subnormal-scale block
// no code can leave the range.
template <int QMAX>
__device__ __forceinline__ float code_fix(float x, const BlockScale& b, float k) {
    const float y = x * b.inv;
    if (b.exact || __builtin_fabsf(y - rintf(y)) > tie_band<QMAX>()) {
        k = rintf(x / b.s);
        k = __builtin_fminf(__builtin_fmaxf(k, -(float)QMAX), (float)QMAX);
    }
    return k;
}

// Integer code of a (fast or fixed) rounded quotient.
template <int QMAX>
__device__ __forceinline__ int code_clamp(float k) {
    return (int)k;
}

// Residual of the error-feedback quantizer and the new EF value:
//   d = fl(k s), r = fl(c - d), e' = fl(fl(be e) + fl(br r)).
// Built without -ffp-contract, so every product and sum rounds separately.
__device__ __forceinline__ float ef_update(float c, int k, float s, float e, float be, float br) {
    float d = (float)k * s;
    float r = c - d;
    float t1 = be * e;
    float t2 = br * r;
    return t1 + t2;
}

// ---------------------------------------------------------------------------
// Philox-4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11).  Each round takes the
// 32x32->64 products of words 0 and 2 with the two round multipliers and
// forms the new state from their halves, the other two words and the round
// key; the key advances by the two Weyl increments between rounds.  The key
// is uniform across the wave, so its schedule stays in scalar registers.
struct Philox4 {
    uint32_t w[4];
};

__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                                 uint32_t k0, uint32_t k1) {
    constexpr uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
    constexpr uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        uint64_t p0 = (uint64_t)M0 * c0;
        uint64_t p1 = (uint64_t)M1 * c2;
        uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        uint32_t n1 = (uint32_t)p1;
        uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        uint32_t n3 = (uint32_t)p0;
        c0 = n0;
        c1 = n1;
        c2 = n2;
        c3 = n3;
        k0 += W0;
        k1 += W1;
    }
    Philox4 o;
    o.w[0] = c0;
    o.w[1] = c1;
    o.w[2] = c2;
    o.w[3] = c3;
    return o;
}

// Stochastic rounding of fp32 x to bf16 with a 16-bit random number: add it
// below the kept 16 bits and truncate; NaN gives the canonical quiet NaN.
__device__ __forceinline__ uint32_t sr_bf16(float x, uint32_t r16) {
    uint32_t u = fbits(x);
    uint32_t h = (u + r16) >> 16;
    return (x != x) ? 0x7FC0u : h;
}

// ---------------------------------------------------------------------------
// Launch geometry shared by the streaming kernels: a wave owns whole tiles
// (a multiple of the quantization block), walking them with a grid stride
// when the grid is capped.
__device__ __forceinline__ size_t wave_id() {
    // threadIdx.x >> 6 is the same on every lane of a wave; say so, so that
    // tile bases and segment lookups stay in scalar registers.
    const uint32_t w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    return (size_t)blockIdx.x * (blockDim.x >> 6) + w;
}
__device__ __forceinline__ size_t wave_count() { return (size_t)gridDim.x * (blockDim.x >> 6); }

// The same wave index with the workgroups taken in an XCD-aware order, for a
// grid of THREADS-thread workgroups that each own THREADS / 64 tiles.  The
// dispatcher hands workgroup b to XCD b % 8 (MI355X has 8 XCDs, each with its
// own L2).  Within every block of 8 C consecutive workgroups, XCD x takes the
// C workgroups starting at x C, so each XCD streams one contiguous run of
// ZQ_XCD_CHUNK tiles at a time instead of every eighth workgroup; a trailing
// partial block keeps the dispatch order.  The map permutes the workgroup
// indices, so each tile is still visited exactly once.  ZQ_XCD_CHUNK = 0
// turns it off.
#ifndef ZQ_XCD_CHUNK
#define ZQ_XCD_CHUNK 16384
#endif
template <uint32_t THREADS>
__device__ __forceinline__ size_t stream_wave_id() {
    constexpr size_t WPG = THREADS / kWave;
    constexpr size_t C = ZQ_XCD_CHUNK / WPG;
    size_t b = blockIdx.x;
    if constexpr (C > 0) {
        const size_t full = (size_t)gridDim.x / (8 * C) * (8 * C);
        if (b < full)
            b = b / (8 * C) * (8 * C) + (b % 8) * C + (b / 8) % C;
    }
    return b * WPG + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}
__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }

// Segment lookup of the batched kernels.  `ends` holds the segments'
// cumulative tile counts (non-decreasing; entries from nseg on are ignored),
// and the segment of tile t is the number of entries <= t.  Lane k keeps
// entries k and k + 64 in registers, so a lookup is one or two vector
// compares and the population counts of their ballots: a few instructions
// instead of a chain of dependent scalar loads (binary search) or a scalar
// compare per entry (scan), both of which load the compute unit's one scalar
// ALU on every tile.
template <int N>
struct SegmentFinder {
    uint32_t e0, e1;
    __device__ __forceinline__ SegmentFinder(const uint32_t (&ends)[N], uint32_t nseg) {
        const uint32_t lane = (uint32_t)lane_id();
        e0 = lane < nseg ? ends[lane] : UINT32_MAX;
        e1 = UINT32_MAX;
        if constexpr (N > kWave)
            e1 = lane + kWave < nseg ? ends[lane + kWave] : UINT32_MAX;
    }
    __device__ __forceinline__ uint32_t operator()(uint32_t t) const {
        static_assert(N <= 2 * kWave, "two table entries per lane at most");
        uint32_t s = (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(t >= e0));
        if constexpr (N > kWave)
            s += (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(t >= e1));
        return s;
    }
};

}  // namespace zq
