// zq_dr_kernels.h -- qgZ receive side: dequantize P int4 chunks, reduce in fp32,
// optionally requantize (with optional error feedback) for the next level.
//
// Definition ("ZeROPlusPlus.md" notes, section 1.2: gradients travel as
// block int4 through an all-to-all, the reduction is done back in full
// precision, inside the node first and then across nodes, with fused
// kernels to cut latency):
//   S = d_0 + d_1 + ... + d_{P-1}   (left to right, d_p = fl(k_p s_p))
//   R = alpha * S;  out = R;  requant: the EF int4 quantizer applied to R.
//
// One pass: P * (0.5 B + 4/B B) read per output element, 4 B written when
// out is requested, 0.5 B + 4/B B (+8 B with requant EF) for the requant.
// In sub-vector u lane l owns the VEC outputs starting at u*64*VEC + VEC*l:
// VEC = 8 for the requant without EF (one 32-bit word of codes per peer, so
// each code load instruction of the wave reads 256 contiguous bytes), 4 for
// the fp32-out reduce and the requant with EF.  The sum order is fixed (ascending peer), so
// the fp32 sums -- and the requant codes that depend on their exact bits --
// are deterministic.  No LDS.
#pragma once

#include <type_traits>

#include "zq_device.h"
#include "zq_dr_launch.h"
#include "zq_launch.h"

#ifndef ZQ_DR_U
#define ZQ_DR_U 2  // sub-vectors of 512 outputs per wave tile
#endif

namespace zq {
namespace {

// VEC outputs per lane per sub-vector: 8 (one 32-bit code word per peer,
// two 16-byte output stores per lane) or 4 (one 16-bit code word per peer,
// one 16-byte store per lane, so each store instruction writes 1 KB
// contiguously).  Both keep 16 outputs per lane per tile.
#ifndef ZQ_DR_VEC_OUT
#define ZQ_DR_VEC_OUT 4
#endif
#ifndef ZQ_DR_VEC_RQ
#define ZQ_DR_VEC_RQ 8
#endif
// With requant EF (two more fp32 streams per output) 4 outputs per lane per
// sub-vector measured best: 1.96 against 2.16 ms at 7.5B / 8 peers, while
// the requant without EF is issue-bound and prefers 8 (0.97 against 1.23 ms).
#ifndef ZQ_DR_VEC_RQEF
#define ZQ_DR_VEC_RQEF 4
#endif
#ifndef ZQ_DR_U_RQEF
#define ZQ_DR_U_RQEF ZQ_DR_U
#endif
#ifndef ZQ_DR_U_RQ
#define ZQ_DR_U_RQ ZQ_DR_U
#endif

template <int B, int V, int UB>
struct DrGeom {
    static constexpr int VEC = V;
    static constexpr int SUB = kWave * VEC;
    static constexpr int LPB = B <= SUB ? B / VEC : kWave;
    static constexpr int SPB = B <= SUB ? 1 : B / SUB;
    static constexpr int U0 = UB * 8 / VEC;
    static constexpr int U = SPB > U0 ? SPB : U0;
    static constexpr int TILE = SUB * U;
    static constexpr int BPT = TILE / B;
};

// Tile geometry of each kernel flavour: fp32 output only, requant, requant
// with its error-feedback buffer.
template <int B, bool RQ, bool EF>
using DrGeomOf = DrGeom<B, RQ ? (EF ? ZQ_DR_VEC_RQEF : ZQ_DR_VEC_RQ) : ZQ_DR_VEC_OUT,
                        RQ ? (EF ? ZQ_DR_U_RQEF : ZQ_DR_U_RQ) : ZQ_DR_U>;

template <int V>
using code_word_t = typename std::conditional<V == 8, uint32_t, uint16_t>::type;

// Signed value of nibble j of a code word (shift it to the top, then an
// arithmetic shift back down sign-extends it).
__device__ __forceinline__ float nib(uint32_t w, int j) {
    return (float)((int32_t)(w << (28 - 4 * j)) >> 28);
}

// The same nibbles divided by 16, from gfx950's v_cvt_off_f32_i4: it reads
// bits [3:0] of its operand as a two's-complement int4 k and returns k / 16,
// which is exact.  Even nibbles are the low halves of the word's bytes, odd
// nibbles those of the word shifted right by 4, and the instruction's operand
// byte select picks the byte, so V nibbles cost V conversions and one shift
// (the empty asm hides the shifted word from the compiler, which would
// otherwise fold the shift into a bit-field extract per nibble).  With
// t = fl(16 s) finite, fl((k / 16) t) = fl(k s) bit for bit: both factors are
// exact and their exact product is k s.  Measured A/B in one process at 7.5B
// / 8 peers, requant without EF: 0.946 -> 0.922 ms; the fp32-out reduce
// gained nothing and keeps the integer decode (ZQ_DR_DECODE_OFF=0 turns the
// k / 16 decode off everywhere).
#ifndef ZQ_DR_DECODE_OFF
#define ZQ_DR_DECODE_OFF 1
#endif
__device__ __forceinline__ float off4(uint32_t v) { return __builtin_amdgcn_cvt_off_f32_i4((int)v); }

template <int V>
__device__ __forceinline__ void nib16(uint32_t w, float (&f)[V]) {
    uint32_t y = w >> 4;
    asm("" : "+v"(y));
    f[0] = off4(w);
    f[1] = off4(y);
    f[2] = off4((w >> 8) & 0xFFu);
    f[3] = off4((y >> 8) & 0xFFu);
    if constexpr (V == 8) {
        f[4] = off4((w >> 16) & 0xFFu);
        f[5] = off4((y >> 16) & 0xFFu);
        f[6] = off4(w >> 24);
        f[7] = off4(y >> 24);
    }
}

// Same rounding as code_fast, by the addition of 1.5 * 2^23: for |y| < 2^22
// the sum lies in [2^23, 2^24), where the fp32 spacing is 1, so it rounds y
// half-to-even onto the integers (1.5 * 2^23 is even) and the subtraction
// recovers rne(y) exactly -- as +0 where rintf gives -0, which the integer
// code does not see.  The caller guarantees a finite block scale, so
// |y| <= qmax (1 + 2^-22) unless `redo` is set anyway.
#ifndef ZQ_DR_FMA_ROUND
#define ZQ_DR_FMA_ROUND 1
#endif
template <int QMAX>
__device__ __forceinline__ float code_fast_rne(float x, const BlockScale& b, bool& redo) {
    if constexpr (ZQ_DR_FMA_ROUND) {
        // The same code from the exact product z = x rcp(s): fma(x, rcp(s),
        // 1.5 2^23) rounds z itself onto the integers, and fma(x, rcp(s), -k)
        // is z - k to 2^-25.  With |z - x / s| < 2^-20 and fl(x / s) within
        // 2^-22 of x / s, a distance of at least 2^-17 - 2^-25 from every
        // half-integer puts z and fl(x / s) on the same side of it, so outside
        // the tie band k = rne(fl(x / s)).  Three dual-issue FMA/add
        // instructions instead of four.
        const float k = __builtin_fmaf(x, b.inv, 0x1.8p23f) - 0x1.8p23f;
        redo |= __builtin_fabsf(__builtin_fmaf(x, b.inv, -k)) > tie_band<QMAX>();
        return k;
    } else {
        const float y = x * b.inv;
        const float k = (y + 0x1.8p23f) - 0x1.8p23f;
        redo |= __builtin_fabsf(y - k) > tie_band<QMAX>();
        return k;
    }
}

// Two's-complement nibbles of V (4 or 8) integer-valued floats in [-7, 7],
// element j in bits 4j..4j+3.  Per group of four the biased digits k_j + 8
// lie in [1, 15], so W = sum (k_j + 8) 16^j has no carries between digits;
// it is an integer below 2^16, exact in fp32, and adding 1.5 * 2^23 puts it
// in the low mantissa bits (the bias 0x8888 rides on that constant).
// Flipping bit 3 of every digit (xor 0x8...8) then gives k_j mod 16.  The
// two groups of eight are joined by a byte permute.
template <int V>
__device__ __forceinline__ uint32_t pack_nibbles_f(const float (&k)[V]) {
    uint32_t h[2];
#pragma unroll
    for (int g = 0; g < V / 4; ++g) {
        const float lo = __builtin_fmaf(k[4 * g + 1], 16.0f, k[4 * g]);
        const float hi = __builtin_fmaf(k[4 * g + 3], 16.0f, k[4 * g + 2]);
        h[g] = fbits(__builtin_fmaf(hi, 256.0f, lo) + (0x1.8p23f + (float)0x8888));
    }
    if constexpr (V == 8)
        return __builtin_amdgcn_perm(h[1], h[0], 0x05040100u) ^ 0x88888888u;
    else
        return (h[0] ^ 0x8888u) & 0xFFFFu;
}

// ef_update with the code given as an exact integer-valued float (+0 for 0).
__device__ __forceinline__ float ef_update_f(float c, float k, float s, float e, float be, float br) {
    float d = k * s;
    float r = c - d;
    float t1 = be * e;
    float t2 = br * r;
    return t1 + t2;
}

// Wave-uniform copy of a value that every lane holds, in scalar registers.
__device__ __forceinline__ size_t uniform64(size_t x) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
    return ((size_t)hi << 32) | lo;
}

// Buffer addressing for the issue-bound requant without EF: every stream of
// a full tile is read and written through a raw buffer resource built in
// scalar registers from the tile's base address, with a 32-bit per-lane
// byte offset, so no 64-bit address arithmetic runs on the vector ALU.  The
// resource spans the tile's bytes of that stream (the offsets stay inside).
// Word 3 is the gfx9-family raw-buffer format word; cache-policy bit 1 is
// the nontemporal hint.  Measured A/B in one process at 7.5B / 8 peers:
// 1.027 -> 0.969 ms for this kernel, while the fp32-out reduce (+1.6 %) and
// the requant with EF (equal) keep plain global accesses.
template <typename T, int POLICY>
__device__ __forceinline__ T buf_load(const void* base, uint32_t bytes, uint32_t off) {
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
    if constexpr (sizeof(T) == 2)
        return __builtin_bit_cast(T, (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, POLICY));
    else if constexpr (sizeof(T) == 4)
        return __builtin_bit_cast(T, (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, POLICY));
    else
        return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, POLICY));
}
template <typename T, int POLICY>
__device__ __forceinline__ void buf_store(T v, void* base, uint32_t bytes, uint32_t off) {
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(base, (short)0, (int)bytes, 0x00020000);
    if constexpr (sizeof(T) == 2)
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, v), r, off, 0, POLICY);
    else if constexpr (sizeof(T) == 4)
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, off, 0, POLICY);
    else
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, v), r, off, 0, POLICY);
}
constexpr int kBufLoadNT = ZQ_NT_LOAD ? 2 : 0;
constexpr int kBufStoreNT = ZQ_NT_STORE ? 2 : 0;

// Up to NB code bytes starting at byte offset ob, only those below nbytes.
template <int NB>
__device__ __forceinline__ uint32_t load_code_word_masked(const uint8_t* p, size_t ob,
                                                          size_t nbytes) {
    uint32_t w = 0;
#pragma unroll
    for (int b = 0; b < NB; ++b)
        if (ob + b < nbytes)
            w |= (uint32_t)p[ob + b] << (8 * b);
    return w;
}

// The code words and scales of every peer for one tile (see dr_tile).
template <int B, int PMAX, bool RQ, bool EF, bool MASK, typename PV>
__device__ __forceinline__ void dr_load(const PV& p, size_t base,
                                        uint32_t (&cw)[PMAX][DrGeomOf<B, RQ, EF>::U],
                                        float (&sc)[PMAX][DrGeomOf<B, RQ, EF>::U]) {
    using G = DrGeomOf<B, RQ, EF>;
    constexpr int V = G::VEC;
    constexpr bool BUF = RQ && !EF && !MASK;  // buffer addressing (see buf_load)
    const int lane = lane_id();
    const size_t n = p.n;
    const size_t nbytes = (n + 1) / 2;
#pragma unroll
    for (int q = 0; q < PMAX; ++q) {
        if (q < (int)p.P) {
#pragma unroll
            for (int u = 0; u < G::U; ++u) {
                const size_t i0 = base + (size_t)u * G::SUB + (size_t)lane * V;
                if constexpr (BUF) {
                    const uint32_t le = (uint32_t)(u * G::SUB + lane * V);
                    cw[q][u] = buf_load<code_word_t<V>, kBufLoadNT>(p.codes_of(q) + base / 2,
                                                                    G::TILE / 2, le / 2);
                    sc[q][u] = buf_load<float, 0>(p.scales_of(q) + base / B, G::TILE / B * 4,
                                                  4u * (le / B));
                } else if constexpr (!MASK) {
                    cw[q][u] = ld_stream((const code_word_t<V>*)(p.codes_of(q) + i0 / 2));
                    sc[q][u] = p.scales_of(q)[i0 / B];
                } else {
                    cw[q][u] = load_code_word_masked<V / 2>(p.codes_of(q), i0 / 2, nbytes);
                    sc[q][u] = i0 < n ? p.scales_of(q)[i0 / B] : 0.0f;
                }
            }
        }
    }
}

// S = d_0 + d_1 + ..., ascending peer order, d = fl(k s) from the integer
// nibble.  Peers are the outer loop so the runtime test q < P is one uniform
// branch per peer, not a select per element.
template <int PMAX, int U, int V, typename PV>
__device__ __forceinline__ void dr_sum_int(const PV& p, const uint32_t (&cw)[PMAX][U],
                                           const float (&sc)[PMAX][U], float (&R)[U][V]) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int j = 0; j < V; ++j)
            R[u][j] = nib(cw[0][u], j) * sc[0][u];
#pragma unroll
    for (int q = 1; q < PMAX; ++q) {
        if (q < (int)p.P) {
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int j = 0; j < V; ++j)
                    R[u][j] = R[u][j] + nib(cw[q][u], j) * sc[q][u];
        }
    }
}

// The same sum from k / 16 (v_cvt_off_f32_i4) times t = fl(16 s).  For
// |s| < 2^124, t = 16 s exactly and every term equals fl(k s) bit for bit.
// A larger, infinite or NaN s makes t infinite or NaN, so every term of that
// block is infinite or NaN (a zero code gives 0 * inf = NaN) and so is every
// sum of the block: the caller checks for that and redoes such a tile with
// dr_sum_int.
template <int PMAX, int U, int V, typename PV>
__device__ __forceinline__ void dr_sum_off(const PV& p, const uint32_t (&cw)[PMAX][U],
                                           const float (&sc)[PMAX][U], float (&R)[U][V]) {
    float f[V];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const float t = sc[0][u] * 16.0f;
        nib16<V>(cw[0][u], f);
#pragma unroll
        for (int j = 0; j < V; ++j)
            R[u][j] = f[j] * t;
    }
#pragma unroll
    for (int q = 1; q < PMAX; ++q) {
        if (q < (int)p.P) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const float t = sc[q][u] * 16.0f;
                nib16<V>(cw[q][u], f);
#pragma unroll
                for (int j = 0; j < V; ++j)
                    R[u][j] = R[u][j] + f[j] * t;
            }
        }
    }
}

// dr_sum_int for one full tile, reloading the inputs one peer at a time in a
// rolled loop: the rare redo path of the k / 16 decode, kept small so that
// it adds no register pressure to the common path.
template <int B, typename G, typename PV>
__device__ __forceinline__ void dr_sum_int_reload(const PV& p, size_t base,
                                                  float (&R)[G::U][G::VEC]) {
    constexpr int V = G::VEC;
    const int lane = lane_id();
#pragma nounroll
    for (uint32_t q = 0; q < p.P; ++q) {
        const uint8_t* codes = p.codes_of(q);
        const float* scales = p.scales_of(q);
#pragma unroll
        for (int u = 0; u < G::U; ++u) {
            const size_t i0 = base + (size_t)u * G::SUB + (size_t)lane * V;
            const uint32_t w = *(const code_word_t<V>*)(codes + i0 / 2);
            const float s = scales[i0 / B];
#pragma unroll
            for (int j = 0; j < V; ++j)
                R[u][j] = q == 0 ? nib(w, j) * s : R[u][j] + nib(w, j) * s;
        }
    }
}

// dr_sum_int for the ragged last tile: inputs past the chunk read as zero
// (code bytes past ceil(n / 2), scales of blocks past n), one peer at a time
// in a rolled loop so that no block size or peer count needs more registers
// than one peer's words.
template <int B, typename G, typename PV>
__device__ __forceinline__ void dr_sum_masked(const PV& p, size_t base, float (&R)[G::U][G::VEC]) {
    constexpr int V = G::VEC;
    const int lane = lane_id();
    const size_t n = p.n;
    const size_t nbytes = (n + 1) / 2;
#pragma nounroll
    for (uint32_t q = 0; q < p.P; ++q) {
        const uint8_t* codes = p.codes_of(q);
        const float* scales = p.scales_of(q);
#pragma unroll
        for (int u = 0; u < G::U; ++u) {
            const size_t i0 = base + (size_t)u * G::SUB + (size_t)lane * V;
            const uint32_t w = load_code_word_masked<V / 2>(codes, i0 / 2, nbytes);
            const float s = i0 < n ? scales[i0 / B] : 0.0f;
#pragma unroll
            for (int j = 0; j < V; ++j)
                R[u][j] = q == 0 ? nib(w, j) * s : R[u][j] + nib(w, j) * s;
        }
    }
}

// R = alpha R, skipped for alpha = 1 (multiplying by one is the identity).
template <int U, int V, typename PV>
__device__ __forceinline__ void dr_alpha(const PV& p, float (&R)[U][V]) {
    if (p.alpha != 1.0f) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int j = 0; j < V; ++j)
                R[u][j] = p.alpha * R[u][j];
    }
}

// Block scale of the requant: s = fl(a / 7) from q0 = a fl(1/7),
// e = fma(-q0, 7, a) (exact), s = fma(e, fl(1/7), q0).  This equals the IEEE
// quotient for every finite a >= 0, subnormals included (checked against
// the IEEE division for all 2^31 non-negative finite floats); a = +inf or
// NaN gives NaN, which the caller's non-finite-scale test sends to
// rq_scales<..., true>, the IEEE division.  3 instructions instead of the
// ~10 of the scaled divide sequence.
#ifndef ZQ_DR_FAST_DIV
#define ZQ_DR_FAST_DIV 1
#endif
template <int QMAX, bool EXACT>
__device__ __forceinline__ BlockScale rq_block_scale(uint32_t amax_bits) {
    if constexpr (EXACT || !ZQ_DR_FAST_DIV) {
        return block_scale<QMAX>(amax_bits);
    } else {
        constexpr float r = 1.0f / (float)QMAX;
        const float a = bitsf(amax_bits);
        const float q0 = a * r;
        const float e = __builtin_fmaf(-q0, (float)QMAX, a);
        BlockScale b;
        b.s = __builtin_fmaf(e, r, q0);
        b.exact = (b.s != 0.0f) && (b.s < 0x1p-126f);
        b.inv = (b.s == 0.0f) ? 0.0f : __builtin_amdgcn_rcpf(b.s);
        return b;
    }
}

// Requant input: c = R (+ the requant EF e2), in place; elements past n are
// zeroed so that they do not enter the block max.
template <int B, bool RQ, bool EF, bool MASK, typename G = DrGeomOf<B, RQ, EF>, typename PV>
__device__ __forceinline__ void rq_compensate(const PV& p, size_t base, float (&c)[G::U][G::VEC],
                                              const float (&e2)[G::U][G::VEC]) {
    constexpr int V = G::VEC;
    if constexpr (EF) {
#pragma unroll
        for (int u = 0; u < G::U; ++u)
#pragma unroll
            for (int j = 0; j < V; ++j)
                c[u][j] = c[u][j] + e2[u][j];
    }
    if constexpr (MASK) {
        const int lane = lane_id();
#pragma unroll
        for (int u = 0; u < G::U; ++u) {
            const size_t i0 = base + (size_t)u * G::SUB + (size_t)lane * V;
#pragma unroll
            for (int j = 0; j < V; ++j)
                if (i0 + j >= p.n)
                    c[u][j] = 0.0f;
        }
    }
}

// Running absmax of one lane's requant inputs, as float bits.  gfx950's
// v_maximum3_f32 takes two |c| per instruction (abs is an operand modifier)
// and, as IEEE 754-2019 maximum, returns NaN when any input is NaN, so a NaN
// sum still gives a non-finite block scale, as the integer maximum over the
// magnitude bits does.  On non-negative floats both orders agree.
#ifndef ZQ_DR_FMAXIMUM
#define ZQ_DR_FMAXIMUM 1
#endif
template <int V>
__device__ __forceinline__ uint32_t lane_absmax(const float (&c)[V], uint32_t m) {
    if constexpr (ZQ_DR_FMAXIMUM) {
        float f = bitsf(m);
#pragma unroll
        for (int j = 0; j < V; ++j)
            f = __builtin_elementwise_maximum(f, __builtin_fabsf(c[j]));
        return fbits(f);
    } else {
#pragma unroll
        for (int j = 0; j < V; ++j)
            m = max(m, absbits(c[j]));
        return m;
    }
}

// The absmax of every block of the requant input and its scale.
template <int B, bool RQ, bool EF, bool EXACT, typename G = DrGeomOf<B, RQ, EF>>
__device__ __forceinline__ void rq_scales(const float (&c)[G::U][G::VEC],
                                          BlockScale (&bs)[G::SPB == 1 ? G::U : G::BPT]) {
    if constexpr (G::SPB == 1) {
#pragma unroll
        for (int u = 0; u < G::U; ++u)
            bs[u] = rq_block_scale<7, EXACT>(group_max<G::LPB>(lane_absmax(c[u], 0u)));
    } else {
#pragma unroll
        for (int b = 0; b < G::BPT; ++b) {
            uint32_t m = 0;
#pragma unroll
            for (int u = b * G::SPB; u < (b + 1) * G::SPB; ++u)
                m = lane_absmax(c[u], m);
            bs[b] = rq_block_scale<7, EXACT>(group_max<kWave>(m));
        }
    }
}

template <int B, int PMAX, bool OUT, bool RQ, bool EF, bool MASK, typename PV>
__device__ __forceinline__ void dr_tile(const PV& p, size_t tile) {
    constexpr bool RQEF = RQ && EF;  // requant with its EF buffer (p.rq_ef)
    using G = DrGeomOf<B, RQ, EF>;
    constexpr int V = G::VEC;
    constexpr bool BUF = RQ && !EF && !MASK;  // buffer addressing (see buf_load)
    const int lane = lane_id();
    const size_t base = (BUF ? uniform64(tile) : tile) * (size_t)G::TILE;
    const size_t n = p.n;

    uint32_t cw[PMAX][G::U];  // code words (VEC nibbles each)
    float sc[PMAX][G::U];
    float e2[G::U][V];

    // Issue every load of the tile first (the ragged tail instead loads and
    // adds one peer at a time, below).
    if constexpr (!MASK)
        dr_load<B, PMAX, RQ, EF, MASK>(p, base, cw, sc);
    if constexpr (RQEF) {
#pragma unroll
        for (int u = 0; u < G::U; ++u) {
            const size_t i0 = base + (size_t)u * G::SUB + (size_t)lane * V;
            if constexpr (!MASK) {
#pragma unroll
                for (int h = 0; h < V / 4; ++h) {
                    const f4 a = ld_stream((const f4*)(p.rq_ef + i0 + 4 * h));
                    e2[u][4 * h] = a.x; e2[u][4 * h + 1] = a.y;
                    e2[u][4 * h + 2] = a.z; e2[u][4 * h + 3] = a.w;
                }
            } else {
#pragma unroll
                for (int j = 0; j < V; ++j)
                    e2[u][j] = i0 + j < n ? p.rq_ef[i0 + j] : 0.0f;
            }
        }
    }

    // Dequantize and reduce, then R = alpha S.  The requant-only flavours
    // decode full tiles through k / 16 (dr_sum_off); a tile whose sums come
    // out non-finite is redone from the integer decode inside the requant's
    // rare branch below.  Every other flavour, and the ragged tail, takes the
    // integer decode.
    constexpr bool OFFDEC = ZQ_DR_DECODE_OFF && RQ && !OUT && !MASK;
    float R[G::U][V];
    if constexpr (MASK)
        dr_sum_masked<B, G>(p, base, R);
    else if constexpr (OFFDEC)
        dr_sum_off<PMAX, G::U, V>(p, cw, sc, R);
    else
        dr_sum_int<PMAX, G::U, V>(p, cw, sc, R);
    dr_alpha<G::U, V>(p, R);

    if constexpr (OUT) {
#pragma unroll
        for (int u = 0; u < G::U; ++u) {
            const size_t i0 = base + (size_t)u * G::SUB + (size_t)lane * V;
            if constexpr (!MASK) {
#pragma unroll
                for (int h = 0; h < V / 4; ++h) {
                    const f4 a = {R[u][4 * h], R[u][4 * h + 1], R[u][4 * h + 2], R[u][4 * h + 3]};
                    if constexpr (BUF)
                        buf_store<f4, kBufStoreNT>(a, p.out + base, G::TILE * 4,
                                                   4u * (uint32_t)(u * G::SUB + lane * V + 4 * h));
                    else
                        st_stream(a, (f4*)(p.out + i0 + 4 * h));
                }
            } else {
#pragma unroll
                for (int j = 0; j < V; ++j)
                    if (i0 + j < n)
                        p.out[i0 + j] = R[u][j];
            }
        }
    }

    if constexpr (RQ) {
        // Compensated requant input, in place (R is not needed any more).
        float (&c)[G::U][V] = R;
        BlockScale bs[G::SPB == 1 ? G::U : G::BPT];
        rq_compensate<B, RQ, EF, MASK>(p, base, c, e2);
        rq_scales<B, RQ, EF, false>(c, bs);
        // Fast codes: rne(c * rcp(s)) by the 1.5 * 2^23 addition.  A tile
        // falls back to the IEEE quotient when an element is in the tie band
        // or a block scale is subnormal, infinite or NaN (uniform branch).
        float kf[G::U][V];
        bool redo = false;
#pragma unroll
        for (int u = 0; u < G::U; ++u) {
            const BlockScale& b = bs[G::SPB == 1 ? u : u / G::SPB];
            redo |= b.exact | !(b.s <= 0x1.fffffep127f);
#pragma unroll
            for (int j = 0; j < V; ++j)
                kf[u][j] = code_fast_rne<7>(c[u][j], b, redo);
        }
        uint32_t packed[G::U];
        if (__builtin_amdgcn_ballot_w64(redo) == 0) {
            // Every |code| <= 7 here: pack the float codes, and use them as
            // exact integers in the error feedback.
#pragma unroll
            for (int u = 0; u < G::U; ++u) {
                packed[u] = pack_nibbles_f<V>(kf[u]);
                if constexpr (RQEF) {
                    const BlockScale& b = bs[G::SPB == 1 ? u : u / G::SPB];
#pragma unroll
                    for (int j = 0; j < V; ++j)
                        e2[u][j] = ef_update_f(c[u][j], kf[u][j], b.s, e2[u][j], p.rq_beta_e,
                                               p.rq_beta_r);
                }
            }
        } else {
            if constexpr (OFFDEC) {
                // Sums that are not all finite show up as a non-finite block
                // scale: redo such a tile from the integer decode.
                bool bad = false;
#pragma unroll
                for (int b = 0; b < (G::SPB == 1 ? G::U : G::BPT); ++b)
                    bad |= !(bs[b].s <= 0x1.fffffep127f);
                if (__builtin_amdgcn_ballot_w64(bad) != 0) {
                    dr_sum_int_reload<B, G>(p, base, R);
                    dr_alpha<G::U, V>(p, R);
                    rq_compensate<B, RQ, EF, MASK>(p, base, c, e2);
                    rq_scales<B, RQ, EF, false>(c, bs);
#pragma unroll
                    for (int u = 0; u < G::U; ++u)
#pragma unroll
                        for (int j = 0; j < V; ++j)
                            kf[u][j] = code_fast_rne<7>(c[u][j], bs[G::SPB == 1 ? u : u / G::SPB],
                                                        bad);
                }
            }
            if constexpr (ZQ_DR_FAST_DIV) {
                // A non-finite absmax (outside the finite-input contract)
                // takes the IEEE division, as the quantizer defines.
                bool nonfinite = false;
#pragma unroll
                for (int b = 0; b < (G::SPB == 1 ? G::U : G::BPT); ++b)
                    nonfinite |= !(bs[b].s <= 0x1.fffffep127f);
                if (__builtin_amdgcn_ballot_w64(nonfinite) != 0)
                    rq_scales<B, RQ, EF, true>(c, bs);
            }
#pragma unroll
            for (int u = 0; u < G::U; ++u) {
                const BlockScale& b = bs[G::SPB == 1 ? u : u / G::SPB];
                packed[u] = 0;
#pragma unroll
                for (int j = 0; j < V; ++j) {
                    const int k = code_clamp<7>(code_fix<7>(c[u][j], b, kf[u][j]));
                    packed[u] |= ((uint32_t)k & 0xFu) << (4 * j);
                    if constexpr (RQEF)
                        e2[u][j] = ef_update(c[u][j], k, b.s, e2[u][j], p.rq_beta_e, p.rq_beta_r);
                }
            }
        }
        if constexpr (G::SPB == 1) {
            if (lane % G::LPB == 0) {
#pragma unroll
                for (int u = 0; u < G::U; ++u) {
                    const size_t i0 = base + (size_t)u * G::SUB + (size_t)lane * V;
                    if (!MASK || i0 < n)
                        p.rq_scales[i0 / B] = bs[u].s;
                }
            }
        } else {
            if (lane == 0) {
#pragma unroll
                for (int b = 0; b < G::BPT; ++b) {
                    const size_t i0 = base + (size_t)b * B;
                    if (!MASK || i0 < n)
                        p.rq_scales[i0 / B] = bs[b].s;
                }
            }
        }
#pragma unroll
        for (int u = 0; u < G::U; ++u) {
            const size_t i0 = base + (size_t)u * G::SUB + (size_t)lane * V;
            if constexpr (!MASK) {
                if constexpr (BUF)
                    buf_store<code_word_t<V>, kBufStoreNT>((code_word_t<V>)packed[u],
                                                           p.rq_codes + base / 2, G::TILE / 2,
                                                           (uint32_t)(u * G::SUB + lane * V) / 2);
                else
                    st_stream((code_word_t<V>)packed[u], (code_word_t<V>*)(p.rq_codes + i0 / 2));
                if constexpr (RQEF) {
#pragma unroll
                    for (int h = 0; h < V / 4; ++h) {
                        const f4 a = {e2[u][4 * h], e2[u][4 * h + 1], e2[u][4 * h + 2],
                                      e2[u][4 * h + 3]};
                        st_stream(a, (f4*)(p.rq_ef + i0 + 4 * h));
                    }
                }
            } else {
#pragma unroll
                for (int b = 0; b < V / 2; ++b)
                    if (i0 + 2 * b < n)
                        p.rq_codes[i0 / 2 + b] = (uint8_t)(packed[u] >> (8 * b));
                if constexpr (RQEF) {
#pragma unroll
                    for (int j = 0; j < V; ++j)
                        if (i0 + j < n)
                            p.rq_ef[i0 + j] = e2[u][j];
                }
            }
        }
    }
}

// PMAX: the kernel serves every P <= PMAX; only PMAX pointer pairs stay
// live, so the common P = 4 / 8 cases keep their pointers in SGPRs.  The
// loop runs the full tiles without bounds checks; the ragged last tile (when
// n is not a multiple of the tile) goes to the one wave whose loop stops
// exactly at it, in the same launch.
template <int B, int PMAX, bool OUT, bool RQ, bool EF>
__global__ __launch_bounds__(kBlockThreads) void dr_kernel(DrParams p) {
    using G = DrGeomOf<B, RQ, EF>;
    const size_t nfull = p.n / G::TILE;
    // Plain dispatch order: the XCD-contiguous order of the streaming
    // kernels measured slower here (P peer streams per XCD run).
    size_t t = wave_id();
    for (; t < nfull; t += wave_count())
        dr_tile<B, PMAX, OUT, RQ, EF, false>(p, t);
    if (t == nfull && p.n % G::TILE)
        dr_tile<B, PMAX, OUT, RQ, EF, true>(p, t);
}

template <int B, int PMAX, bool OUT, bool RQ, bool EF>
hipError_t launch_b(const DrParams& p, hipStream_t stream) {
    using G = DrGeomOf<B, RQ, EF>;
    const size_t ntiles = (p.n + G::TILE - 1) / G::TILE;
    DrParams arg = p;
    void* args[] = {(void*)&arg};
    // Requant without EF keeps a persistent grid; with EF (two more fp32
    // streams) one tile per wave keeps more bytes in flight and is faster.
    const Geometry geom = (RQ && !EF) ? kGeomReduceRequant : kGeomReduce;
    return hipLaunchKernel((const void*)&dr_kernel<B, PMAX, OUT, RQ, EF>,
                           grid_for_tiles(ntiles, geom), dim3(geom.threads), args, 0, stream);
}

template <int B, int PMAX>
hipError_t launch_flags(const DrParams& p, hipStream_t st) {
    const bool out = p.out != nullptr, rq = p.rq_codes != nullptr, ef = p.rq_ef != nullptr;
    if (out && !rq)
        return launch_b<B, PMAX, true, false, false>(p, st);
    if (!out && rq)
        return ef ? launch_b<B, PMAX, false, true, true>(p, st)
                  : launch_b<B, PMAX, false, true, false>(p, st);
    if (out && rq)
        return ef ? launch_b<B, PMAX, true, true, true>(p, st)
                  : launch_b<B, PMAX, true, true, false>(p, st);
    return hipErrorInvalidValue;
}

template <int B>
hipError_t launch_peers(const DrParams& p, hipStream_t st) {
    if (p.P <= 2)
        return launch_flags<B, 2>(p, st);
    if (p.P <= 4)
        return launch_flags<B, 4>(p, st);
    if (p.P <= 8)
        return launch_flags<B, 8>(p, st);
    return launch_flags<B, 16>(p, st);
}

// ---------------------------------------------------------------------------
// Batched segments: the per-parameter receive side ("Merge LoCo with Zero++",
// review thread: the LoCo path reduces parameter by parameter, each with its
// own requant error-feedback buffer).  A launch takes up to kDrSegs segments
// (the table rides in the kernel arguments) and runs all of their tiles:
// first the full ones, a wave finding its segment from the cumulative
// full-tile counts (SegmentFinder), then the ragged last tiles, the k-th of
// which belongs to segment tail_seg[k].
#ifndef ZQ_DR_SEGS
#define ZQ_DR_SEGS 48
#endif
constexpr int kDrSegs = ZQ_DR_SEGS;

struct DrBatch {
    DrSegment seg[kDrSegs];
    uint32_t tile_end[kDrSegs];  // cumulative full tiles through segment s
    uint8_t tail_seg[kDrSegs];   // segment of the k-th ragged last tile
    uint32_t nseg;
    uint32_t full;   // full tiles of all segments
    uint32_t total;  // full + ragged tiles
    uint32_t P;
    float alpha, rq_beta_e, rq_beta_r;
};
static_assert(kDrSegs <= 256, "tail_seg holds 8-bit segment indices");

// A segment seen through the reduce tile's parameter interface.
struct DrSegView {
    const uint8_t* codes;
    const float* scales;
    uint64_t cstride, sstride;
    uint32_t P;
    size_t n;
    float alpha;
    float* out;
    uint8_t* rq_codes;
    float* rq_scales;
    float* rq_ef;
    float rq_beta_e, rq_beta_r;

    __device__ const uint8_t* codes_of(uint32_t q) const { return codes + q * cstride; }
    __device__ const float* scales_of(uint32_t q) const { return scales + q * sstride; }
};

template <int B, int PMAX, bool OUT, bool RQ, bool EF>
__global__ __launch_bounds__(kBlockThreads) void dr_batched_kernel(DrBatch b) {
    using G = DrGeomOf<B, RQ, EF>;
    const SegmentFinder<kDrSegs> find(b.tile_end, b.nseg);
    size_t ts = wave_id();
    for (; ts < b.full; ts += wave_count()) {
        const uint32_t t = (uint32_t)ts;
        const uint32_t s = find(t);
        const DrSegment& g = b.seg[s];
        const DrSegView v = {g.codes,    g.scales,    g.codes_stride, g.scales_stride, b.P,
                             g.n,        b.alpha,     g.out,          g.rq_codes,      g.rq_scales,
                             g.rq_ef,    b.rq_beta_e, b.rq_beta_r};
        dr_tile<B, PMAX, OUT, RQ, EF, false>(v, t - (s ? b.tile_end[s - 1] : 0u));
    }
    for (; ts < b.total; ts += wave_count()) {
        const DrSegment& g = b.seg[b.tail_seg[ts - b.full]];
        const DrSegView v = {g.codes,    g.scales,    g.codes_stride, g.scales_stride, b.P,
                             g.n,        b.alpha,     g.out,          g.rq_codes,      g.rq_scales,
                             g.rq_ef,    b.rq_beta_e, b.rq_beta_r};
        dr_tile<B, PMAX, OUT, RQ, EF, true>(v, g.n / G::TILE);
    }
}

template <int B, int PMAX, bool OUT, bool RQ, bool EF>
hipError_t launch_batched_b(const DrSegment* segs, uint32_t n_seg, const DrBatchArgs& a,
                            hipStream_t stream) {
    using G = DrGeomOf<B, RQ, EF>;
    static_assert(G::TILE >= 512, "2^40-element segments need tiles of >= 512");
    // One tile per wave for every flavour: with segments the persistent grid
    // of the single requant call measured 1.5-2.5 % slower (7.5B model, 327
    // tensors, builds A/B in one process with the measuring order rotated).
    const Geometry geom = kGeomReduce;
    uint32_t i = 0;
    while (i < n_seg) {
        DrBatch bt = {};
        bt.P = a.P;
        bt.alpha = a.alpha;
        bt.rq_beta_e = a.rq_beta_e;
        bt.rq_beta_r = a.rq_beta_r;
        uint64_t full = 0, tails = 0;
        // A launch takes segments while its tile count (32-bit in the
        // kernel's table) stays below 2^32.
        while (i < n_seg && bt.nseg < (uint32_t)kDrSegs) {
            const DrSegment& g = segs[i];
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
            hipLaunchKernel((const void*)&dr_batched_kernel<B, PMAX, OUT, RQ, EF>,
                            grid_for_tiles(tiles, geom), dim3(geom.threads), args, 0, stream);
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

template <int B, int PMAX>
hipError_t launch_batched_flags(const DrSegment* segs, uint32_t n_seg, const DrBatchArgs& a,
                                hipStream_t st) {
    if (a.out && !a.rq)
        return launch_batched_b<B, PMAX, true, false, false>(segs, n_seg, a, st);
    if (!a.out && a.rq)
        return a.rq_ef ? launch_batched_b<B, PMAX, false, true, true>(segs, n_seg, a, st)
                       : launch_batched_b<B, PMAX, false, true, false>(segs, n_seg, a, st);
    if (a.out && a.rq)
        return a.rq_ef ? launch_batched_b<B, PMAX, true, true, true>(segs, n_seg, a, st)
                       : launch_batched_b<B, PMAX, true, true, false>(segs, n_seg, a, st);
    return hipErrorInvalidValue;
}

template <int B>
hipError_t launch_batched_peers(const DrSegment* segs, uint32_t n_seg, const DrBatchArgs& a,
                                hipStream_t st) {
    if (a.P <= 2)
        return launch_batched_flags<B, 2>(segs, n_seg, a, st);
    if (a.P <= 4)
        return launch_batched_flags<B, 4>(segs, n_seg, a, st);
    if (a.P <= 8)
        return launch_batched_flags<B, 8>(segs, n_seg, a, st);
    return launch_batched_flags<B, 16>(segs, n_seg, a, st);
}

}  // namespace

// One launcher per block size, each compiled in its own translation unit
// (zq_dr_b*.hip for single calls, zq_drb_b*.hip for batched ones) so that
// the instantiations build in parallel.
#define ZQ_DR_LAUNCHER(BLK) \
    hipError_t launch_dr_b##BLK(const DrParams& p, hipStream_t st) { return launch_peers<BLK>(p, st); }
#define ZQ_DRB_LAUNCHER(BLK)                                                                  \
    hipError_t launch_drb_b##BLK(const DrSegment* segs, uint32_t n_seg, const DrBatchArgs& a, \
                                 hipStream_t st) {                                             \
        return launch_batched_peers<BLK>(segs, n_seg, a, st);                                  \
    }

}  // namespace zq
