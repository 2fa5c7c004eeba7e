// zq_abi.hip -- the extern "C" entry points of libzq: host-side argument
// validation, then one kernel launch on the caller's stream.  Every check
// runs before anything is enqueued, so an error status means no device work
// was issued.  No state, no allocation.
#include <stdint.h>

#include <algorithm>
#include <cstring>
#include <vector>

#include "../../include/zq.h"
#include "zq_launch.h"

namespace {

constexpr size_t kMaxElems = (size_t)1 << 60;
constexpr size_t kMaxSegElems = (size_t)1 << 40;  // per segment of a batched call

bool valid_block(uint32_t b) { return b >= 32 && b <= 4096 && (b & (b - 1)) == 0; }

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Byte ranges [a, a+na) and [b, b+nb) intersect (NULL or empty never does).
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0)
        return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + nb && b0 < a0 + na;
}

size_t nblocks(size_t n, uint32_t block) { return (n + block - 1) / block; }

// Element types of the data streams; the values double as zq::ElemType.
bool known_dtype(int d) { return d == ZQ_FP32 || d == ZQ_BF16 || d == ZQ_FP16; }
size_t dtype_bytes(int d) { return d == ZQ_FP32 ? 4 : 2; }
static_assert(ZQ_FP32 == zq::kF32 && ZQ_BF16 == zq::kBF16 && ZQ_FP16 == zq::kF16,
              "zq_dtype values are the kernels' element types");

zq_status launched(hipError_t e) { return e == hipSuccess ? ZQ_OK : ZQ_ERR_LAUNCH; }

// The integer a C caller passed for an enum parameter.  Values outside the
// enumerators are legal in C but not representable in the C++ enum type, so
// they are read as bytes (memcpy), never as an enum value.
template <typename E>
int raw_enum(const E& e) {
    static_assert(sizeof(E) == sizeof(int), "enums of the ABI are int-sized");
    int v;
    std::memcpy(&v, &e, sizeof v);
    return v;
}

}  // namespace

extern "C" {

zq_status zq_quantize_ef_int4(const void* g, zq_dtype g_dtype_arg, float* ef, size_t n, uint32_t block,
                              float beta_e, float beta_r, uint8_t* codes, float* scales,
                              void* stream) {
    const int g_dtype = raw_enum(g_dtype_arg);
    if (!known_dtype(g_dtype))
        return ZQ_ERR_DTYPE;
    if (!valid_block(block))
        return ZQ_ERR_BLOCK;
    if (n > kMaxElems)
        return ZQ_ERR_SIZE;
    if (n == 0)
        return ZQ_OK;
    if (!g || !codes || !scales)
        return ZQ_ERR_NULL;
    if (!aligned(g, 16) || !aligned(ef, 16) || !aligned(codes, 16) || !aligned(scales, 4))
        return ZQ_ERR_ALIGN;
    const size_t gb = n * dtype_bytes(g_dtype), eb = ef ? n * 4 : 0;
    const size_t cb = zq_int4_code_bytes(n), sb = nblocks(n, block) * 4;
    if (overlap(codes, cb, g, gb) || overlap(codes, cb, ef, eb) || overlap(codes, cb, scales, sb) ||
        overlap(scales, sb, g, gb) || overlap(scales, sb, ef, eb) || overlap(ef, eb, g, gb))
        return ZQ_ERR_ALIAS;
    return launched(zq::launch_quantize_ef_int4(g, g_dtype, ef, n, block, beta_e,
                                                beta_r, codes, scales, (hipStream_t)stream));
}

zq_status zq_quantize_ef_int4_permuted(const void* g, zq_dtype g_dtype_arg, float* ef, size_t n,
                                       uint32_t block, float beta_e, float beta_r, uint8_t* codes,
                                       float* scales, uint32_t n_part,
                                       const uint32_t* slot_of_part, void* stream) {
    const int g_dtype = raw_enum(g_dtype_arg);
    if (!known_dtype(g_dtype))
        return ZQ_ERR_DTYPE;
    if (!valid_block(block))
        return ZQ_ERR_BLOCK;
    if (n > kMaxElems || n_part < 1 || n_part > zq::kMaxParts)
        return ZQ_ERR_SIZE;
    if (n == 0)
        return ZQ_OK;
    if (!g || !codes || !scales || !slot_of_part)
        return ZQ_ERR_NULL;
    const size_t part_len = n / n_part;
    if (part_len * n_part != n || part_len % block || part_len < std::max<size_t>(1024, block))
        return ZQ_ERR_SIZE;
    zq::PartPerm perm = {};
    perm.part_len = part_len;
    perm.n_part = n_part;
    bool seen[zq::kMaxParts] = {};
    for (uint32_t p = 0; p < n_part; ++p) {
        const uint32_t s = slot_of_part[p];
        if (s >= n_part || seen[s])
            return ZQ_ERR_SIZE;
        seen[s] = true;
        perm.slot[p] = s;
    }
    if (!aligned(g, 16) || !aligned(ef, 16) || !aligned(codes, 16) || !aligned(scales, 4))
        return ZQ_ERR_ALIGN;
    const size_t gb = n * dtype_bytes(g_dtype), eb = ef ? n * 4 : 0;
    const size_t cb = zq_int4_code_bytes(n), sb = nblocks(n, block) * 4;
    if (overlap(codes, cb, g, gb) || overlap(codes, cb, ef, eb) || overlap(codes, cb, scales, sb) ||
        overlap(scales, sb, g, gb) || overlap(scales, sb, ef, eb) || overlap(ef, eb, g, gb))
        return ZQ_ERR_ALIAS;
    return launched(zq::launch_quantize_ef_int4_permuted(g, g_dtype, ef, n, block,
                                                         beta_e, beta_r, codes, scales, perm,
                                                         (hipStream_t)stream));
}

zq_status zq_quantize_ef_int4_batched(const zq_efq_segment* segs, uint32_t n_seg,
                                      zq_dtype g_dtype_arg, uint32_t block, float beta_e,
                                      float beta_r, void* stream) {
    const int g_dtype = raw_enum(g_dtype_arg);
    if (!known_dtype(g_dtype))
        return ZQ_ERR_DTYPE;
    if (!valid_block(block))
        return ZQ_ERR_BLOCK;
    if (n_seg == 0)
        return ZQ_OK;
    if (!segs)
        return ZQ_ERR_NULL;
    if (n_seg > 65536)
        return ZQ_ERR_SIZE;
    struct Range {
        uintptr_t lo, hi;
        bool written;
    };
    std::vector<Range> ranges;
    std::vector<zq::EfqSegment> dev;
    ranges.reserve(4 * (size_t)n_seg);
    dev.reserve(n_seg);
    int ef_state = -1;  // unknown / 0 none / 1 all
    const size_t esz = dtype_bytes(g_dtype);
    for (uint32_t i = 0; i < n_seg; ++i) {
        const zq_efq_segment& s = segs[i];
        if (s.n > kMaxSegElems)
            return ZQ_ERR_SIZE;
        if (s.n == 0)
            continue;
        if (!s.g || !s.codes || !s.scales)
            return ZQ_ERR_NULL;
        const int has_ef = s.ef ? 1 : 0;
        if (ef_state >= 0 && has_ef != ef_state)
            return ZQ_ERR_NULL;
        ef_state = has_ef;
        if (!aligned(s.g, 16) || !aligned(s.ef, 16) || !aligned(s.codes, 16) ||
            !aligned(s.scales, 4))
            return ZQ_ERR_ALIGN;
        ranges.push_back({(uintptr_t)s.g, (uintptr_t)s.g + esz * s.n, false});
        if (s.ef)
            ranges.push_back({(uintptr_t)s.ef, (uintptr_t)s.ef + 4 * s.n, true});
        ranges.push_back({(uintptr_t)s.codes, (uintptr_t)s.codes + zq_int4_code_bytes(s.n), true});
        ranges.push_back({(uintptr_t)s.scales, (uintptr_t)s.scales + 4 * nblocks(s.n, block), true});
        dev.push_back({s.g, s.ef, s.codes, s.scales, s.n});
    }
    if (dev.empty())
        return ZQ_OK;
    std::sort(ranges.begin(), ranges.end(),
              [](const Range& a, const Range& b) { return a.lo < b.lo; });
    uintptr_t max_end_any = 0, max_end_written = 0;
    for (const Range& r : ranges) {
        if (r.lo < (r.written ? max_end_any : max_end_written))
            return ZQ_ERR_ALIAS;
        max_end_any = std::max(max_end_any, r.hi);
        if (r.written)
            max_end_written = std::max(max_end_written, r.hi);
    }
    return launched(zq::launch_quantize_ef_int4_batched(dev.data(), (uint32_t)dev.size(),
                                                        g_dtype, ef_state == 1, block,
                                                        beta_e, beta_r, (hipStream_t)stream));
}

zq_status zq_dequant_reduce(uint32_t P, const uint8_t* const* codes, const float* const* scales,
                            size_t n_chunk, uint32_t block, float alpha, float* out,
                            uint8_t* rq_codes, float* rq_scales, float* rq_ef, float rq_beta_e,
                            float rq_beta_r, void* stream) {
    if (P < 1 || P > zq::kMaxPeers)
        return ZQ_ERR_PEERS;
    if (!valid_block(block))
        return ZQ_ERR_BLOCK;
    if (n_chunk > kMaxElems)
        return ZQ_ERR_SIZE;
    if (n_chunk == 0)
        return ZQ_OK;
    if (!codes || !scales)
        return ZQ_ERR_NULL;
    for (uint32_t p = 0; p < P; ++p)
        if (!codes[p] || !scales[p])
            return ZQ_ERR_NULL;
    if (!out && !rq_codes)
        return ZQ_ERR_NULL;
    if ((rq_codes == nullptr) != (rq_scales == nullptr) || (rq_ef && !rq_codes))
        return ZQ_ERR_NULL;
    for (uint32_t p = 0; p < P; ++p)
        if (!aligned(codes[p], 16) || !aligned(scales[p], 4))
            return ZQ_ERR_ALIGN;
    if (!aligned(out, 16) || !aligned(rq_codes, 16) || !aligned(rq_scales, 4) ||
        !aligned(rq_ef, 16))
        return ZQ_ERR_ALIGN;
    const size_t cb = zq_int4_code_bytes(n_chunk), sb = nblocks(n_chunk, block) * 4;
    const size_t ob = out ? n_chunk * 4 : 0, rcb = rq_codes ? cb : 0, rsb = rq_codes ? sb : 0;
    const size_t reb = rq_ef ? n_chunk * 4 : 0;
    const void* outs[4] = {out, rq_codes, rq_scales, rq_ef};
    const size_t outb[4] = {ob, rcb, rsb, reb};
    for (int i = 0; i < 4; ++i) {
        for (int j = i + 1; j < 4; ++j)
            if (overlap(outs[i], outb[i], outs[j], outb[j]))
                return ZQ_ERR_ALIAS;
        for (uint32_t p = 0; p < P; ++p)
            if (overlap(outs[i], outb[i], codes[p], cb) || overlap(outs[i], outb[i], scales[p], sb))
                return ZQ_ERR_ALIAS;
    }
    zq::DrParams prm = {};
    for (uint32_t p = 0; p < P; ++p) {
        prm.codes[p] = codes[p];
        prm.scales[p] = scales[p];
    }
    prm.P = P;
    prm.n = n_chunk;
    prm.alpha = alpha;
    prm.out = out;
    prm.rq_codes = rq_codes;
    prm.rq_scales = rq_scales;
    prm.rq_ef = rq_ef;
    prm.rq_beta_e = rq_beta_e;
    prm.rq_beta_r = rq_beta_r;
    return launched(zq::launch_dequant_reduce(prm, block, (hipStream_t)stream));
}

zq_status zq_dequant_reduce_batched(const zq_dr_segment* segs, uint32_t n_seg, uint32_t P,
                                    uint32_t block, float alpha, float rq_beta_e, float rq_beta_r,
                                    void* stream) {
    if (P < 1 || P > zq::kMaxPeers)
        return ZQ_ERR_PEERS;
    if (!valid_block(block))
        return ZQ_ERR_BLOCK;
    if (n_seg == 0)
        return ZQ_OK;
    if (!segs)
        return ZQ_ERR_NULL;
    if (n_seg > 65536)
        return ZQ_ERR_SIZE;
    struct Range {
        uintptr_t lo, hi;
        bool written;
    };
    std::vector<Range> ranges;
    std::vector<zq::DrSegment> dev;
    ranges.reserve(6 * (size_t)n_seg);
    dev.reserve(n_seg);
    int has_out = -1, has_rq = -1, has_ef = -1;  // unknown / 0 none / 1 all
    const auto same = [](int& state, bool v) {
        if (state >= 0 && state != (int)v)
            return false;
        state = v;
        return true;
    };
    constexpr uint64_t kMaxStride = (uint64_t)1 << 50;
    for (uint32_t i = 0; i < n_seg; ++i) {
        const zq_dr_segment& g = segs[i];
        if (g.n > kMaxSegElems)
            return ZQ_ERR_SIZE;
        if (g.n == 0)
            continue;
        if (!g.codes || !g.scales)
            return ZQ_ERR_NULL;
        if (!same(has_out, g.out != nullptr) || !same(has_rq, g.rq_codes != nullptr) ||
            !same(has_ef, g.rq_ef != nullptr) || (g.rq_codes == nullptr) != (g.rq_scales == nullptr) ||
            (g.rq_ef && !g.rq_codes) || (!g.out && !g.rq_codes))
            return ZQ_ERR_NULL;
        const size_t cb = zq_int4_code_bytes(g.n), nb = nblocks(g.n, block);
        if (P > 1 && (g.codes_stride < cb || g.scales_stride < nb || g.codes_stride > kMaxStride ||
                      g.scales_stride > kMaxStride))
            return ZQ_ERR_SIZE;
        if (!aligned(g.codes, 16) || !aligned(g.scales, 4) || (P > 1 && g.codes_stride % 16) ||
            !aligned(g.out, 16) || !aligned(g.rq_codes, 16) || !aligned(g.rq_scales, 4) ||
            !aligned(g.rq_ef, 16))
            return ZQ_ERR_ALIGN;
        const uint64_t cspan = (uint64_t)(P - 1) * (P > 1 ? g.codes_stride : 0) + cb;
        const uint64_t sspan = 4 * ((uint64_t)(P - 1) * (P > 1 ? g.scales_stride : 0) + nb);
        ranges.push_back({(uintptr_t)g.codes, (uintptr_t)g.codes + cspan, false});
        ranges.push_back({(uintptr_t)g.scales, (uintptr_t)g.scales + sspan, false});
        if (g.out)
            ranges.push_back({(uintptr_t)g.out, (uintptr_t)g.out + 4 * g.n, true});
        if (g.rq_codes) {
            ranges.push_back({(uintptr_t)g.rq_codes, (uintptr_t)g.rq_codes + cb, true});
            ranges.push_back({(uintptr_t)g.rq_scales, (uintptr_t)g.rq_scales + 4 * nb, true});
        }
        if (g.rq_ef)
            ranges.push_back({(uintptr_t)g.rq_ef, (uintptr_t)g.rq_ef + 4 * g.n, true});
        dev.push_back({g.codes, g.scales, P > 1 ? g.codes_stride : 0, P > 1 ? g.scales_stride : 0,
                       g.n, g.out, g.rq_codes, g.rq_scales, g.rq_ef});
    }
    if (dev.empty())
        return ZQ_OK;
    std::sort(ranges.begin(), ranges.end(),
              [](const Range& a, const Range& b) { return a.lo < b.lo; });
    uintptr_t max_end_any = 0, max_end_written = 0;
    for (const Range& r : ranges) {
        if (r.lo < (r.written ? max_end_any : max_end_written))
            return ZQ_ERR_ALIAS;
        max_end_any = std::max(max_end_any, r.hi);
        if (r.written)
            max_end_written = std::max(max_end_written, r.hi);
    }
    const zq::DrBatchArgs a = {P, alpha, rq_beta_e, rq_beta_r, has_out == 1, has_rq == 1,
                               has_ef == 1};
    return launched(zq::launch_dequant_reduce_batched(dev.data(), (uint32_t)dev.size(), a, block,
                                                      (hipStream_t)stream));
}

zq_status zq_quant_int8(const void* w, zq_dtype w_dtype_arg, size_t n, uint32_t block, int8_t* codes,
                        float* scales, void* stream) {
    const int w_dtype = raw_enum(w_dtype_arg);
    if (!known_dtype(w_dtype))
        return ZQ_ERR_DTYPE;
    if (!valid_block(block))
        return ZQ_ERR_BLOCK;
    if (n > kMaxElems)
        return ZQ_ERR_SIZE;
    if (n == 0)
        return ZQ_OK;
    if (!w || !codes || !scales)
        return ZQ_ERR_NULL;
    if (!aligned(w, 16) || !aligned(codes, 16) || !aligned(scales, 4))
        return ZQ_ERR_ALIGN;
    const size_t wb = n * dtype_bytes(w_dtype), sb = nblocks(n, block) * 4;
    if (overlap(codes, n, w, wb) || overlap(scales, sb, w, wb) || overlap(codes, n, scales, sb))
        return ZQ_ERR_ALIAS;
    return launched(
        zq::launch_quant_int8(w, w_dtype, n, block, codes, scales, (hipStream_t)stream));
}

zq_status zq_dequant_int8(const int8_t* codes, const float* scales, size_t n, uint32_t block,
                          void* out, zq_dtype out_dtype_arg, void* stream) {
    const int out_dtype = raw_enum(out_dtype_arg);
    if (!known_dtype(out_dtype))
        return ZQ_ERR_DTYPE;
    if (!valid_block(block))
        return ZQ_ERR_BLOCK;
    if (n > kMaxElems)
        return ZQ_ERR_SIZE;
    if (n == 0)
        return ZQ_OK;
    if (!codes || !scales || !out)
        return ZQ_ERR_NULL;
    if (!aligned(codes, 16) || !aligned(scales, 4) || !aligned(out, 16))
        return ZQ_ERR_ALIGN;
    const size_t ob = n * dtype_bytes(out_dtype), sb = nblocks(n, block) * 4;
    if (overlap(out, ob, codes, n) || overlap(out, ob, scales, sb))
        return ZQ_ERR_ALIAS;
    return launched(zq::launch_dequant_int8(codes, scales, n, block, out, out_dtype,
                                            (hipStream_t)stream));
}

zq_status zq_sr_accumulate(uint16_t* dst_bf16, uint16_t* src_bf16, size_t n, uint64_t seed,
                           uint64_t counter_base, int zero_src, void* stream) {
    if (n > kMaxElems || counter_base > UINT64_MAX - n)
        return ZQ_ERR_SIZE;
    if (n == 0)
        return ZQ_OK;
    if (!dst_bf16 || !src_bf16)
        return ZQ_ERR_NULL;
    if (!aligned(dst_bf16, 16) || !aligned(src_bf16, 16))
        return ZQ_ERR_ALIGN;
    if (overlap(dst_bf16, n * 2, src_bf16, n * 2))
        return ZQ_ERR_ALIAS;
    return launched(zq::launch_sr_accumulate(dst_bf16, src_bf16, n, seed, counter_base,
                                             zero_src != 0, (hipStream_t)stream));
}

zq_status zq_sr_accumulate_batched(const zq_sr_segment* segs, uint32_t n_seg, int zero_src,
                                   void* stream) {
    if (n_seg == 0)
        return ZQ_OK;
    if (!segs)
        return ZQ_ERR_NULL;
    if (n_seg > 65536)
        return ZQ_ERR_SIZE;
    // Written ranges (every dst; every src buffer when zero_src) may overlap
    // nothing else; read ranges (src slices) may overlap each other only.
    struct Range {
        uintptr_t lo, hi;
        bool written;
    };
    std::vector<Range> ranges;
    std::vector<zq::SrSegment> dev;
    ranges.reserve(2 * (size_t)n_seg);
    dev.reserve(n_seg);
    for (uint32_t i = 0; i < n_seg; ++i) {
        const zq_sr_segment& g = segs[i];
        if (g.n > kMaxSegElems || g.src_len > kMaxSegElems || g.src_offset > g.src_len ||
            g.n > g.src_len - g.src_offset || g.counter_base > UINT64_MAX - g.n)
            return ZQ_ERR_SIZE;
        const bool touches_src = g.n > 0 || (zero_src && g.src_len > 0);
        if ((g.n > 0 && !g.dst) || (touches_src && !g.src))
            return ZQ_ERR_NULL;
        if (!aligned(g.dst, 16) || !aligned(g.src, 16) || (g.src_offset & 7u))
            return ZQ_ERR_ALIGN;
        if (g.n > 0)
            ranges.push_back({(uintptr_t)g.dst, (uintptr_t)g.dst + 2 * g.n, true});
        if (zero_src && g.src_len > 0)
            ranges.push_back({(uintptr_t)g.src, (uintptr_t)g.src + 2 * g.src_len, true});
        else if (g.n > 0)
            ranges.push_back({(uintptr_t)(g.src + g.src_offset),
                              (uintptr_t)(g.src + g.src_offset) + 2 * g.n, false});
        dev.push_back({g.dst, g.src, g.n, g.src_offset, g.src_len, g.seed, g.counter_base});
    }
    std::sort(ranges.begin(), ranges.end(),
              [](const Range& a, const Range& b) { return a.lo < b.lo; });
    uintptr_t max_end_any = 0, max_end_written = 0;
    for (const Range& r : ranges) {
        if (r.lo < (r.written ? max_end_any : max_end_written))
            return ZQ_ERR_ALIAS;
        max_end_any = std::max(max_end_any, r.hi);
        if (r.written)
            max_end_written = std::max(max_end_written, r.hi);
    }
    return launched(zq::launch_sr_accumulate_batched(dev.data(), (uint32_t)dev.size(),
                                                     zero_src != 0, (hipStream_t)stream));
}

uint32_t zq_zeropp_slots(uint32_t intra, uint32_t inter, uint32_t* slot_of_part) {
    if (!slot_of_part || intra == 0 || inter == 0 || (uint64_t)intra * inter > zq::kMaxParts)
        return 0;
    // Local rank j receives slots j * inter .. j * inter + inter - 1 of every
    // GPU in its node, and sends entry i of what it reduced to node i.
    for (uint32_t j = 0; j < intra; ++j)
        for (uint32_t i = 0; i < inter; ++i)
            slot_of_part[i * intra + j] = j * inter + i;
    return intra * inter;
}

size_t zq_int4_code_bytes(size_t n) { return n / 2 + (n & 1); }

size_t zq_num_blocks(size_t n, uint32_t block) { return block ? nblocks(n, block) : 0; }

const char* zq_status_str(zq_status s) {
    switch (raw_enum(s)) {
        case ZQ_OK: return "ZQ_OK";
        case ZQ_ERR_NULL: return "ZQ_ERR_NULL: a required pointer is NULL";
        case ZQ_ERR_SIZE: return "ZQ_ERR_SIZE: sizes inconsistent or too large";
        case ZQ_ERR_BLOCK: return "ZQ_ERR_BLOCK: block must be a power of two in [32, 4096]";
        case ZQ_ERR_ALIGN: return "ZQ_ERR_ALIGN: misaligned pointer";
        case ZQ_ERR_ALIAS: return "ZQ_ERR_ALIAS: an output overlaps another buffer";
        case ZQ_ERR_PEERS: return "ZQ_ERR_PEERS: P must be in [1, 16]";
        case ZQ_ERR_DTYPE: return "ZQ_ERR_DTYPE: unknown dtype";
        case ZQ_ERR_LAUNCH: return "ZQ_ERR_LAUNCH: HIP kernel launch failed";
    }
    return "unknown zq_status";
}

uint32_t zq_abi_version(void) { return ZQ_ABI_VERSION; }

}  // extern "C"
