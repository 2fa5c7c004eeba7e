// abi_driver.cpp -- the host side of libzq's C ABI (argument validation,
// range sorting, segment tables) under AddressSanitizer and
// UndefinedBehaviorSanitizer, without a GPU: the kernel launchers are
// replaced by stubs that check what the ABI layer hands them and launch
// nothing.  Every device pointer here is a fake address that is never
// dereferenced.  Test infrastructure only (built and run by
// tests/test_sanitizers.py).
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "../../include/zq.h"
#include "../../weight_communication_zero_amd/csrc/zq_launch.h"

static int failures = 0;
static int launches = 0;
#define CHECK(c)                                                             \
    do {                                                                     \
        if (!(c)) {                                                          \
            std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            failures++;                                                      \
        }                                                                    \
    } while (0)

namespace zq {
hipError_t launch_quantize_ef_int4(const void* g, int, float*, size_t n, uint32_t, float, float,
                                   uint8_t* codes, float* scales, hipStream_t) {
    CHECK(g && codes && scales && n > 0);
    launches++;
    return hipSuccess;
}
hipError_t launch_quantize_ef_int4_permuted(const void* g, int, float*, size_t n, uint32_t block,
                                            float, float, uint8_t*, float*, const PartPerm& perm,
                                            hipStream_t) {
    CHECK(g && perm.n_part >= 1 && perm.n_part <= kMaxParts);
    CHECK(perm.part_len * perm.n_part == n && perm.part_len % block == 0);
    launches++;
    return hipSuccess;
}
hipError_t launch_quantize_ef_int4_batched(const EfqSegment* segs, uint32_t n_seg, int, bool,
                                           uint32_t, float, float, hipStream_t) {
    uint64_t sum = 0;
    for (uint32_t i = 0; i < n_seg; ++i)
        sum += segs[i].n;  // read every entry the ABI layer built
    CHECK(n_seg > 0 && sum > 0);
    launches++;
    return hipSuccess;
}
hipError_t launch_dequant_reduce(const DrParams& p, uint32_t, hipStream_t) {
    CHECK(p.P >= 1 && p.P <= kMaxPeers && p.n > 0);
    for (uint32_t q = 0; q < p.P; ++q)
        CHECK(p.codes[q] && p.scales[q]);
    launches++;
    return hipSuccess;
}
hipError_t launch_dequant_reduce_batched(const DrSegment* segs, uint32_t n_seg,
                                         const DrBatchArgs& a, uint32_t, hipStream_t) {
    CHECK(n_seg > 0 && a.P >= 1 && a.P <= kMaxPeers && (a.out || a.rq));
    for (uint32_t i = 0; i < n_seg; ++i)
        CHECK(segs[i].codes && segs[i].scales && segs[i].n > 0);
    launches++;
    return hipSuccess;
}
hipError_t launch_quant_int8(const void*, int, size_t, uint32_t, int8_t*, float*, hipStream_t) {
    launches++;
    return hipSuccess;
}
hipError_t launch_dequant_int8(const int8_t*, const float*, size_t, uint32_t, void*, int,
                               hipStream_t) {
    launches++;
    return hipSuccess;
}
hipError_t launch_sr_accumulate(uint16_t*, uint16_t*, size_t, uint64_t, uint64_t, bool,
                                hipStream_t) {
    launches++;
    return hipSuccess;
}
hipError_t launch_sr_accumulate_batched(const SrSegment* segs, uint32_t n_seg, bool, hipStream_t) {
    uint64_t sum = 0;
    for (uint32_t i = 0; i < n_seg; ++i)
        sum += segs[i].n + segs[i].len;
    CHECK(n_seg > 0);
    (void)sum;
    launches++;
    return hipSuccess;
}
}  // namespace zq

static char* fake(uint64_t off) { return reinterpret_cast<char*>(0x100000000ull + off); }

int main() {
    // single calls: invalid, then valid
    CHECK(zq_quantize_ef_int4(fake(0), (zq_dtype)5, nullptr, 64, 128, 1, 1, (uint8_t*)fake(1 << 20),
                              (float*)fake(2 << 20), nullptr) == ZQ_ERR_DTYPE);
    CHECK(zq_quantize_ef_int4(fake(0), ZQ_FP32, nullptr, 64, 100, 1, 1, (uint8_t*)fake(1 << 20),
                              (float*)fake(2 << 20), nullptr) == ZQ_ERR_BLOCK);
    CHECK(zq_quantize_ef_int4(fake(0), ZQ_FP32, nullptr, 1000, 128, 1, 1, (uint8_t*)fake(256),
                              (float*)fake(2 << 20), nullptr) == ZQ_ERR_ALIAS);
    CHECK(zq_quantize_ef_int4(fake(0), ZQ_BF16, (float*)fake(4 << 20), 1000, 128, 1, 1,
                              (uint8_t*)fake(1 << 20), (float*)fake(2 << 20), nullptr) == ZQ_OK);
    std::vector<uint32_t> slots(256);
    CHECK(zq_zeropp_slots(16, 16, slots.data()) == 256);
    CHECK(zq_zeropp_slots(16, 17, slots.data()) == 0);
    CHECK(zq_quantize_ef_int4_permuted(fake(0), ZQ_FP32, nullptr, 256 * 1024, 128, 1, 1,
                                       (uint8_t*)fake(8 << 20), (float*)fake(16 << 20), 256,
                                       slots.data(), nullptr) == ZQ_OK);
    slots[7] = slots[8];
    CHECK(zq_quantize_ef_int4_permuted(fake(0), ZQ_FP32, nullptr, 256 * 1024, 128, 1, 1,
                                       (uint8_t*)fake(8 << 20), (float*)fake(16 << 20), 256,
                                       slots.data(), nullptr) == ZQ_ERR_SIZE);
    const uint8_t* cp[16];
    const float* sp[16];
    for (int q = 0; q < 16; ++q) {
        cp[q] = (const uint8_t*)fake((uint64_t)q << 24);
        sp[q] = (const float*)fake(((uint64_t)q << 24) + (1 << 23));
    }
    CHECK(zq_dequant_reduce(17, cp, sp, 4096, 128, 1, (float*)fake(1ull << 32), nullptr, nullptr,
                            nullptr, 0, 1, nullptr) == ZQ_ERR_PEERS);
    CHECK(zq_dequant_reduce(16, cp, sp, 4096, 128, 1, (float*)fake(1ull << 32), nullptr, nullptr,
                            nullptr, 0, 1, nullptr) == ZQ_OK);
    CHECK(zq_dequant_reduce(16, cp, sp, 4096, 128, 1, (float*)fake(64), nullptr, nullptr, nullptr,
                            0, 1, nullptr) == ZQ_ERR_ALIAS);
    CHECK(zq_quant_int8(fake(0), ZQ_BF16, 4097, 2048, (int8_t*)fake(1 << 20), (float*)fake(2 << 20),
                        nullptr) == ZQ_OK);
    CHECK(zq_dequant_int8((int8_t*)fake(0), (float*)fake(1 << 20), 4097, 2048, fake(2 << 20),
                          ZQ_BF16, nullptr) == ZQ_OK);
    CHECK(zq_sr_accumulate((uint16_t*)fake(0), (uint16_t*)fake(1 << 20), 1000, 1, ~0ull - 10, 0,
                           nullptr) == ZQ_ERR_SIZE);
    CHECK(zq_sr_accumulate((uint16_t*)fake(0), (uint16_t*)fake(1 << 20), 1000, 1, 5, 1, nullptr) ==
          ZQ_OK);

    // batched calls at their largest table size, then with an overlap
    const uint32_t S = 65536;
    std::vector<zq_efq_segment> es(S);
    for (uint32_t i = 0; i < S; ++i) {
        const uint64_t b = (uint64_t)i << 16;
        es[i] = {fake(b), (float*)fake(b + 0x4000), (uint8_t*)fake(b + 0x8000),
                 (float*)fake(b + 0xC000), 1024};
    }
    CHECK(zq_quantize_ef_int4_batched(es.data(), S, ZQ_FP32, 128, 1, 1, nullptr) == ZQ_OK);
    es[S - 1].codes = (uint8_t*)fake(((uint64_t)(S - 2) << 16) + 0x8000);
    CHECK(zq_quantize_ef_int4_batched(es.data(), S, ZQ_FP32, 128, 1, 1, nullptr) == ZQ_ERR_ALIAS);
    CHECK(zq_quantize_ef_int4_batched(es.data(), S + 1, ZQ_FP32, 128, 1, 1, nullptr) ==
          ZQ_ERR_SIZE);
    std::vector<zq_sr_segment> ss(S);
    for (uint32_t i = 0; i < S; ++i) {
        const uint64_t b = (uint64_t)i << 16;
        ss[i] = {(uint16_t*)fake(b), (uint16_t*)fake(b + 0x4000), 100, 8, 200, i, 8ull * i};
    }
    CHECK(zq_sr_accumulate_batched(ss.data(), S, 1, nullptr) == ZQ_OK);
    ss[3].src_offset = 4;
    CHECK(zq_sr_accumulate_batched(ss.data(), S, 1, nullptr) == ZQ_ERR_ALIGN);
    ss[3].src_offset = 8;
    ss[5].dst = ss[4].dst + 48;
    CHECK(zq_sr_accumulate_batched(ss.data(), S, 0, nullptr) == ZQ_ERR_ALIAS);

    std::vector<zq_dr_segment> ds(S);
    for (uint32_t i = 0; i < S; ++i) {
        const uint64_t b = (uint64_t)i << 16;
        ds[i] = {(const uint8_t*)fake(b), (const float*)fake(b + 0x2000), 256, 4, 512,
                 nullptr, (uint8_t*)fake(b + 0x4000), (float*)fake(b + 0x6000),
                 (float*)fake(b + 0x8000)};
    }
    CHECK(zq_dequant_reduce_batched(ds.data(), S, 8, 128, 1, 0.9f, 1, nullptr) == ZQ_OK);
    ds[9].rq_ef = nullptr;
    CHECK(zq_dequant_reduce_batched(ds.data(), S, 8, 128, 1, 0.9f, 1, nullptr) == ZQ_ERR_NULL);
    ds[9].rq_ef = (float*)fake(((uint64_t)9 << 16) + 0x8000);
    ds[11].rq_codes = (uint8_t*)fake(((uint64_t)12 << 16) + 0x100);  // inside 12's codes
    CHECK(zq_dequant_reduce_batched(ds.data(), S, 8, 128, 1, 0.9f, 1, nullptr) == ZQ_ERR_ALIAS);

    CHECK(launches == 9);
    for (int s = 0; s < 12; ++s)
        CHECK(zq_status_str((zq_status)s) != nullptr);
#ifdef ZQ_SANITIZER_CANARY
    // planted out-of-bounds read: proves the sanitizer build is armed
    std::vector<int> v(4);
    volatile int sink = v.data()[4];
    (void)sink;
#endif
    if (failures) {
        std::fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    std::printf("abi driver: %d launches validated, all checks passed\n", launches);
    return 0;
}
