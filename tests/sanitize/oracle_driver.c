/*
 * oracle_driver.c -- runs every entry point of the CPU oracle
 * (oracle/zq_oracle.c) over edge-case shapes with exactly sized heap
 * buffers, for a build under AddressSanitizer and UndefinedBehaviorSanitizer:
 * any out-of-bounds access, use of uninitialised size arithmetic or
 * undefined conversion aborts the run.  It also checks that arguments the
 * oracle must refuse are refused without writing anything.  Test
 * infrastructure only (built and run by tests/test_sanitizers.py).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int orc_quant_block(const float *x, size_t m, int qmax, int32_t *k, float *s_out);
int32_t orc_int4_decode(const uint8_t *codes, size_t i);
int orc_quantize_ef_int4(const void *g, int g_is_bf16, float *ef, size_t n, uint32_t block,
                         float beta_e, float beta_r, uint8_t *codes, float *scales);
int orc_zeropp_slots(uint32_t intra, uint32_t inter, uint32_t *slot_of_part);
int orc_quantize_ef_int4_permuted(const void *g, int g_is_bf16, float *ef, size_t n,
                                  uint32_t block, float beta_e, float beta_r, uint32_t n_part,
                                  const uint32_t *slot_of_part, uint8_t *codes, float *scales);
int orc_dequant_reduce(uint32_t P, const uint8_t *const *codes, const float *const *scales,
                       size_t n_chunk, uint32_t block, float alpha, float *out,
                       uint8_t *rq_codes, float *rq_scales, float *rq_ef, float rq_beta_e,
                       float rq_beta_r, float *work);
int orc_quant_int8(const void *w, int w_is_bf16, size_t n, uint32_t block, int8_t *codes,
                   float *scales);
int orc_dequant_int8(const int8_t *codes, const float *scales, size_t n, uint32_t block,
                     void *out, int out_is_bf16);
uint16_t orc_bf16_rne(float f);
void orc_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]);
uint32_t orc_sr_r16(uint64_t seed, uint64_t q);
uint16_t orc_sr_round(float x, uint32_t r16);
int orc_sr_accumulate(uint16_t *dst, uint16_t *src, size_t n, uint64_t seed,
                      uint64_t counter_base, int zero_src);
int orc_sr_accumulate_segments(uint32_t n_seg, uint16_t *const *dst, uint16_t *const *src,
                               const uint64_t *n, const uint64_t *off, const uint64_t *len,
                               const uint64_t *seed, const uint64_t *cbase, int zero_src);
void orc_volume_bytes(uint64_t M, uint32_t block_w, uint32_t block_g, uint64_t out[2]);
void orc_sr_r16_fill(uint64_t seed, uint64_t q0, size_t n, uint16_t *out);

static int failures = 0;
#define CHECK(c)                                                             \
    do {                                                                     \
        if (!(c)) {                                                          \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            failures++;                                                      \
        }                                                                    \
    } while (0)

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void)
{
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return (uint32_t)rng_state;
}

/* n exactly-sized allocations; malloc(0) may return NULL, so keep one byte */
static void *xalloc(size_t bytes)
{
    void *p = malloc(bytes ? bytes : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    memset(p, 0xA5, bytes ? bytes : 1);
    return p;
}

static float rnd_grad(void) { return ((float)(rnd() % 2001) - 1000.0f) * 1e-6f; }

static void fill_f32(float *x, size_t n)
{
    for (size_t i = 0; i < n; i++)
        x[i] = rnd_grad();
    if (n > 2) { /* specials inside the contract */
        x[0] = 0.0f;
        x[n / 2] = -0.0f;
        x[n - 1] = 1e-40f; /* subnormal */
    }
}

static void fill_bf16(uint16_t *x, size_t n)
{
    for (size_t i = 0; i < n; i++)
        x[i] = orc_bf16_rne(rnd_grad());
}

static size_t nblk(size_t n, uint32_t b) { return (n + b - 1) / b; }

static void quantizers(void)
{
    const uint32_t blocks[] = {2, 4, 32, 128, 4096};
    for (size_t bi = 0; bi < sizeof blocks / sizeof blocks[0]; bi++) {
        uint32_t B = blocks[bi];
        size_t sizes[] = {0, 1, 2, 3, B - 1, B, B + 1, 3 * (size_t)B + 5};
        for (size_t si = 0; si < sizeof sizes / sizeof sizes[0]; si++) {
            size_t n = sizes[si];
            for (int bf = 0; bf < 2; bf++) {
                for (int with_ef = 0; with_ef < 2; with_ef++) {
                    void *g = xalloc(n * (bf ? 2 : 4));
                    if (bf)
                        fill_bf16(g, n);
                    else
                        fill_f32(g, n);
                    float *ef = with_ef ? xalloc(n * 4) : NULL;
                    if (ef)
                        fill_f32(ef, n);
                    uint8_t *codes = xalloc((n + 1) / 2);
                    float *scales = xalloc(nblk(n, B) * 4);
                    CHECK(orc_quantize_ef_int4(g, bf, ef, n, B, 0.9f, 1.0f, codes, scales) == 0);
                    for (size_t i = 0; i < n; i++) {
                        int32_t k = orc_int4_decode(codes, i);
                        CHECK(k >= -7 && k <= 7);
                    }
                    int8_t *c8 = xalloc(n);
                    float *s8 = xalloc(nblk(n, B) * 4);
                    CHECK(orc_quant_int8(g, bf, n, B, c8, s8) == 0);
                    void *w = xalloc(n * 4);
                    CHECK(orc_dequant_int8(c8, s8, n, B, w, 0) == 0);
                    CHECK(orc_dequant_int8(c8, s8, n, B, w, 1) == 0);
                    free(g);
                    free(ef);
                    free(codes);
                    free(scales);
                    free(c8);
                    free(s8);
                    free(w);
                }
            }
        }
    }
}

static void reducer(void)
{
    const uint32_t peers[] = {1, 2, 3, 16};
    const uint32_t blocks[] = {2, 32, 4096};
    for (size_t pi = 0; pi < 4; pi++) {
        for (size_t bi = 0; bi < 3; bi++) {
            uint32_t P = peers[pi], B = blocks[bi];
            size_t sizes[] = {1, B - 1, 2 * (size_t)B + 3};
            for (size_t si = 0; si < 3; si++) {
                size_t n = sizes[si];
                uint8_t *codes[16];
                float *scales[16];
                for (uint32_t p = 0; p < P; p++) {
                    codes[p] = xalloc((n + 1) / 2);
                    scales[p] = xalloc(nblk(n, B) * 4);
                    for (size_t i = 0; i < (n + 1) / 2; i++)
                        codes[p][i] = (uint8_t)rnd();
                    for (size_t b = 0; b < nblk(n, B); b++)
                        scales[p][b] = (float)(rnd() % 1000) * 1e-7f;
                }
                for (int mode = 0; mode < 4; mode++) {
                    int want_out = mode != 1, rq = mode >= 1, ef = mode == 3;
                    float *out = want_out ? xalloc(n * 4) : NULL;
                    uint8_t *rqc = rq ? xalloc((n + 1) / 2) : NULL;
                    float *rqs = rq ? xalloc(nblk(n, B) * 4) : NULL;
                    float *rqe = ef ? xalloc(n * 4) : NULL;
                    if (rqe)
                        fill_f32(rqe, n);
                    float *work = xalloc(n * 4);
                    CHECK(orc_dequant_reduce(P, (const uint8_t *const *)codes,
                                             (const float *const *)scales, n, B, 0.25f, out, rqc,
                                             rqs, rqe, 0.9f, 1.0f, work) == 0);
                    free(out);
                    free(rqc);
                    free(rqs);
                    free(rqe);
                    free(work);
                }
                for (uint32_t p = 0; p < P; p++) {
                    free(codes[p]);
                    free(scales[p]);
                }
            }
        }
    }
}

static void permuted(void)
{
    const uint32_t shapes[][2] = {{4, 2}, {8, 4}, {1, 1}, {3, 5}};
    for (size_t t = 0; t < 4; t++) {
        uint32_t intra = shapes[t][0], inter = shapes[t][1], m = intra * inter;
        uint32_t *slots = xalloc(m * 4);
        CHECK(orc_zeropp_slots(intra, inter, slots) == 0);
        for (int bf = 0; bf < 2; bf++) {
            uint32_t B = 32;
            size_t part = 3 * B, n = part * m;
            void *g = xalloc(n * (bf ? 2 : 4));
            if (bf)
                fill_bf16(g, n);
            else
                fill_f32(g, n);
            float *ef = xalloc(n * 4);
            fill_f32(ef, n);
            uint8_t *codes = xalloc(n / 2);
            float *scales = xalloc(n / B * 4);
            CHECK(orc_quantize_ef_int4_permuted(g, bf, ef, n, B, 0.9f, 1.0f, m, slots, codes,
                                                scales) == 0);
            CHECK(orc_quantize_ef_int4_permuted(g, bf, NULL, n, B, 0.9f, 1.0f, m, slots, codes,
                                                scales) == 0);
            free(g);
            free(ef);
            free(codes);
            free(scales);
        }
        free(slots);
    }
}

static void stochastic_rounding(void)
{
    size_t sizes[] = {0, 1, 7, 8, 9, 1000};
    for (size_t si = 0; si < 6; si++) {
        size_t n = sizes[si];
        uint16_t *dst = xalloc(n * 2), *src = xalloc(n * 2);
        fill_bf16(dst, n);
        fill_bf16(src, n);
        CHECK(orc_sr_accumulate(dst, src, n, 42, (1ull << 35) + 3, 1) == 0);
        for (size_t i = 0; i < n; i++)
            CHECK(src[i] == 0);
        free(dst);
        free(src);
    }
    enum { S = 5 };
    uint16_t *dst[S], *src[S];
    uint64_t n[S], off[S], len[S], seed[S], cb[S];
    for (int i = 0; i < S; i++) {
        len[i] = 8 * (1 + rnd() % 20);
        off[i] = 8 * (rnd() % (len[i] / 8));
        n[i] = i == 2 ? 0 : rnd() % (len[i] - off[i] + 1);
        seed[i] = rnd();
        cb[i] = ((uint64_t)rnd() << 20) + off[i];
        dst[i] = xalloc(n[i] * 2);
        src[i] = xalloc(len[i] * 2);
        fill_bf16(dst[i], n[i]);
        fill_bf16(src[i], len[i]);
    }
    CHECK(orc_sr_accumulate_segments(S, dst, src, n, off, len, seed, cb, 0) == 0);
    CHECK(orc_sr_accumulate_segments(S, dst, src, n, off, len, seed, cb, 1) == 0);
    for (int i = 0; i < S; i++) {
        for (uint64_t j = 0; j < len[i]; j++)
            CHECK(src[i][j] == 0);
        free(dst[i]);
        free(src[i]);
    }
    uint16_t *r = xalloc(64 * 2);
    orc_sr_r16_fill(7, ~0ull - 64, 64, r);
    free(r);
    uint32_t ctr[4] = {1, 2, 3, 4}, key[2] = {5, 6}, o[4];
    orc_philox4x32_10(ctr, key, o);
    CHECK(orc_sr_round(NAN, 5) == 0x7FC0);
    uint64_t v[2];
    orc_volume_bytes(1ull << 40, 2048, 128, v);
    CHECK(v[0] == 6ull << 40);
}

static void refusals(void)
{
    float g[64] = {0};
    uint8_t codes[32];
    float scales[32];
    int8_t c8[64];
    memset(codes, 0x5A, sizeof codes);
    const uint32_t bad_blocks[] = {0, 1, 3, 4097, 8192};
    for (int i = 0; i < 5; i++) {
        CHECK(orc_quantize_ef_int4(g, 0, NULL, 64, bad_blocks[i], 0, 1, codes, scales) != 0);
        CHECK(orc_quant_int8(g, 0, 64, bad_blocks[i], c8, scales) != 0);
    }
    for (int i = 0; i < 32; i++)
        CHECK(codes[i] == 0x5A);
    CHECK(orc_quantize_ef_int4(g, 0, NULL, 64, 32, 0, 1, NULL, scales) != 0);
    CHECK(orc_quantize_ef_int4(NULL, 0, NULL, 64, 32, 0, 1, codes, scales) != 0);
    CHECK(orc_quant_int8(g, 0, 64, 32, NULL, scales) != 0);
    CHECK(orc_dequant_int8(c8, scales, 64, 32, NULL, 0) != 0);
    const uint8_t *cp[1] = {codes};
    const float *sp[1] = {scales};
    float work[64];
    CHECK(orc_dequant_reduce(0, cp, sp, 64, 32, 1, work, NULL, NULL, NULL, 0, 1, work) != 0);
    CHECK(orc_dequant_reduce(1, cp, sp, 64, 32, 1, NULL, NULL, NULL, NULL, 0, 1, work) != 0);
    CHECK(orc_dequant_reduce(1, cp, sp, 64, 32, 1, work, codes, NULL, NULL, 0, 1, work) != 0);
    CHECK(orc_dequant_reduce(1, cp, sp, 64, 8192, 1, work, NULL, NULL, NULL, 0, 1, work) != 0);
    uint32_t slots[4] = {0, 1, 1, 3};
    CHECK(orc_quantize_ef_int4_permuted(g, 0, NULL, 64, 16, 0, 1, 4, slots, codes, scales) != 0);
    slots[2] = 2;
    CHECK(orc_quantize_ef_int4_permuted(g, 0, NULL, 64, 32, 0, 1, 4, slots, codes, scales) != 0);
    CHECK(orc_quantize_ef_int4_permuted(g, 0, NULL, 64, 16, 0, 1, 4, slots, codes, scales) == 0);
    CHECK(orc_zeropp_slots(0, 1, slots) != 0);
    CHECK(orc_sr_accumulate(NULL, NULL, 4, 0, 0, 0) != 0);
    uint16_t d[4], s8[8];
    uint16_t *dp[1] = {d}, *spp[1] = {s8};
    uint64_t n1[1] = {4}, off1[1] = {6}, len1[1] = {8}, sd[1] = {0}, cb1[1] = {0};
    CHECK(orc_sr_accumulate_segments(1, dp, spp, n1, off1, len1, sd, cb1, 0) != 0);
}

int main(void)
{
    quantizers();
    reducer();
    permuted();
    stochastic_rounding();
    refusals();
#ifdef ZQ_SANITIZER_CANARY
    /* planted out-of-bounds read: proves the sanitizer build is armed */
    int *a = xalloc(4 * sizeof(int));
    volatile int sink = a[4];
    (void)sink;
    free(a);
#endif
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("oracle driver: all entry points ran clean\n");
    return 0;
}
