/*
 * zq_c_step.c -- a native C caller of libzq with its own device memory and
 * stream (HIP runtime only, no Python): one small pass of the hot path,
 * inputs read from and outputs written to raw little-endian files in DIR.
 *
 *   DIR/g.bin    fp32[4 * NC]  gradient of this rank (4 chunks of NC)
 *   DIR/ef.bin   fp32[4 * NC]  its error-feedback buffer
 *   DIR/w.bin    bf16[NW]      weights for qwZ
 *   DIR/dst.bin  bf16[NS], DIR/src.bin bf16[NS]   SR accumulate operands
 * writes codes.out scales.out ef.out (EF int4 quantize, block 128, beta 0.9 / 1),
 * red.out rqc.out rqs.out (4-way reduce of the 4 chunks, alpha 1/4, requant),
 * c8.out s8.out wd.out (int8 block 2048 and its bf16 dequant), dst.out
 * (SR accumulate, seed 77, counter base 5).  Exit status 0 on success.
 * Test infrastructure (run by tests/test_gpu_native.py).
 */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "zq.h"

#define NC 40064u   /* 313 blocks of 128, a ragged reduce tile; 4 chunks per rank */
#define NW 10277u   /* qwZ weights, a partial last block */
#define NS 5003u    /* SR elements, a ragged tile */
#define B 128u

static const char *dir;

static int fail(const char *what, int code) {
    fprintf(stderr, "zq_c_step: %s (%d)\n", what, code);
    return 1;
}

static void *load(const char *name, size_t bytes) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE *f = fopen(path, "rb");
    void *p = malloc(bytes);
    if (!f || !p || fread(p, 1, bytes, f) != bytes) {
        fprintf(stderr, "zq_c_step: cannot read %s\n", path);
        exit(2);
    }
    fclose(f);
    return p;
}

static int save(const char *name, const void *dev, size_t bytes) {
    char path[4096];
    void *h = malloc(bytes);
    if (!h || hipMemcpy(h, dev, bytes, hipMemcpyDeviceToHost) != hipSuccess)
        return fail("copy back", 0);
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE *f = fopen(path, "wb");
    if (!f || fwrite(h, 1, bytes, f) != bytes)
        return fail("write output", 0);
    fclose(f);
    free(h);
    return 0;
}

static void *upload(const char *name, size_t bytes) {
    void *h = load(name, bytes), *d = NULL;
    if (hipMalloc(&d, bytes) != hipSuccess || hipMemcpy(d, h, bytes, hipMemcpyHostToDevice) != hipSuccess) {
        fprintf(stderr, "zq_c_step: upload %s failed\n", name);
        exit(3);
    }
    free(h);
    return d;
}

static void *device(size_t bytes) {
    void *d = NULL;
    if (hipMalloc(&d, bytes) != hipSuccess) {
        fprintf(stderr, "zq_c_step: hipMalloc failed\n");
        exit(3);
    }
    return d;
}

int main(int argc, char **argv) {
    if (argc != 2)
        return fail("usage: zq_c_step DIR", 0);
    dir = argv[1];
    const size_t n = 4 * (size_t)NC;
    float *g = upload("g.bin", n * 4), *ef = upload("ef.bin", n * 4);
    uint16_t *w = upload("w.bin", NW * 2), *dst = upload("dst.bin", NS * 2), *src = upload("src.bin", NS * 2);
    uint8_t *codes = device(zq_int4_code_bytes(n));
    float *scales = device(zq_num_blocks(n, B) * 4);
    float *red = device(NC * 4);
    uint8_t *rqc = device(zq_int4_code_bytes(NC));
    float *rqs = device(zq_num_blocks(NC, B) * 4);
    int8_t *c8 = device(NW);
    float *s8 = device(zq_num_blocks(NW, 2048) * 4);
    uint16_t *wd = device(NW * 2);
    hipStream_t st;
    if (hipStreamCreate(&st) != hipSuccess)
        return fail("hipStreamCreate", 0);

    zq_status s;
    /* a refused call (misaligned gradient) returns its status and enqueues nothing */
    s = zq_quantize_ef_int4((const char *)g + 4, ZQ_FP32, ef, n - 1, B, 0.9f, 1.0f, codes, scales, st);
    if (s != ZQ_ERR_ALIGN)
        return fail("misaligned gradient not refused", s);

    s = zq_quantize_ef_int4(g, ZQ_FP32, ef, n, B, 0.9f, 1.0f, codes, scales, st);
    if (s != ZQ_OK)
        return fail(zq_status_str(s), s);
    const uint8_t *cp[4];
    const float *sp[4];
    for (unsigned j = 0; j < 4; ++j) {
        cp[j] = codes + j * (NC / 2);
        sp[j] = scales + j * (NC / B);
    }
    s = zq_dequant_reduce(4, cp, sp, NC, B, 0.25f, red, rqc, rqs, NULL, 0.0f, 1.0f, st);
    if (s != ZQ_OK)
        return fail(zq_status_str(s), s);
    s = zq_quant_int8(w, ZQ_BF16, NW, 2048, c8, s8, st);
    if (s == ZQ_OK)
        s = zq_dequant_int8(c8, s8, NW, 2048, wd, ZQ_BF16, st);
    if (s != ZQ_OK)
        return fail(zq_status_str(s), s);
    s = zq_sr_accumulate(dst, src, NS, 77, 5, 0, st);
    if (s != ZQ_OK)
        return fail(zq_status_str(s), s);
    if (hipStreamSynchronize(st) != hipSuccess)
        return fail("hipStreamSynchronize", 0);

    if (save("codes.out", codes, zq_int4_code_bytes(n)) || save("scales.out", scales, zq_num_blocks(n, B) * 4) ||
        save("ef.out", ef, n * 4) || save("red.out", red, NC * 4) ||
        save("rqc.out", rqc, zq_int4_code_bytes(NC)) || save("rqs.out", rqs, zq_num_blocks(NC, B) * 4) ||
        save("c8.out", c8, NW) || save("s8.out", s8, zq_num_blocks(NW, 2048) * 4) ||
        save("wd.out", wd, NW * 2) || save("dst.out", dst, NS * 2))
        return 1;
    hipStreamDestroy(st);
    void *all[] = {g, ef, w, dst, src, codes, scales, red, rqc, rqs, c8, s8, wd};
    for (size_t i = 0; i < sizeof all / sizeof all[0]; ++i)
        hipFree(all[i]);
    puts("zq_c_step: ok");
    return 0;
}
