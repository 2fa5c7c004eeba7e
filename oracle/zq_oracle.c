/*
 * zq_oracle.c -- plain, single-threaded CPU oracle for the ZeRO++ / LoCo
 * block-quantization path and llm.c-style stochastic-rounding accumulation.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or constant with the GPU library; it is written straight from
 * the definitions below, one element at a time, with no blocking or fusion.
 *
 * Sources (web pages this path is defined by):
 *   [LoCo]   "Merge LoCo with Zero++" (DeepSpeed pull request 6730), Overview
 *            and the review thread on the LoCo quant kernel and the per-
 *            parameter error-feedback buffer.
 *   [ZeRO++] "ZeROPlusPlus.md" reading notes on the ZeRO++ paper: abstract,
 *            section 1 (communication volume) and section 1.2 (qwZ, hpZ, qgZ).
 *   [llm.c]  "Zero 2 #593" (llm.c pull request): review of llmc/cuda_utils.cuh
 *            (vector_add with stochastic rounding) and llmc/zero.cuh
 *            (zeroing the reduced buffer).
 *   [Philox] Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as
 *            1, 2, 3", SC'11, section on the Philox family.
 *
 * Arithmetic is IEEE-754 binary32 with round-to-nearest-even (the pages do
 * not fix a precision; the scheme is defined on fp32 values, so the oracle
 * computes in fp32 exactly as the definition states, each operation rounded
 * once).  Build with -O2 -ffp-contract=off and no fast-math so that the
 * compiler neither fuses a*b+c into one rounding nor reorders anything.
 *
 * Parity status of each function (pins live in the CPU test suite):
 *   orc_quant_block, orc_quantize_ef_int4, orc_quantize_ef_int4_permuted,
 *   orc_zeropp_slots, orc_dequant_reduce, orc_dequant_reduce_segments,
 *   orc_quant_int8, orc_dequant_int8,
 *   orc_bf16_rne, orc_f16_rne, orc_f16_to_f32, orc_sr_round,
 *   orc_philox4x32_10, orc_sr_accumulate,
 *   orc_sr_accumulate_segments, orc_volume_bytes: pinned.
 *
 * Every entry point that takes buffers checks its arguments first and
 * returns ORC_EINVAL (writing nothing) on NULL outputs, a block size the
 * fixed per-block work arrays cannot hold (block must be even and in
 * [2, 4096]), or inconsistent sizes; 0 means done.
 *   Agreement with DeepSpeed's or llm.c's own numerics: parity unpinned
 *   (the pages carry no code or outputs of theirs).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#define ORC_EINVAL (-1)

static int bad_block(uint32_t block) { return block < 2 || block > 4096 || (block & 1u); }

/* Element types of the 16- and 32-bit data streams (the int4 path's g, the
 * int8 path's w and its dequantized output): IEEE binary32, bf16 (the top
 * half of a binary32 pattern) and IEEE binary16. */
#define ORC_F32 0
#define ORC_BF16 1
#define ORC_F16 2

static int bad_dtype(int dtype) { return dtype != ORC_F32 && dtype != ORC_BF16 && dtype != ORC_F16; }

/* ---------------------------------------------------------------- bf16 -- */

/* bf16 -> fp32 is exact: the bf16 pattern is the top half of the fp32 one. */
static float bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static uint32_t f32_bits(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return u;
}

/* fp32 -> bf16, round to nearest, ties to even.  Keep the top 16 bits and
 * round on the 16 dropped ones: add just under half an ulp, plus one more
 * when the kept part is odd, so an exact tie goes to the even neighbour.
 * Carries propagate into the exponent, which is the correct rounding to the
 * next binade or to infinity.  NaN becomes the canonical quiet NaN 0x7FC0. */
uint16_t orc_bf16_rne(float f)
{
    if (isnan(f))
        return 0x7FC0u;
    uint32_t u = f32_bits(f);
    uint32_t keep_lsb = (u >> 16) & 1u;
    u += 0x7FFFu + keep_lsb;
    return (uint16_t)(u >> 16);
}

/* ---------------------------------------------------------------- fp16 -- */

/* IEEE 754 binary16: sign bit, 5 exponent bits with bias 15, 10 fraction
 * bits.  Exponent field 0 holds zero and the subnormals f * 2^-24, field 31
 * infinity (f = 0) and NaN.  Widening to binary32 is exact: a normal value is
 * (1024 + f) * 2^(e - 25), which binary32 holds; a NaN keeps its sign and
 * payload (shifted into the top of the binary32 fraction) and is quiet. */
static float f16_to_f32(uint16_t h)
{
    uint32_t sign = (uint32_t)(h >> 15) & 1u, e = (uint32_t)(h >> 10) & 0x1Fu, f = h & 0x3FFu;
    float v;
    if (e == 31) {
        uint32_t u = (sign << 31) | 0x7F800000u | (f << 13) | (f ? 0x00400000u : 0u);
        memcpy(&v, &u, sizeof v);
        return v;
    }
    if (e == 0)
        v = ldexpf((float)f, -24);
    else
        v = ldexpf((float)(f | 0x400u), (int)e - 25);
    return sign ? -v : v;
}

/* fp32 -> fp16, round to nearest, ties to even, from the definition: count
 * the value in units of the result's last place (2^-24 below 2^-14, the
 * subnormal range; 2^(E-10) for 2^E <= |x| < 2^(E+1)), which is an exact
 * power-of-two scaling, round that count to an integer (rintf, ties to even),
 * and assemble the pattern; a count that rounds up to the next power of two
 * carries into the exponent field by plain addition.  |x| >= 65520 (half an
 * ulp above the largest finite 65504) rounds to infinity; NaN becomes the
 * quiet NaN 0x7E00 with x's sign. */
uint16_t orc_f16_rne(float x)
{
    uint16_t sign = (uint16_t)((f32_bits(x) >> 16) & 0x8000u);
    if (isnan(x))
        return (uint16_t)(sign | 0x7E00u);
    float a = fabsf(x);
    if (a >= 65520.0f)
        return (uint16_t)(sign | 0x7C00u);
    if (a < 0x1p-14f)
        return (uint16_t)(sign | (uint16_t)rintf(a * 0x1p24f));
    int E;
    frexpf(a, &E); /* a = m 2^E, m in [0.5, 1): 2^(E-1) <= a < 2^E */
    E -= 1;
    uint32_t q = (uint32_t)rintf(ldexpf(a, 10 - E)); /* in [1024, 2048] */
    return (uint16_t)(sign | ((((uint32_t)(E + 15)) << 10) + (q - 1024u)));
}

/* One element of a data stream of the given type, widened to fp32. */
static float load_elem(const void *p, int dtype, size_t i)
{
    if (dtype == ORC_BF16)
        return bf16_to_f32(((const uint16_t *)p)[i]);
    if (dtype == ORC_F16)
        return f16_to_f32(((const uint16_t *)p)[i]);
    return ((const float *)p)[i];
}

/* fp16 exports for the pins: widening and rounding of one value. */
float orc_f16_to_f32(uint16_t h) { return f16_to_f32(h); }

/* ---------------------------------------------------- block quantizer -- */

/* Symmetric per-block absmax quantization, [ZeRO++] section 1.2 (qwZ uses
 * int8, qgZ int4; every block is quantized on its own).  The scheme:
 *   a = max |x_i|                       (exact)
 *   s = fl(a / qmax)                    (one IEEE divide)
 *   k_i = 0 if s == 0, else clamp(rne(fl(x_i / s)), -qmax, qmax)
 * Rounding is applied to the fp32 quotient, not to the exact ratio. */
void orc_quant_block(const float *x, size_t m, int qmax, int32_t *k, float *s_out)
{
    float a = 0.0f;
    for (size_t i = 0; i < m; i++) {
        float v = fabsf(x[i]);
        if (v > a)
            a = v;
    }
    float s = a / (float)qmax;
    for (size_t i = 0; i < m; i++) {
        if (s == 0.0f) {
            k[i] = 0;
            continue;
        }
        float q = x[i] / s;
        float r = rintf(q); /* default rounding mode: nearest, ties to even */
        /* clamp to [-qmax, qmax] with IEEE maxNum / minNum: for any number
         * this is the plain clamp; a NaN quotient, which only non-finite
         * inputs produce (outside the contract), gives -qmax */
        r = fmaxf(r, -(float)qmax);
        r = fminf(r, (float)qmax);
        k[i] = (int32_t)r;
    }
    *s_out = s;
}

/* Two's-complement nibble of code k; element 2j goes to the low nibble of
 * byte j, element 2j+1 to the high nibble. */
static void put_nibble(uint8_t *codes, size_t i, int32_t k)
{
    uint8_t nib = (uint8_t)((uint32_t)k & 0xFu);
    if ((i & 1u) == 0)
        codes[i / 2] = (uint8_t)((codes[i / 2] & 0xF0u) | nib);
    else
        codes[i / 2] = (uint8_t)((codes[i / 2] & 0x0Fu) | (uint8_t)(nib << 4));
}

/* Signed value of the nibble holding element i. */
static int32_t get_nibble(const uint8_t *codes, size_t i)
{
    uint32_t nib = (i & 1u) ? (uint32_t)(codes[i / 2] >> 4) : (uint32_t)(codes[i / 2] & 0xFu);
    return (nib & 8u) ? (int32_t)nib - 16 : (int32_t)nib;
}

int32_t orc_int4_decode(const uint8_t *codes, size_t i) { return get_nibble(codes, i); }

/* ------------------------------------------ EF int4 quantize (LoCo) -- */

/* Block int4 gradient quantization with error feedback, applied to the
 * gradient before it is communicated ([LoCo] Overview; the buffer is kept
 * per parameter, [LoCo] review thread).  Per element, in this order:
 *   c  = fl(g + e)            (c = g when there is no EF buffer)
 *   (k, s) = block quantizer of c with qmax = 7
 *   d  = fl(k * s)
 *   r  = fl(c - d)
 *   e' = fl(fl(beta_e * e) + fl(beta_r * r))     (only with an EF buffer)
 * g holds fp32, bf16 or fp16 values (g_dtype ORC_F32, ORC_BF16, ORC_F16);
 * 16-bit values are widened to fp32 exactly before anything else.
 * codes: ceil(n/2) bytes, scales: ceil(n/block) floats, ef: n floats or NULL.
 * block must be even and at most 4096.  The last block may be partial; its
 * scale uses only its own elements. */
int orc_quantize_ef_int4(const void *g, int g_dtype, float *ef, size_t n, uint32_t block,
                         float beta_e, float beta_r, uint8_t *codes, float *scales)
{
    if (bad_block(block) || bad_dtype(g_dtype) || (n > 0 && (!g || !codes || !scales)))
        return ORC_EINVAL;
    float c[4096];
    int32_t k[4096];
    size_t nb = (n + block - 1) / block;
    for (size_t b = 0; b < nb; b++) {
        size_t lo = b * (size_t)block;
        size_t m = n - lo < block ? n - lo : block;
        for (size_t j = 0; j < m; j++) {
            size_t i = lo + j;
            float gi = load_elem(g, g_dtype, i);
            c[j] = ef ? gi + ef[i] : gi;
        }
        float s;
        orc_quant_block(c, m, 7, k, &s);
        scales[b] = s;
        for (size_t j = 0; j < m; j++) {
            size_t i = lo + j;
            put_nibble(codes, i, k[j]);
            if (ef) {
                float d = (float)k[j] * s;
                float r = c[j] - d;
                float t1 = beta_e * ef[i];
                float t2 = beta_r * r;
                ef[i] = t1 + t2;
            }
        }
        if (m & 1u) /* odd element count: the unused high nibble is zero */
            codes[(lo + m) / 2] &= 0x0Fu;
    }
    return 0;
}

/* ----------------------------- hierarchical partition order (ZeRO++) -- */

/* ZeRO++ reduces gradients hierarchically, inside the node first and then
 * across nodes ([ZeRO++] section 1.2).  With `intra` GPUs per node and
 * `inter` nodes, rank r = node * intra + local owns partition r.  The
 * intra-node all-to-all sends chunk j of each GPU's buffer -- slots
 * j * inter .. j * inter + inter - 1 -- to local rank j; after the intra-node
 * reduction the inter-node all-to-all sends sub-chunk i of that result to
 * node i.  Partition r therefore has to sit in slot local * inter + node for
 * the two exchanges to bring it to rank r.  slot_of_part gets intra * inter
 * entries. */
int orc_zeropp_slots(uint32_t intra, uint32_t inter, uint32_t *slot_of_part)
{
    if (intra < 1 || inter < 1 || !slot_of_part)
        return ORC_EINVAL;
    for (uint32_t node = 0; node < inter; node++)
        for (uint32_t local = 0; local < intra; local++)
            slot_of_part[node * intra + local] = local * inter + node;
    return 0;
}

/* The EF int4 quantizer above with its outputs in a permuted partition
 * order.  The n elements form n_part equal partitions of whole blocks;
 * partition p is quantized exactly as orc_quantize_ef_int4 quantizes those
 * elements within the whole buffer (its blocks are the same blocks), and
 * its codes and scales are stored where partition slot_of_part[p] lies in
 * that function's layout.  g and ef keep their natural order. */
int orc_quantize_ef_int4_permuted(const void *g, int g_dtype, float *ef, size_t n,
                                  uint32_t block, float beta_e, float beta_r, uint32_t n_part,
                                  const uint32_t *slot_of_part, uint8_t *codes, float *scales)
{
    if (bad_block(block) || bad_dtype(g_dtype) || n_part < 1 || !slot_of_part || !g || !codes ||
        !scales)
        return ORC_EINVAL;
    size_t part = n / n_part;
    if (part * n_part != n || part % block != 0)
        return ORC_EINVAL;
    for (uint32_t p = 0; p < n_part; p++) { /* a permutation of 0 .. n_part-1 */
        if (slot_of_part[p] >= n_part)
            return ORC_EINVAL;
        for (uint32_t q = 0; q < p; q++)
            if (slot_of_part[q] == slot_of_part[p])
                return ORC_EINVAL;
    }
    for (uint32_t p = 0; p < n_part; p++) {
        size_t from = p * part;
        size_t to = slot_of_part[p] * part;
        const void *gp = g_dtype == ORC_F32 ? (const void *)((const float *)g + from)
                                            : (const void *)((const uint16_t *)g + from);
        int rc = orc_quantize_ef_int4(gp, g_dtype, ef ? ef + from : NULL, part, block, beta_e,
                                      beta_r, codes + to / 2, scales + to / block);
        if (rc)
            return rc;
    }
    return 0;
}

/* --------------------------------- dequantize + full-precision reduce -- */

/* qgZ receive side ([ZeRO++] section 1.2): P int4 chunks, each with its own
 * per-block scales, are dequantized and reduced in fp32.  Order is fixed:
 *   S = d_0;  S = fl(S + d_p) for p = 1 .. P-1,  d_p = fl(k_p * s_p)
 *   R = fl(alpha * S)          (alpha = 1 leaves S unchanged bit for bit)
 * out (n_chunk floats) receives R when non-NULL.  When rq_codes is non-NULL,
 * R is quantized again for the next level of the hierarchy (reduce inside
 * the node, then across nodes): the EF int4 quantizer above with input R,
 * optional EF buffer rq_ef and coefficients (rq_beta_e, rq_beta_r). */
int orc_dequant_reduce(uint32_t P, const uint8_t *const *codes, const float *const *scales,
                       size_t n_chunk, uint32_t block, float alpha, float *out,
                       uint8_t *rq_codes, float *rq_scales, float *rq_ef,
                       float rq_beta_e, float rq_beta_r, float *work /* n_chunk floats */)
{
    if (bad_block(block) || P < 1 || !codes || !scales || (!out && !rq_codes) ||
        (rq_codes && !rq_scales) || (rq_ef && !rq_codes) || (n_chunk > 0 && !work))
        return ORC_EINVAL;
    for (uint32_t p = 0; p < P; p++)
        if (n_chunk > 0 && (!codes[p] || !scales[p]))
            return ORC_EINVAL;
    for (size_t i = 0; i < n_chunk; i++) {
        size_t b = i / block;
        float S = (float)get_nibble(codes[0], i) * scales[0][b];
        for (uint32_t p = 1; p < P; p++) {
            float d = (float)get_nibble(codes[p], i) * scales[p][b];
            S = S + d;
        }
        float R = alpha * S;
        work[i] = R;
        if (out)
            out[i] = R;
    }
    if (rq_codes)
        return orc_quantize_ef_int4(work, 0, rq_ef, n_chunk, block, rq_beta_e, rq_beta_r, rq_codes,
                                    rq_scales);
    return 0;
}

/* The receive side parameter by parameter ([LoCo] review thread: the LoCo
 * path reduces each parameter's chunks separately, each with its own requant
 * error-feedback buffer): segment i is the reduce above over P chunks of n[i]
 * elements, peer p's chunk starting at codes[i] + p * cstride[i] bytes and
 * scales[i] + p * sstride[i] floats, into out[i] and / or rq_codes[i],
 * rq_scales[i], rq_ef[i] (any of these arrays may be NULL: no such output in
 * any segment).  work holds the largest n[i] floats. */
int orc_dequant_reduce_segments(uint32_t n_seg, const uint8_t *const *codes,
                                const float *const *scales, const uint64_t *cstride,
                                const uint64_t *sstride, const uint64_t *n, float *const *out,
                                uint8_t *const *rq_codes, float *const *rq_scales,
                                float *const *rq_ef, uint32_t P, uint32_t block, float alpha,
                                float rq_beta_e, float rq_beta_r, float *work)
{
    if (n_seg > 0 && (!codes || !scales || !cstride || !sstride || !n || !work))
        return ORC_EINVAL;
    if (P < 1 || P > 64)
        return ORC_EINVAL;
    for (uint32_t i = 0; i < n_seg; i++) {
        const uint8_t *cp[64];
        const float *sp[64];
        for (uint32_t p = 0; p < P; p++) {
            cp[p] = codes[i] + p * cstride[i];
            sp[p] = scales[i] + p * sstride[i];
        }
        if (n[i] == 0)
            continue;
        int rc = orc_dequant_reduce(P, cp, sp, n[i], block, alpha, out ? out[i] : NULL,
                                    rq_codes ? rq_codes[i] : NULL,
                                    rq_scales ? rq_scales[i] : NULL, rq_ef ? rq_ef[i] : NULL,
                                    rq_beta_e, rq_beta_r, work);
        if (rc)
            return rc;
    }
    return 0;
}

/* ------------------------------------------------ qwZ int8 weights -- */

/* Block int8 weight quantization before the forward all-gather ([ZeRO++]
 * section 1.2, qwZ, whose weights are fp16): the block quantizer with
 * qmax = 127, one fp32 scale per block, codes stored as int8.  w holds fp32,
 * bf16 or fp16 values (w_dtype), widened to fp32 exactly. */
int orc_quant_int8(const void *w, int w_dtype, size_t n, uint32_t block, int8_t *codes,
                   float *scales)
{
    if (bad_block(block) || bad_dtype(w_dtype) || (n > 0 && (!w || !codes || !scales)))
        return ORC_EINVAL;
    float x[4096];
    int32_t k[4096];
    size_t nb = (n + block - 1) / block;
    for (size_t b = 0; b < nb; b++) {
        size_t lo = b * (size_t)block;
        size_t m = n - lo < block ? n - lo : block;
        for (size_t j = 0; j < m; j++)
            x[j] = load_elem(w, w_dtype, lo + j);
        orc_quant_block(x, m, 127, k, &scales[b]);
        for (size_t j = 0; j < m; j++)
            codes[lo + j] = (int8_t)k[j];
    }
    return 0;
}

/* Dequantize after the all-gather: w' = fl(k * s), stored as fp32, or as
 * bf16 or fp16 rounded to nearest even from that fp32 value (out_dtype). */
int orc_dequant_int8(const int8_t *codes, const float *scales, size_t n, uint32_t block,
                     void *out, int out_dtype)
{
    if (block < 1 || bad_dtype(out_dtype) || (n > 0 && (!codes || !scales || !out)))
        return ORC_EINVAL;
    for (size_t i = 0; i < n; i++) {
        float v = (float)codes[i] * scales[i / block];
        if (out_dtype == ORC_BF16)
            ((uint16_t *)out)[i] = orc_bf16_rne(v);
        else if (out_dtype == ORC_F16)
            ((uint16_t *)out)[i] = orc_f16_rne(v);
        else
            ((float *)out)[i] = v;
    }
    return 0;
}

/* ------------------------------------------------------- Philox4x32 -- */

/* Philox-4x32 with 10 rounds, from the SC'11 paper.  State: four 32-bit
 * words; key: two 32-bit words.  One round multiplies words 0 and 2 by the
 * two round multipliers, and builds the new state from the products' high
 * and low halves, the other two words and the round key.  The key is bumped
 * by the two Weyl constants between rounds. */
#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

void orc_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4])
{
    uint32_t x0 = ctr_in[0], x1 = ctr_in[1], x2 = ctr_in[2], x3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int round = 0; round < 10; round++) {
        if (round > 0) {
            k0 += PHILOX_W0;
            k1 += PHILOX_W1;
        }
        uint64_t p0 = (uint64_t)PHILOX_M0 * (uint64_t)x0;
        uint64_t p1 = (uint64_t)PHILOX_M1 * (uint64_t)x2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t y0 = hi1 ^ x1 ^ k0;
        uint32_t y1 = lo1;
        uint32_t y2 = hi0 ^ x3 ^ k1;
        uint32_t y3 = lo0;
        x0 = y0;
        x1 = y1;
        x2 = y2;
        x3 = y3;
    }
    out[0] = x0;
    out[1] = x1;
    out[2] = x2;
    out[3] = x3;
}

/* The 16-bit random number for global element index q under seed:
 * Philox counter (q >> 3) (low word, high word, 0, 0), key (seed low word,
 * seed high word); one Philox call yields four 32-bit words, i.e. eight
 * 16-bit halves, used for q = 8c .. 8c+7 in order (low half first). */
uint32_t orc_sr_r16(uint64_t seed, uint64_t q)
{
    uint64_t c = q >> 3;
    uint32_t ctr[4] = {(uint32_t)c, (uint32_t)(c >> 32), 0u, 0u};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t w[4];
    orc_philox4x32_10(ctr, key, w);
    uint32_t word = w[(q & 7u) >> 1];
    return (q & 1u) ? (word >> 16) : (word & 0xFFFFu);
}

/* ------------------------------------- stochastic rounding to bf16 -- */

/* Stochastic rounding of fp32 x to bf16 with a 16-bit uniform r16: add r16
 * to the 16 bits that bf16 drops and truncate.  The magnitude rounds up with
 * probability (dropped bits)/2^16, so the result equals x in expectation
 * ([llm.c] review of vector_add: stochastic rounding keeps accumulation
 * correct in expectation).  NaN gives the canonical quiet NaN. */
uint16_t orc_sr_round(float x, uint32_t r16)
{
    if (isnan(x))
        return 0x7FC0u;
    uint32_t u = f32_bits(x);
    u = u + (r16 & 0xFFFFu);
    return (uint16_t)(u >> 16);
}

/* Gradient accumulation into a bf16 buffer, [llm.c] review of vector_add:
 * for each element the sum of the two bf16 values is formed in fp32, then
 * rounded stochastically back to bf16; the random number of element i is
 * that of global index counter_base + i.  With zero_src, the source element
 * is cleared after it is read (the pages' suggestion to fold the zeroing of
 * the reduced buffer into the add). */
int orc_sr_accumulate(uint16_t *dst, uint16_t *src, size_t n, uint64_t seed,
                      uint64_t counter_base, int zero_src)
{
    if (n > 0 && (!dst || !src))
        return ORC_EINVAL;
    for (size_t i = 0; i < n; i++) {
        float x = bf16_to_f32(dst[i]) + bf16_to_f32(src[i]);
        dst[i] = orc_sr_round(x, orc_sr_r16(seed, counter_base + i));
        if (zero_src)
            src[i] = 0;
    }
    return 0;
}

/* llm.c's per-tensor ZeRO-2 gradient accumulation ([llm.c] review of
 * llmc/zero.cuh): for tensor i in order, its shard dst[i][0, n[i])
 * accumulates the slice src[i][off[i], off[i] + n[i]) of the tensor's
 * reduced buffer with the stochastic-rounding add above (seed[i], counter
 * base cbase[i]); then, with zero_src, the whole reduced buffer
 * src[i][0, len[i]) is set to zero -- the memset the reviewers suggest
 * folding into the add. */
int orc_sr_accumulate_segments(uint32_t n_seg, uint16_t *const *dst, uint16_t *const *src,
                               const uint64_t *n, const uint64_t *off, const uint64_t *len,
                               const uint64_t *seed, const uint64_t *cbase, int zero_src)
{
    if (n_seg > 0 && (!dst || !src || !n || !off || !len || !seed || !cbase))
        return ORC_EINVAL;
    for (uint32_t i = 0; i < n_seg; i++) {
        if (off[i] > len[i] || n[i] > len[i] - off[i])
            return ORC_EINVAL;
        if ((n[i] > 0 && !dst[i]) || ((n[i] > 0 || (zero_src && len[i] > 0)) && !src[i]))
            return ORC_EINVAL;
    }
    for (uint32_t i = 0; i < n_seg; i++) {
        if (n[i] > 0)
            orc_sr_accumulate(dst[i], src[i] + off[i], n[i], seed[i], cbase[i], 0);
        if (zero_src && len[i] > 0)
            memset(src[i], 0, len[i] * sizeof(uint16_t));
    }
    return 0;
}

/* ------------------------------------------- communication volume -- */

/* Bytes one GPU sends per step for M parameters, [ZeRO++] abstract and
 * section 1.2.  ZeRO-3: two fp16 all-gathers of the weights and one fp16
 * reduce-scatter of the gradients: 3 * 2M bytes.  ZeRO++: int8 weights with
 * one fp32 scale per block_w elements, nothing across nodes for the backward
 * gather (hpZ keeps a replica in the node), int4 gradients with one fp32
 * scale per block_g elements.  out[0] = ZeRO bytes, out[1] = ZeRO++ bytes. */
void orc_volume_bytes(uint64_t M, uint32_t block_w, uint32_t block_g, uint64_t out[2])
{
    uint64_t zero3 = 3u * 2u * M;
    uint64_t qwz = M + 4u * ((M + block_w - 1) / block_w);
    uint64_t hpz = 0;
    uint64_t qgz = (M + 1) / 2 + 4u * ((M + block_g - 1) / block_g);
    out[0] = zero3;
    out[1] = qwz + hpz + qgz;
}

/* The random numbers of indices q0 .. q0+n-1 in order (for the statistical
 * tests of the stream). */
void orc_sr_r16_fill(uint64_t seed, uint64_t q0, size_t n, uint16_t *out)
{
    for (size_t i = 0; i < n; i++)
        out[i] = (uint16_t)orc_sr_r16(seed, q0 + i);
}
