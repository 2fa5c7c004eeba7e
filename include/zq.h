/*
 * zq.h -- C ABI of libzq: the data-parallel hot path of ZeRO++ quantized
 * communication with LoCo error feedback, and llm.c-style stochastic-rounding
 * gradient accumulation, as hand-written HIP kernels for AMD Instinct MI355X
 * (gfx950).
 *
 * Sources (web pages; each entry point cites the passage that defines it):
 *   [LoCo]   "Merge LoCo with Zero++" (DeepSpeed pull request 6730):
 *            Overview; review thread on the per-parameter error-feedback
 *            buffer and on the LoCo quant kernel.
 *   [ZeRO++] "ZeROPlusPlus.md" reading notes on the ZeRO++ paper: abstract
 *            and section 1.2 (qwZ block int8 weights, hpZ, qgZ block int4
 *            gradients via all-to-all, reduce in full precision, intra-node
 *            then inter-node).
 *   [llm.c]  "Zero 2 #593" (llm.c pull request): review of llmc/zero.cuh
 *            (per-tensor vector_add on the reduced shard, then zeroing) and of
 *            llmc/cuda_utils.cuh (vector_add with stochastic rounding).
 *
 * Conventions shared by every compute entry point
 *   - Buffers are DEVICE pointers on the current HIP device unless stated.
 *     The caller allocates and frees everything; libzq never allocates,
 *     frees, or keeps a pointer past the call, and holds no mutable global
 *     state, so calls are reentrant and thread-safe.
 *   - `stream` is a hipStream_t passed as void*; NULL is the null stream.
 *     Every call only enqueues kernels on it and returns; results are ready
 *     when the stream reaches that point.
 *   - Arguments are validated on the host first; on any error the call
 *     returns that status and enqueues nothing.  dtype, block and P are
 *     checked first; then n == 0 is a no-op (ZQ_OK) that touches no pointer.
 *   - Data streams (g, ef, out, int4/int8 codes, w, dst, src) must be
 *     16-byte aligned (ZQ_ERR_ALIGN); per-block scale arrays must be 4-byte
 *     aligned.  Element counts may be any size up to 2^60 (ZQ_ERR_SIZE
 *     beyond); indexing is 64-bit.
 *   - block is a power of two in [32, 4096] (ZQ_ERR_BLOCK).
 *   - Inputs are expected finite.  A NaN or infinity inside a block makes
 *     that block's scale non-finite; results for it are defined by the same
 *     arithmetic but are outside the supported contract.
 *   - Results are defined by IEEE binary32 arithmetic, round to nearest
 *     even, no fused multiply-add, denormals kept, applied in the order each
 *     formula below is written (the kernels may take other instruction
 *     sequences, e.g. fused ones, only where they give the same bits);
 *     integer codes, scales (as bits), error-feedback buffers and bf16 / fp16
 *     outputs are bit-exact functions of the inputs.
 *
 * Layouts
 *   int4 codes: two's-complement nibbles, element 2j in the low nibble of
 *     byte j; ceil(n/2) bytes; for odd n the last high nibble is 0.
 *   int8 codes: one int8 per element.
 *   scales: one fp32 per block of `block` consecutive elements,
 *     ceil(n/block) of them; a partial last block's scale covers only its
 *     own elements.
 *   bf16, fp16: uint16 bit patterns.
 */
#ifndef ZQ_H
#define ZQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 1: the single-call entry points (the permuted quantize included) and the
 *    batched SR and EF quantize;
 * 2: adds ZQ_FP16, zq_zeropp_slots and zq_dequant_reduce_batched (earlier
 *    calls and layouts unchanged). */
#define ZQ_ABI_VERSION 2u

typedef enum {
    ZQ_OK = 0,
    ZQ_ERR_NULL = 1,   /* a required pointer is NULL                      */
    ZQ_ERR_SIZE = 2,   /* sizes inconsistent or too large                 */
    ZQ_ERR_BLOCK = 3,  /* block not a power of two in [32, 4096]          */
    ZQ_ERR_ALIGN = 4,  /* pointer misaligned (see conventions)            */
    ZQ_ERR_ALIAS = 5,  /* an output overlaps an input or another output   */
    ZQ_ERR_PEERS = 6,  /* P outside [1, 16]                               */
    ZQ_ERR_DTYPE = 7,  /* unknown dtype                                   */
    ZQ_ERR_LAUNCH = 8  /* the HIP kernel launch itself failed             */
} zq_status;

/* Element type of a data stream: IEEE binary32, bf16 (the top half of a
 * binary32 pattern) or IEEE binary16.  16-bit inputs are widened to fp32
 * exactly; 16-bit outputs are rounded to nearest even from fp32. */
typedef enum { ZQ_FP32 = 0, ZQ_BF16 = 1, ZQ_FP16 = 2 } zq_dtype;

/*
 * zq_quantize_ef_int4 -- block int4 gradient quantization with LoCo error
 * feedback ([LoCo] Overview: error feedback applied to the 4-bit gradients
 * before communication; [LoCo] review thread: the EF buffer lives with each
 * parameter; [ZeRO++] section 1.2: qgZ block-based int4 quantization).
 *
 * For each block of `block` elements, with e the EF buffer:
 *   c_i  = fl(g_i + e_i)                 (c_i = g_i when ef == NULL)
 *   a    = max_i |c_i|,  s = fl(a / 7)
 *   k_i  = 0 if s == 0, else clamp(round_half_even(fl(c_i / s)), -7, 7)
 *   d_i  = fl(k_i * s),  r_i = fl(c_i - d_i)
 *   e_i <- fl(fl(beta_e * e_i) + fl(beta_r * r_i))       (ef != NULL only)
 * LoCo's literal update is beta_e = beta, beta_r = 1; plain error feedback is
 * (0, 1); a moving-average reading is (beta, 1 - beta).
 *
 *   g       [n] fp32, bf16 or fp16 (g_dtype; the LoCo kernel's gradients are
 *           half precision, [LoCo] review thread), read only.
 *   ef      [n] fp32, read-modify-write in place; NULL for no error feedback.
 *   codes   [ceil(n/2)] bytes, written.     scales [ceil(n/block)] fp32, written.
 * Errors: NULL g/codes/scales; bad dtype or block; misalignment; codes or
 * scales overlapping g, ef or each other; ef overlapping g.
 */
zq_status zq_quantize_ef_int4(const void *g, zq_dtype g_dtype, float *ef, size_t n,
                              uint32_t block, float beta_e, float beta_r, uint8_t *codes,
                              float *scales, void *stream);

/*
 * zq_quantize_ef_int4_permuted -- zq_quantize_ef_int4 writing its codes and
 * scales in a permuted partition order, so that after the two all-to-alls of
 * hierarchical qgZ every rank holds its own contiguous partition ([ZeRO++]
 * section 1.2: gradients are reduced inside the node first, then across
 * nodes; the slices are reordered before quantization for that).
 *
 * The n elements are n_part equal partitions of part_len = n / n_part
 * elements.  Partition p's codes and scales are written where partition
 * slot_of_part[p] would be in zq_quantize_ef_int4's output; g and ef keep
 * their natural order.  ZeRO++'s order for intra GPUs per node and inter
 * nodes (n_part = intra * inter) is what zq_zeropp_slots writes.
 *
 *   n_part        1 .. 256; part_len must be a multiple of block and at least
 *                 max(1024, block) (ZQ_ERR_SIZE otherwise).
 *   slot_of_part  HOST array of n_part distinct values in [0, n_part)
 *                 (ZQ_ERR_SIZE if not a permutation).
 * Other arguments and errors as zq_quantize_ef_int4.
 */
zq_status zq_quantize_ef_int4_permuted(const void *g, zq_dtype g_dtype, float *ef, size_t n,
                                       uint32_t block, float beta_e, float beta_r, uint8_t *codes,
                                       float *scales, uint32_t n_part,
                                       const uint32_t *slot_of_part, void *stream);

/*
 * zq_quantize_ef_int4_batched -- zq_quantize_ef_int4 over many tensors in one
 * call: DeepSpeed's LoCo path quantizes parameter by parameter, each with
 * its own error-feedback buffer ([LoCo] review thread: the EF buffer kept on
 * each parameter, p.inter_ef_buf); here one pass covers all of them, up to
 * 80 tensors per kernel launch (the table travels in the kernel arguments;
 * nothing is allocated).
 *
 * Segment i is exactly zq_quantize_ef_int4(seg.g, g_dtype, seg.ef, seg.n,
 * block, beta_e, beta_r, seg.codes, seg.scales): blocks restart at every
 * segment and a segment's last block may be partial.
 *   segs   HOST array of n_seg segments; every pointer 16-byte aligned (scales
 *          4-byte); ef is NULL in all segments or in none (ZQ_ERR_NULL).
 * Errors: as zq_quantize_ef_int4 per segment; ZQ_ERR_SIZE for n_seg > 65536
 * or a segment longer than 2^40 elements; ZQ_ERR_ALIAS when any output (or
 * EF buffer) overlaps any other range of any segment.
 */
typedef struct {
    const void *g;
    float *ef;
    uint8_t *codes;
    float *scales;
    uint64_t n;
} zq_efq_segment;

zq_status zq_quantize_ef_int4_batched(const zq_efq_segment *segs, uint32_t n_seg, zq_dtype g_dtype,
                                      uint32_t block, float beta_e, float beta_r, void *stream);

/*
 * zq_dequant_reduce -- qgZ receive side: dequantize the P int4 chunks an
 * all-to-all delivers to this GPU and reduce them in full precision, with an
 * optional requantization for the next level of the hierarchy ([ZeRO++]
 * section 1.2: int4 on the wire, reduction back in full precision, first
 * inside the node and then across nodes; the kernels are fused to cut
 * latency).
 *
 * For element i of the chunk (block b = i / block):
 *   S_i = d_{0,i};  S_i = fl(S_i + d_{p,i}) for p = 1 .. P-1,
 *   d_{p,i} = fl(k_{p,i} * s_{p,b});   R_i = fl(alpha * S_i)
 * out_i = R_i when out != NULL.  When rq_codes != NULL, R is quantized again
 * exactly as zq_quantize_ef_int4 does (same block, input R, EF buffer rq_ef
 * with coefficients rq_beta_e, rq_beta_r, or no EF when rq_ef == NULL).
 *
 *   P        number of chunks, 1 <= P <= 16.
 *   codes    HOST array of P device pointers, each [ceil(n_chunk/2)] bytes.
 *   scales   HOST array of P device pointers, each [ceil(n_chunk/block)] fp32.
 *   out      [n_chunk] fp32 written, or NULL.
 *   rq_codes [ceil(n_chunk/2)] bytes and rq_scales [ceil(n_chunk/block)] fp32
 *            written, or both NULL.  rq_ef [n_chunk] fp32 read-modify-write
 *            or NULL (only with rq_codes).
 * At least one of out / rq_codes is required (ZQ_ERR_NULL otherwise).
 * Outputs must not overlap any input chunk or each other (ZQ_ERR_ALIAS).
 */
zq_status zq_dequant_reduce(uint32_t P, const uint8_t *const *codes, const float *const *scales,
                            size_t n_chunk, uint32_t block, float alpha, float *out,
                            uint8_t *rq_codes, float *rq_scales, float *rq_ef, float rq_beta_e,
                            float rq_beta_r, void *stream);

/*
 * zq_dequant_reduce_batched -- zq_dequant_reduce over many tensors in one
 * call: DeepSpeed's LoCo path reduces what the all-to-all delivered
 * parameter by parameter, each parameter with its own requant error-feedback
 * buffer ([LoCo] review thread: all_to_all_loco_quant_reduce over the
 * parameters to reduce, each with p.inter_ef_buf); here one pass covers all
 * of them, up to 48 tensors per kernel launch (the table travels in the
 * kernel arguments; nothing is allocated).
 *
 * Segment i is exactly zq_dequant_reduce(P, {codes + q * codes_stride},
 * {scales + q * scales_stride}, n, block, alpha, out, rq_codes, rq_scales,
 * rq_ef, rq_beta_e, rq_beta_r): peer q's chunk of the tensor starts
 * codes_stride bytes and scales_stride floats after peer q - 1's, the layout
 * an all-to-all receive buffer has.  Blocks restart at every segment and a
 * segment's last block may be partial.
 *   segs   HOST array of n_seg segments (read during the call only).
 *          codes 16-byte aligned, codes_stride a multiple of 16 and at least
 *          ceil(n/2) (any value when P == 1); scales 4-byte aligned,
 *          scales_stride at least ceil(n/block); out, rq_codes, rq_ef
 *          16-byte aligned, rq_scales 4-byte aligned.  out is NULL in every
 *          non-empty segment or in none, and so are rq_codes (with rq_scales)
 *          and rq_ef (only with rq_codes); at least one of out / rq_codes.
 * Errors: ZQ_ERR_PEERS, ZQ_ERR_BLOCK; ZQ_ERR_NULL (segs NULL with n_seg > 0,
 * a NULL input of a non-empty segment, outputs present in some segments
 * only, or neither output); ZQ_ERR_SIZE (n_seg > 65536, a segment longer than
 * 2^40 elements, a stride too short or above 2^50); ZQ_ERR_ALIGN;
 * ZQ_ERR_ALIAS (any written range overlapping any input range or another
 * written range of any segment; inputs may overlap each other).
 */
typedef struct {
    const uint8_t *codes;
    const float *scales;
    uint64_t codes_stride;   /* bytes between peers' code chunks    */
    uint64_t scales_stride;  /* floats between peers' scale chunks  */
    uint64_t n;              /* elements per chunk                  */
    float *out;
    uint8_t *rq_codes;
    float *rq_scales;
    float *rq_ef;
} zq_dr_segment;

zq_status zq_dequant_reduce_batched(const zq_dr_segment *segs, uint32_t n_seg, uint32_t P,
                                    uint32_t block, float alpha, float rq_beta_e, float rq_beta_r,
                                    void *stream);

/*
 * zq_quant_int8 -- qwZ: block int8 quantization of the weights before the
 * forward all-gather ([ZeRO++] section 1.2: fp16 to int8, an independent
 * quantization per block of parameters for accuracy).
 *   s = fl(max|w| / 127);  k_i = 0 if s == 0 else clamp(rne(fl(w_i / s)), -127, 127)
 *   w      [n] fp32, bf16 or fp16 (w_dtype; the pages' qwZ weights are fp16),
 *          read only.
 *   codes  [n] int8 written.   scales [ceil(n/block)] fp32 written.
 */
zq_status zq_quant_int8(const void *w, zq_dtype w_dtype, size_t n, uint32_t block, int8_t *codes,
                        float *scales, void *stream);

/*
 * zq_dequant_int8 -- qwZ receive side: w'_i = fl(k_i * s_b), stored as fp32
 * or rounded to nearest even bf16 or fp16 ([ZeRO++] section 1.2: the weights
 * return to fp16 for the layer's compute); fp16 results from 65520 in
 * magnitude up are infinite.
 *   codes [n] int8, scales [ceil(n/block)] fp32, read only.
 *   out   [n] fp32, bf16 or fp16 (out_dtype), written; must not overlap the
 *         inputs.
 */
zq_status zq_dequant_int8(const int8_t *codes, const float *scales, size_t n, uint32_t block,
                          void *out, zq_dtype out_dtype, void *stream);

/*
 * zq_sr_accumulate -- llm.c ZeRO-2 gradient accumulation into the bf16 shard
 * with stochastic rounding ([llm.c] review of llmc/cuda_utils.cuh: the sum of
 * the two bf16 values is formed in fp32 and rounded stochastically, so
 * accumulation is correct in expectation; review of llmc/zero.cuh: the
 * zeroing of the reduced buffer can be folded into the same kernel).
 *
 *   x_i   = fl(float(dst_i) + float(src_i))
 *   q     = counter_base + i
 *   W     = Philox4x32-10(counter = (lo32(q>>3), hi32(q>>3), 0, 0),
 *                         key = (lo32(seed), hi32(seed)))
 *   r16   = 16-bit half (q & 1) (low half first) of word W[(q & 7) >> 1]
 *   dst_i = 0x7FC0 if x_i is NaN, else ((bits(x_i) + r16) mod 2^32) >> 16
 *   src_i = 0 afterwards when zero_src != 0.
 * Using the GLOBAL element index as the counter makes a shard's accumulation
 * (counter_base = shard offset) bit-identical to the same slice of a
 * full-buffer accumulation.
 *
 *   dst [n] bf16 read-modify-write;  src [n] bf16 read (written when
 *   zero_src).  dst and src must not overlap (ZQ_ERR_ALIAS).  counter_base + n
 *   must not exceed 2^64 - 1 (ZQ_ERR_SIZE).
 */
zq_status zq_sr_accumulate(uint16_t *dst_bf16, uint16_t *src_bf16, size_t n, uint64_t seed,
                           uint64_t counter_base, int zero_src, void *stream);

/*
 * zq_sr_accumulate_batched -- the per-tensor loop of llm.c's ZeRO-2 gradient
 * accumulation in one call ([llm.c] review of llmc/zero.cuh: for each tensor
 * i, vector_add(shard_i, reduced_i + rank * n_i, n_i, seed + i) followed by a
 * memset of the whole reduced_i -- tiny back-to-back kernels whose idle gaps
 * the reviewers point out, and the memset that could be fused into the add).
 *
 * Segment i does exactly what zq_sr_accumulate(seg.dst, seg.src +
 * seg.src_offset, seg.n, seg.seed, seg.counter_base, 0) does, and then, when
 * zero_src != 0, sets ALL seg.src_len elements of seg.src to 0 (the read
 * slice after it is read).  Segments run in one pass, up to 50 per kernel
 * launch (the table travels in the kernel arguments; nothing is allocated).
 *
 *   segs      HOST array of n_seg segments (read during the call only).
 *   dst       [n] bf16 accumulator, 16-byte aligned.
 *   src       [src_len] bf16 reduced buffer, 16-byte aligned; src_offset is
 *             a multiple of 8 and src_offset + n <= src_len.
 *   seed, counter_base   as in zq_sr_accumulate (counter_base + n <= 2^64 - 1).
 * Errors: ZQ_ERR_NULL (segs NULL with n_seg > 0, or a NULL buffer of a
 * non-empty segment), ZQ_ERR_SIZE (offset / length / counter overflow, a
 * segment longer than 2^40 elements, or n_seg > 65536), ZQ_ERR_ALIGN, ZQ_ERR_ALIAS (any written range -- a dst, or
 * a src buffer when zero_src -- overlapping any other segment's range).
 */
typedef struct {
    uint16_t *dst;
    uint16_t *src;
    uint64_t n;
    uint64_t src_offset;
    uint64_t src_len;
    uint64_t seed;
    uint64_t counter_base;
} zq_sr_segment;

zq_status zq_sr_accumulate_batched(const zq_sr_segment *segs, uint32_t n_seg, int zero_src,
                                   void *stream);

/*
 * zq_zeropp_slots -- ZeRO++'s partition order for zq_quantize_ef_int4_permuted
 * ([ZeRO++] section 1.2: gradients are reduced inside the node first, then
 * across nodes, and the slices are reordered before quantization so that
 * both all-to-alls deliver each rank its own partition).  Host only.
 *
 * With `intra` GPUs per node and `inter` nodes, rank r = node * intra + local
 * owns partition r.  The intra-node all-to-all sends chunk j of a GPU's
 * quantized buffer (slots j * inter .. j * inter + inter - 1) to local rank
 * j; after the intra-node reduce, sub-chunk i of the result goes to node i.
 * Partition r must therefore sit in slot local * inter + node:
 *   slot_of_part[node * intra + local] = local * inter + node.
 *
 *   slot_of_part  HOST array of intra * inter entries, written.
 * Returns intra * inter, or 0 (writing nothing) when slot_of_part is NULL,
 * intra or inter is 0, or intra * inter exceeds 256 (the most partitions
 * zq_quantize_ef_int4_permuted takes).
 */
uint32_t zq_zeropp_slots(uint32_t intra, uint32_t inter, uint32_t *slot_of_part);

/* Host-only helpers (no device work, usable without a GPU). */
size_t zq_int4_code_bytes(size_t n);               /* ceil(n/2)                        */
size_t zq_num_blocks(size_t n, uint32_t block);    /* ceil(n/block); 0 if block == 0   */
const char *zq_status_str(zq_status s);            /* static string, never NULL        */
uint32_t zq_abi_version(void);                     /* ZQ_ABI_VERSION                   */

#ifdef __cplusplus
}
#endif

#endif /* ZQ_H */
