/*
 * zpq.h -- C ABI of libzpq: block-quantized communication kernels of ZeRO++
 * (qwZ and qgZ) for AMD Instinct MI355X (gfx950).
 *
 * Sources (web pages about "ZeRO++: Extremely Efficient Collective
 * Communication for Giant Model Training", arXiv 2306.10209):
 *   [SUM] atlas.scime.ai summary page ("ZeRO++: ... for Large Model Training")
 *   [ABS] mlsanity.com index page, section "Abstract (arXiv)"
 *   [LIT] anthology-of-the-sota record LIT-102, section "Key takeaways"
 *
 * Quantizer (the pages say only "block-wise"; it is fixed here as follows):
 *   a block is `block` consecutive elements; its scale is
 *   s = fl32(max|x| / qmax) with qmax = 127 (INT8) or 7 (INT4); each code is
 *   q = clamp(round_half_even(fl32(x / s)), -qmax, qmax) using IEEE fp32
 *   division; a block whose scale is 0 has all codes 0.  Dequantization is
 *   d = fl32(q * s), rounded to nearest even into the output type.  INT4
 *   codes are two's-complement nibbles, two per byte, element 2k in the low
 *   nibble of byte k.  Results are bit-identical to that definition for all
 *   finite inputs, with two qualifications: where the definition itself
 *   produces a NaN (a reduced sum that meets +inf and -inf), the result is a
 *   NaN of unspecified sign and payload; and a block whose reduced sums are
 *   not all finite has unspecified INT4 codes and scale (the quantizer is
 *   defined on finite values only).  Non-finite inputs give unspecified (but
 *   in-bounds) results.
 *
 * Conventions shared by every entry point:
 *   - All buffer arguments are DEVICE pointers owned by the caller; the
 *     library allocates nothing, keeps no state between calls and never
 *     synchronizes.  Work is enqueued on `stream` (a hipStream_t; NULL is the
 *     null stream) and the call returns before it completes.
 *   - Arguments are checked on the host before anything is launched; on any
 *     error nothing is launched and nothing is written.  Checked: pointers
 *     non-NULL (may be NULL only when there are no elements), 16-byte aligned,
 *     and input and output ranges disjoint; sizes non-negative and whole
 *     blocks (callers pad, as ZeRO pads partitions); block in
 *     {32, 64, 128, 256, 512}; element types valid.
 *   - Element counts are 64-bit, at most 2^40 (else ZPQ_ERR_SIZE); buffers
 *     above 2^31 bytes are supported.
 *   - ZPQ_ERR_LAUNCH reports a launch failure from the HIP runtime (for
 *     example a device other than gfx950), read with hipGetLastError after
 *     the launches: an error left pending by an earlier HIP call on the same
 *     host thread is reported (and cleared) the same way.
 *   - Calls that write the same output concurrently race; calls on one
 *     stream are ordered.
 */
#ifndef ZPQ_H
#define ZPQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ZPQ_ABI_VERSION 1

typedef enum {
    ZPQ_OK = 0,
    ZPQ_ERR_NULL = 1,    /* a required pointer is NULL */
    ZPQ_ERR_SIZE = 2,    /* negative size, or not a whole number of blocks / slices */
    ZPQ_ERR_BLOCK = 3,   /* block not in {32, 64, 128, 256, 512} */
    ZPQ_ERR_ALIGN = 4,   /* a pointer is not 16-byte aligned */
    ZPQ_ERR_DTYPE = 5,   /* element type not supported by this entry point */
    ZPQ_ERR_MODE = 6,    /* not exactly one output mode selected */
    ZPQ_ERR_LAUNCH = 7,  /* the HIP runtime refused the launch */
    ZPQ_ERR_ARG = 8,     /* other invalid argument (L, N, n_src, divisor) */
    ZPQ_ERR_ALIAS = 9    /* an output range overlaps an input range */
} zpq_status;

/* Element types of float tensors (passed as int32_t). */
typedef enum { ZPQ_F32 = 0, ZPQ_F16 = 1, ZPQ_BF16 = 2 } zpq_dtype;

typedef void* zpq_stream; /* hipStream_t */

/*
 * qwZ quantize: INT8 block quantization of a weight shard before the forward
 * all-gather ([SUM] "Approach": block-wise INT8 quantization of weights for
 * the forward all-gather; [ABS]: block-quantization based all-gather).
 *
 *   x      [n] elements of type x_dtype (ZPQ_F32, ZPQ_F16 or ZPQ_BF16)
 *   codes  [n] int8 codes in [-127, 127], same order as x        (written)
 *   scales [n / block] fp32 scales, one per block, in order       (written)
 */
zpq_status zpq_quant_i8(const void* x, int32_t x_dtype, int64_t n, int32_t block,
                        int8_t* codes, float* scales, zpq_stream stream);

/*
 * qwZ dequantize: the gathered INT8 buffer back to a float type after the
 * all-gather ([SUM] "Approach"; [ABS]).  A gathered buffer of W shards is the
 * concatenation of their codes and of their scales, so this is one call.
 *
 *   codes  [n] int8, scales [n / block] fp32
 *   y      [n] elements of type y_dtype: RNE(fl32(q * s))          (written)
 */
zpq_status zpq_dequant_i8(const int8_t* codes, const float* scales, int64_t n,
                          int32_t block, void* y, int32_t y_dtype, zpq_stream stream);

/*
 * Non-blocked (per-tensor) INT8 quantization: one scale for the whole tensor.
 * The ablation baseline of qwZ ([SUM] Measured effects table: basic
 * non-blocked instead of block-based quantization, which hurt convergence;
 * Surprising findings: naive non-blocked INT8 weights diverged).
 *
 *   x      [n] elements of type x_dtype; n % 16 == 0 (callers pad with zeros)
 *   codes  [n] int8 codes in [-127, 127]                          (written)
 *   scale  [1] fp32: fl32(max|x| / 127)                            (written)
 * The codes buffer also holds intermediate per-workgroup maxima during the
 * call (three kernels on `stream`); nothing else is touched.
 */
zpq_status zpq_quant_i8_tensor(const void* x, int32_t x_dtype, int64_t n, int8_t* codes,
                               float* scale, zpq_stream stream);

/*
 * qgZ, before the intra-node all-to-all: tensor-slice reordering fused with
 * INT4 block quantization ([SUM] "Approach": slice reordering for correct
 * placement ahead of a 2-hop all-to-all of INT4 gradients; [ABS]: all-to-all
 * based quantized gradient averaging in place of reduce-scatter).
 *
 * The W = L*N ranks are numbered r = node*L + local; rank r owns flat slice r
 * of S = n / W elements.  Send position p = j*N + m (j < L, m < N) carries
 * slice m*L + j, so that after hop 1 (chunk j -> local rank j) and hop 2
 * (position m of a chunk -> node m) every slice sits at its owner.
 *
 *   grad   [n] elements of type g_dtype; n % (L*N*block) == 0
 *   codes  [n / 2] bytes: packed INT4 codes of the reordered tensor;
 *          bytes [j*n/(2L), (j+1)*n/(2L)) are the hop-1 chunk for local rank j
 *   scales [n / block] fp32 scales of the reordered tensor (chunk j is
 *          [j*n/(L*block), (j+1)*n/(L*block)))
 */
zpq_status zpq_qgz_reorder_quant_i4(const void* grad, int32_t g_dtype, int64_t n,
                                    int32_t local_ranks, int32_t nodes, int32_t block,
                                    uint8_t* codes, float* scales, zpq_stream stream);

/*
 * qgZ, after each all-to-all hop: dequantize the n_src received INT4 chunks,
 * reduce them in fp32 in source order 0..n_src-1 starting from +0 (one
 * rounding per addition, no fused multiply-add), then either
 *   mode I4 (hop 1): requantize the sum to INT4 with the same block size;
 *            the result is the hop-2 send buffer (position m = slice for
 *            node m)   -- out_codes [chunk/2], out_scales [chunk/block];
 *   mode FLOAT (hop 2): y = RNE_out(fl32(sum / divisor)) -- the averaged
 *            gradient slice; divisor is the world size W  -- out_vals [chunk]
 *            of type out_dtype (ZPQ_F32, ZPQ_F16 or ZPQ_BF16).
 * Exactly one mode: (out_codes, out_scales non-NULL and out_vals NULL) or
 * the reverse, else ZPQ_ERR_MODE.  FLOAT mode needs 0 < divisor < inf.
 * ([SUM] "Approach" and "Surprising findings": dequantize before reduction,
 * two hops, intra-node then inter-node; [LIT] second bullet: reduction done
 * locally in higher precision.)
 *
 *   in_codes  [n_src][chunk/2] bytes, source-major (as received)
 *   in_scales [n_src][chunk/block] fp32
 * Scales must be finite.
 */
zpq_status zpq_qgz_dequant_reduce_requant_i4(const uint8_t* in_codes, const float* in_scales,
                                             int32_t n_src, int64_t chunk_elems, int32_t block,
                                             uint8_t* out_codes, float* out_scales,
                                             void* out_vals, int32_t out_dtype, float divisor,
                                             zpq_stream stream);

/* Human-readable name of a status code (static string, never NULL). */
const char* zpq_status_str(zpq_status s);

/* ZPQ_ABI_VERSION of the loaded library. */
int32_t zpq_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ZPQ_H */
