/*
 * zpq_ref.c -- CPU oracle for the ZeRO++ block-quantized communication path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  The product library
 * (libzpq) never calls it, includes it, or shares code with it.
 *
 * What it computes.  The ZeRO++ pages describe two quantized collectives of
 * ZeRO-3 data parallelism:
 *   - qwZ: weights are quantized block-wise to INT8 before the forward
 *     all-gather and dequantized after it (ZeRO++ summary page, atlas.scime.ai,
 *     "Approach"; ZeRO++ index page, mlsanity.com, "Abstract (arXiv)", first
 *     technique).
 *   - qgZ: gradients are reordered slice-wise, quantized to INT4 and averaged
 *     with a two-hop all-to-all (intra-node, then inter-node) in which every
 *     receiver dequantizes before it reduces (summary page, "Approach" and
 *     "Surprising findings"; LIT-102 anthology record, "Key takeaways",
 *     second bullet: the reduction happens locally in higher precision).
 * The pages say "block-wise" and no more.  The quantizer used here is fixed as:
 *   scale s = fl32(absmax / qmax), qmax = 127 (INT8) or 7 (INT4), kept in fp32;
 *   code  q = clamp(round_half_even(fl32(x / s)), -qmax, qmax), IEEE division;
 *   a block whose scale is 0 gets codes 0;
 *   INT4 codes are two's-complement nibbles, two per byte, element 2k in the
 *   low nibble of byte k.
 * The reduction is an fp32 sum in source-rank order 0..K-1 starting from +0,
 * one rounding per addition; the final hop divides by the world size.
 *
 * Style: the steps are written one after another, in the order above, with
 * scalar float arithmetic.  Build with -O2 -ffp-contract=off and without
 * -ffast-math, so that every float operation is one IEEE binary32 operation
 * rounded to nearest-even (x86-64 uses SSE for float; no x87 excess precision).
 *
 * Step map (names used by the tests):
 *   O1 widen        zpq_ref_f16_to_f32 / zpq_ref_bf16_to_f32
 *   O2-O4 quantize  zpq_ref_block_quant
 *   O5 pack         zpq_ref_pack_i4 / zpq_ref_unpack_i4
 *   O6 dequantize   zpq_ref_block_dequant (+ zpq_ref_f32_to_f16 / _bf16)
 *   O7 reorder      zpq_ref_reorder
 *   O8 reduce       zpq_ref_reduce_add
 *   O9 average      zpq_ref_average
 * and four compositions that mirror libzpq's entry points (its per-tensor
 * quantizer is zpq_ref_quant_i8 with a single block spanning the tensor).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define REF_OK 0
#define REF_ERR_ARG 1
#define REF_ERR_NONFINITE 2
#define REF_ERR_NOMEM 3

/* Element types, numbered like the product's ABI (an interface both sides
 * must agree on; the numbering is the only thing shared, by value). */
#define REF_F32 0
#define REF_F16 1
#define REF_BF16 2

/* ------------------------------------------------------------------------ */
/* O1 / O6: conversions between fp32 and the 16-bit formats, written from the
 * IEEE 754 binary16 definition and the bfloat16 layout (the top half of a
 * binary32).  No hardware conversion instruction is used.                   */

static float f16_bits_to_f32(uint16_t h) {
    int sign = h >> 15;
    int e = (h >> 10) & 0x1F;
    int m = h & 0x3FF;
    float v;
    if (e == 0) {
        v = ldexpf((float)m, -24);                 /* subnormal: m * 2^-24 */
    } else if (e == 31) {
        v = m ? NAN : INFINITY;
    } else {
        v = ldexpf((float)(1024 + m), e - 25);     /* (1 + m/1024) * 2^(e-15) */
    }
    return sign ? -v : v;
}

static float bf16_bits_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* Round a non-negative finite float to the nearest multiple of the power of
 * two `quantum`, ties to an even multiple.  a / quantum and the product back
 * are exact (scaling by a power of two inside the float range). */
static float round_to_quantum(float a, float quantum) {
    float m = a / quantum;
    float r = rintf(m);       /* default rounding mode: nearest, ties to even */
    return r * quantum;
}

static uint16_t f32_to_f16_bits(float x) {
    uint32_t u;
    memcpy(&u, &x, 4);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000);
    float a = fabsf(x);
    if (isnan(x)) return (uint16_t)(sign | 0x7E00);
    if (isinf(x)) return (uint16_t)(sign | 0x7C00);
    /* spacing of binary16 numbers around a: 2^-24 below 2^-14 (subnormals),
     * else 2^(e-10) where 2^e <= a < 2^(e+1) */
    float quantum;
    if (a < ldexpf(1.0f, -14)) {
        quantum = ldexpf(1.0f, -24);
    } else {
        int e;
        frexpf(a, &e);                    /* a = f * 2^e with 0.5 <= f < 1 */
        quantum = ldexpf(1.0f, (e - 1) - 10);
    }
    float r = round_to_quantum(a, quantum);
    if (r >= 65536.0f) return (uint16_t)(sign | 0x7C00);     /* overflow */
    if (r < ldexpf(1.0f, -14)) {
        /* subnormal (or the first normal, 2^-14 = 1024 * 2^-24, which encodes
         * as 0x400 by the same formula) */
        return (uint16_t)(sign | (uint16_t)(r / ldexpf(1.0f, -24)));
    }
    int e;
    float f = frexpf(r, &e);              /* r = f * 2^e, f in [0.5, 1) */
    int mant = (int)(f * 2048.0f) - 1024; /* 11 significant bits */
    int bexp = (e - 1) + 15;
    return (uint16_t)(sign | (uint16_t)(bexp << 10) | (uint16_t)mant);
}

static uint16_t f32_to_bf16_bits(float x) {
    uint32_t u;
    memcpy(&u, &x, 4);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000);
    if (isnan(x)) return (uint16_t)(sign | 0x7FC0);
    if (isinf(x)) return (uint16_t)(sign | 0x7F80);
    float a = fabsf(x);
    /* bfloat16 keeps 8 significant bits and binary32's exponent range:
     * spacing 2^(e-7) for normal a, 2^-133 among binary32 subnormals */
    float quantum;
    if (a < ldexpf(1.0f, -126)) {
        quantum = ldexpf(1.0f, -133);
    } else {
        int e;
        frexpf(a, &e);
        quantum = ldexpf(1.0f, (e - 1) - 7);
    }
    float r = round_to_quantum(a, quantum);   /* overflows to +inf past the top */
    uint32_t ru;
    memcpy(&ru, &r, 4);
    return (uint16_t)(sign | (uint16_t)(ru >> 16));
}

void zpq_ref_f16_to_f32(const uint16_t* h, int64_t n, float* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = f16_bits_to_f32(h[i]);
}
void zpq_ref_bf16_to_f32(const uint16_t* b, int64_t n, float* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = bf16_bits_to_f32(b[i]);
}
void zpq_ref_f32_to_f16(const float* x, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = f32_to_f16_bits(x[i]);
}
void zpq_ref_f32_to_bf16(const float* x, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16_bits(x[i]);
}

/* ------------------------------------------------------------------------ */
/* O2-O4: symmetric block quantizer.  Blocks are the contiguous runs
 * [b*block, (b+1)*block); the summary page's "Approach" and the surprising
 * finding about non-blocked INT8 weights are why the scale is per block.   */
int zpq_ref_block_quant(const float* x, int64_t n, int32_t block, int32_t qmax,
                        int8_t* codes, float* scales) {
    if (n < 0 || block <= 0 || n % block != 0 || qmax <= 0 || qmax > 127)
        return REF_ERR_ARG;
    for (int64_t i = 0; i < n; ++i)
        if (!isfinite(x[i])) return REF_ERR_NONFINITE;
    const float fq = (float)qmax;
    for (int64_t b = 0; b < n / block; ++b) {
        const float* xb = x + b * block;
        /* O2: absmax of the block */
        float a = 0.0f;
        for (int32_t i = 0; i < block; ++i) {
            float v = fabsf(xb[i]);
            if (v > a) a = v;
        }
        /* O3: scale */
        float s = a / fq;
        scales[b] = s;
        /* O4: codes */
        for (int32_t i = 0; i < block; ++i) {
            int8_t q = 0;
            if (s != 0.0f) {
                float t = xb[i] / s;
                float r = rintf(t);           /* round half to even */
                if (r > fq) r = fq;
                if (r < -fq) r = -fq;
                q = (int8_t)r;
            }
            codes[b * block + i] = q;
        }
    }
    return REF_OK;
}

/* O6: dequantize, d = fl32(q * s), one multiplication per element. */
int zpq_ref_block_dequant(const int8_t* codes, const float* scales, int64_t n,
                          int32_t block, float* out) {
    if (n < 0 || block <= 0 || n % block != 0) return REF_ERR_ARG;
    for (int64_t i = 0; i < n; ++i) {
        float s = scales[i / block];
        out[i] = (float)codes[i] * s;
    }
    return REF_OK;
}

/* O5: INT4 packing: byte k = (q[2k] & 0xF) | (q[2k+1] & 0xF) << 4. */
int zpq_ref_pack_i4(const int8_t* codes, int64_t n, uint8_t* packed) {
    if (n < 0 || n % 2 != 0) return REF_ERR_ARG;
    for (int64_t k = 0; k < n / 2; ++k) {
        uint8_t lo = (uint8_t)(codes[2 * k] & 0x0F);
        uint8_t hi = (uint8_t)(codes[2 * k + 1] & 0x0F);
        packed[k] = (uint8_t)(lo | (hi << 4));
    }
    return REF_OK;
}

static int8_t nibble_to_int(uint8_t v) {
    return (int8_t)(v >= 8 ? (int)v - 16 : (int)v);   /* two's complement */
}

int zpq_ref_unpack_i4(const uint8_t* packed, int64_t n, int8_t* codes) {
    if (n < 0 || n % 2 != 0) return REF_ERR_ARG;
    for (int64_t k = 0; k < n / 2; ++k) {
        codes[2 * k] = nibble_to_int(packed[k] & 0x0F);
        codes[2 * k + 1] = nibble_to_int((uint8_t)(packed[k] >> 4));
    }
    return REF_OK;
}

/* ------------------------------------------------------------------------ */
/* O7: tensor slice reordering before the first all-to-all (summary page,
 * "Approach": reordering so that every slice ends at the right rank).
 * W = L*N ranks, rank r = node*L + local, rank r owns flat slice r of size
 * S = n/W.  Hop 1 sends contiguous chunk j (N slices) to local rank j of the
 * node; hop 2 sends position m of that chunk to node m.  For slice s to end
 * at rank s, send position p = j*N + m must carry slice s = m*L + j. */
int zpq_ref_reorder(const void* src, int64_t elem_bytes, int64_t n, int32_t L,
                    int32_t N, void* dst) {
    if (elem_bytes <= 0 || n < 0 || L < 1 || N < 1) return REF_ERR_ARG;
    int64_t W = (int64_t)L * N;
    if (n % W != 0) return REF_ERR_ARG;
    int64_t S = n / W;
    const unsigned char* s8 = (const unsigned char*)src;
    unsigned char* d8 = (unsigned char*)dst;
    for (int32_t j = 0; j < L; ++j) {
        for (int32_t m = 0; m < N; ++m) {
            int64_t p = (int64_t)j * N + m;     /* send position */
            int64_t s = (int64_t)m * L + j;     /* slice it carries */
            memcpy(d8 + p * S * elem_bytes, s8 + s * S * elem_bytes,
                   (size_t)(S * elem_bytes));
        }
    }
    return REF_OK;
}

/* O8: one step of the reduction, acc = fl32(acc + d), element by element.
 * Called once per source, in source-rank order. */
void zpq_ref_reduce_add(float* acc, const float* d, int64_t n) {
    for (int64_t i = 0; i < n; ++i) acc[i] = acc[i] + d[i];
}

/* O9: averaging at the last hop: y = fl32(acc / divisor), IEEE division. */
void zpq_ref_average(const float* acc, int64_t n, float divisor, float* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = acc[i] / divisor;
}

/* ------------------------------------------------------------------------ */
/* Compositions mirroring the four libzpq entry points.                     */

static int widen(const void* x, int dtype, int64_t n, float* out) {
    if (dtype == REF_F32) {
        memcpy(out, x, (size_t)n * 4);
    } else if (dtype == REF_F16) {
        zpq_ref_f16_to_f32((const uint16_t*)x, n, out);
    } else if (dtype == REF_BF16) {
        zpq_ref_bf16_to_f32((const uint16_t*)x, n, out);
    } else {
        return REF_ERR_ARG;
    }
    return REF_OK;
}

static int narrow(const float* v, int64_t n, void* y, int dtype) {
    if (dtype == REF_F32) {
        memcpy(y, v, (size_t)n * 4);
    } else if (dtype == REF_F16) {
        zpq_ref_f32_to_f16(v, n, (uint16_t*)y);
    } else if (dtype == REF_BF16) {
        zpq_ref_f32_to_bf16(v, n, (uint16_t*)y);
    } else {
        return REF_ERR_ARG;
    }
    return REF_OK;
}

static int64_t dtype_bytes(int dtype) {
    return dtype == REF_F32 ? 4 : (dtype == REF_F16 || dtype == REF_BF16) ? 2 : 0;
}

/* qwZ, before the all-gather: widen, then INT8 block quantize. */
int zpq_ref_quant_i8(const void* x, int dtype, int64_t n, int32_t block,
                     int8_t* codes, float* scales) {
    if (dtype_bytes(dtype) == 0 || n < 0) return REF_ERR_ARG;
    float* xf = (float*)malloc((size_t)(n > 0 ? n : 1) * 4);
    if (!xf) return REF_ERR_NOMEM;
    int rc = widen(x, dtype, n, xf);
    if (rc == REF_OK) rc = zpq_ref_block_quant(xf, n, block, 127, codes, scales);
    free(xf);
    return rc;
}

/* qwZ, after the all-gather: INT8 dequantize, then round to the output type. */
int zpq_ref_dequant_i8(const int8_t* codes, const float* scales, int64_t n,
                       int32_t block, void* y, int dtype) {
    if (dtype_bytes(dtype) == 0 || n < 0) return REF_ERR_ARG;
    float* d = (float*)malloc((size_t)(n > 0 ? n : 1) * 4);
    if (!d) return REF_ERR_NOMEM;
    int rc = zpq_ref_block_dequant(codes, scales, n, block, d);
    if (rc == REF_OK) rc = narrow(d, n, y, dtype);
    free(d);
    return rc;
}

/* qgZ, before hop 1: slice reorder, widen, INT4 block quantize, pack. */
int zpq_ref_qgz_reorder_quant_i4(const void* g, int dtype, int64_t n, int32_t L,
                                 int32_t N, int32_t block, uint8_t* codes,
                                 float* scales) {
    int64_t eb = dtype_bytes(dtype);
    if (eb == 0 || n < 0 || L < 1 || N < 1 || block <= 0) return REF_ERR_ARG;
    if (n % ((int64_t)L * N * block) != 0 || block % 2 != 0) return REF_ERR_ARG;
    size_t cnt = (size_t)(n > 0 ? n : 1);
    void* ro = malloc(cnt * (size_t)eb);
    float* xf = (float*)malloc(cnt * 4);
    int8_t* q = (int8_t*)malloc(cnt);
    int rc = (ro && xf && q) ? REF_OK : REF_ERR_NOMEM;
    if (rc == REF_OK) rc = zpq_ref_reorder(g, eb, n, L, N, ro);
    if (rc == REF_OK) rc = widen(ro, dtype, n, xf);
    if (rc == REF_OK) rc = zpq_ref_block_quant(xf, n, block, 7, q, scales);
    if (rc == REF_OK) rc = zpq_ref_pack_i4(q, n, codes);
    free(ro);
    free(xf);
    free(q);
    return rc;
}

/* qgZ, after each hop: for each of the K received chunks in source order,
 * unpack and dequantize it and add it into the fp32 accumulator; then either
 * requantize the sum to INT4 (hop 1, the result is the hop-2 send buffer) or
 * divide by the world size and round to the output type (hop 2).
 * Inputs: in_codes [K][chunk/2] bytes, in_scales [K][chunk/block].
 * Exactly one output mode: (out_codes, out_scales) or out_vals. */
int zpq_ref_qgz_dequant_reduce_requant_i4(const uint8_t* in_codes,
                                          const float* in_scales, int32_t K,
                                          int64_t chunk, int32_t block,
                                          uint8_t* out_codes, float* out_scales,
                                          void* out_vals, int out_dtype,
                                          float divisor) {
    if (K < 1 || chunk < 0 || block <= 0 || chunk % block != 0 || block % 2 != 0)
        return REF_ERR_ARG;
    int mode_i4 = (out_codes != NULL && out_scales != NULL && out_vals == NULL);
    int mode_fl = (out_codes == NULL && out_scales == NULL && out_vals != NULL);
    if (mode_i4 == mode_fl) return REF_ERR_ARG;
    if (mode_fl && dtype_bytes(out_dtype) == 0) return REF_ERR_ARG;
    size_t cnt = (size_t)(chunk > 0 ? chunk : 1);
    float* acc = (float*)malloc(cnt * 4);
    float* d = (float*)malloc(cnt * 4);
    int8_t* q = (int8_t*)malloc(cnt);
    int rc = (acc && d && q) ? REF_OK : REF_ERR_NOMEM;
    if (rc == REF_OK) {
        for (int64_t e = 0; e < chunk; ++e) acc[e] = 0.0f;    /* +0 */
        for (int32_t i = 0; i < K && rc == REF_OK; ++i) {
            rc = zpq_ref_unpack_i4(in_codes + (int64_t)i * (chunk / 2), chunk, q);
            if (rc == REF_OK)
                rc = zpq_ref_block_dequant(q, in_scales + (int64_t)i * (chunk / block),
                                           chunk, block, d);
            if (rc == REF_OK) zpq_ref_reduce_add(acc, d, chunk);
        }
    }
    if (rc == REF_OK && mode_i4) {
        rc = zpq_ref_block_quant(acc, chunk, block, 7, q, out_scales);
        if (rc == REF_OK) rc = zpq_ref_pack_i4(q, chunk, out_codes);
    } else if (rc == REF_OK) {
        zpq_ref_average(acc, chunk, divisor, d);
        rc = narrow(d, chunk, out_vals, out_dtype);
    }
    free(acc);
    free(d);
    free(q);
    return rc;
}
