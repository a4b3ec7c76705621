/*
 * libzpq from plain C: the five entry points through include/zpq.h and the
 * HIP runtime's C API only (no Python, no torch), on one GPU, compared byte
 * for byte with the CPU oracle's C functions.  Test infrastructure.
 *
 * Inputs are finite fp16 values from a SplitMix64 counter (magnitudes
 * 2^-14 .. 2^6, both signs).  Prints "c_api_check: ok" and exits 0, or
 * names the first failing check and exits 1.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "zpq.h"

/* the oracle (oracle/zpq_ref.c), element types numbered as in zpq.h */
int zpq_ref_quant_i8(const void* x, int dtype, int64_t n, int32_t block, int8_t* codes,
                     float* scales);
int zpq_ref_dequant_i8(const int8_t* codes, const float* scales, int64_t n, int32_t block,
                       void* y, int dtype);
int zpq_ref_qgz_reorder_quant_i4(const void* g, int dtype, int64_t n, int32_t L, int32_t N,
                                 int32_t block, uint8_t* codes, float* scales);
int zpq_ref_qgz_dequant_reduce_requant_i4(const uint8_t* in_codes, const float* in_scales,
                                          int32_t K, int64_t chunk, int32_t block,
                                          uint8_t* out_codes, float* out_scales, void* out_vals,
                                          int out_dtype, float divisor);

static uint64_t splitmix64(uint64_t x) {
    x += 0x9E3779B97F4A7C15ull;
    x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
    x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
    return x ^ (x >> 31);
}

#define HIP_OK(call)                                                              \
    do {                                                                          \
        hipError_t e_ = (call);                                                   \
        if (e_ != hipSuccess) {                                                   \
            printf("c_api_check: %s failed: %s\n", #call, hipGetErrorString(e_)); \
            exit(1);                                                              \
        }                                                                         \
    } while (0)

static int failed = 0;

static void check_status(zpq_status st, const char* what) {
    if (st != ZPQ_OK) {
        printf("c_api_check: %s returned %d (%s)\n", what, (int)st, zpq_status_str(st));
        failed = 1;
    }
}

static void compare(const void* dev, const void* want, size_t bytes, const char* what) {
    unsigned char* got = (unsigned char*)malloc(bytes);
    HIP_OK(hipMemcpy(got, dev, bytes, hipMemcpyDeviceToHost));
    for (size_t i = 0; i < bytes; ++i) {
        if (got[i] != ((const unsigned char*)want)[i]) {
            printf("c_api_check: %s differs from the oracle at byte %zu\n", what, i);
            failed = 1;
            break;
        }
    }
    free(got);
}

static void* dalloc(size_t bytes) {
    void* p = NULL;
    HIP_OK(hipMalloc(&p, bytes));
    return p;
}

int main(void) {
    const int32_t L = 2, N = 3, B8 = 256, B4 = 64;
    const int64_t n = 150 * 256;                  /* a multiple of 256 and of L*N*64 */
    const int64_t chunk = n / L, slice = n / (L * N);

    uint16_t* x = (uint16_t*)malloc(n * 2);
    for (int64_t i = 0; i < n; ++i) {
        uint64_t r = splitmix64(0x5EEDull * 1000003ull + (uint64_t)i);
        uint16_t e = (uint16_t)(1 + r % 20), m = (uint16_t)((r >> 8) & 0x3FF);
        x[i] = (uint16_t)(((r >> 20) & 1) << 15 | e << 10 | m);
    }
    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));
    void* dx = dalloc(n * 2);
    HIP_OK(hipMemcpy(dx, x, n * 2, hipMemcpyHostToDevice));

    /* qwZ: quantize, dequantize */
    int8_t* rc8 = (int8_t*)malloc(n);
    float* rs8 = (float*)malloc((n / B8) * 4);
    uint16_t* ry8 = (uint16_t*)malloc(n * 2);
    if (zpq_ref_quant_i8(x, ZPQ_F16, n, B8, rc8, rs8) || zpq_ref_dequant_i8(rc8, rs8, n, B8, ry8, ZPQ_F16)) {
        printf("c_api_check: oracle failed\n");
        return 1;
    }
    int8_t* dc8 = (int8_t*)dalloc(n);
    float* ds8 = (float*)dalloc((n / B8) * 4);
    void* dy8 = dalloc(n * 2);
    check_status(zpq_quant_i8(dx, ZPQ_F16, n, B8, dc8, ds8, stream), "zpq_quant_i8");
    check_status(zpq_dequant_i8(dc8, ds8, n, B8, dy8, ZPQ_F16, stream), "zpq_dequant_i8");
    HIP_OK(hipStreamSynchronize(stream));
    compare(dc8, rc8, n, "INT8 codes");
    compare(ds8, rs8, (n / B8) * 4, "INT8 scales");
    compare(dy8, ry8, n * 2, "dequantized values");

    /* per-tensor INT8 */
    float rst;
    if (zpq_ref_quant_i8(x, ZPQ_F16, n, (int32_t)n, rc8, &rst)) return 1;
    float* dst = (float*)dalloc(16);
    check_status(zpq_quant_i8_tensor(dx, ZPQ_F16, n, dc8, dst, stream), "zpq_quant_i8_tensor");
    HIP_OK(hipStreamSynchronize(stream));
    compare(dc8, rc8, n, "per-tensor codes");
    compare(dst, &rst, 4, "per-tensor scale");

    /* qgZ: reorder + INT4, hop 1 (own send chunks as the L received ones), hop 2 */
    uint8_t* rc4 = (uint8_t*)malloc(n / 2);
    float* rs4 = (float*)malloc((n / B4) * 4);
    uint8_t* rc5 = (uint8_t*)malloc(chunk / 2);
    float* rs5 = (float*)malloc((chunk / B4) * 4);
    float* ry6 = (float*)malloc(slice * 4);
    if (zpq_ref_qgz_reorder_quant_i4(x, ZPQ_F16, n, L, N, B4, rc4, rs4) ||
        zpq_ref_qgz_dequant_reduce_requant_i4(rc4, rs4, L, chunk, B4, rc5, rs5, NULL, 0, 1.0f) ||
        zpq_ref_qgz_dequant_reduce_requant_i4(rc5, rs5, N, slice, B4, NULL, NULL, ry6, ZPQ_F32,
                                              (float)(L * N))) {
        printf("c_api_check: oracle failed\n");
        return 1;
    }
    uint8_t* dc4 = (uint8_t*)dalloc(n / 2);
    float* ds4 = (float*)dalloc((n / B4) * 4);
    uint8_t* dc5 = (uint8_t*)dalloc(chunk / 2);
    float* ds5 = (float*)dalloc((chunk / B4) * 4);
    float* dy6 = (float*)dalloc(slice * 4);
    check_status(zpq_qgz_reorder_quant_i4(dx, ZPQ_F16, n, L, N, B4, dc4, ds4, stream),
                 "zpq_qgz_reorder_quant_i4");
    check_status(zpq_qgz_dequant_reduce_requant_i4(dc4, ds4, L, chunk, B4, dc5, ds5, NULL, 0,
                                                   1.0f, stream), "hop 1");
    check_status(zpq_qgz_dequant_reduce_requant_i4(dc5, ds5, N, slice, B4, NULL, NULL, dy6,
                                                   ZPQ_F32, (float)(L * N), stream), "hop 2");
    HIP_OK(hipStreamSynchronize(stream));
    compare(dc4, rc4, n / 2, "INT4 send codes");
    compare(ds4, rs4, (n / B4) * 4, "INT4 send scales");
    compare(dc5, rc5, chunk / 2, "hop-1 codes");
    compare(ds5, rs5, (chunk / B4) * 4, "hop-1 scales");
    compare(dy6, ry6, slice * 4, "hop-2 averages");

    /* an invalid argument is refused on the host, nothing launched */
    if (zpq_quant_i8(dx, ZPQ_F16, n, 100, dc8, ds8, stream) != ZPQ_ERR_BLOCK) {
        printf("c_api_check: block 100 was not refused\n");
        failed = 1;
    }
    if (zpq_abi_version() != ZPQ_ABI_VERSION) {
        printf("c_api_check: ABI version mismatch\n");
        failed = 1;
    }
    HIP_OK(hipStreamDestroy(stream));
    if (!failed) printf("c_api_check: ok\n");
    return failed;
}
