// zpq.hip -- libzpq: ZeRO++ block-quantized communication kernels for gfx950.
//
// Four kernels on the data-parallel path of ZeRO++ (arXiv 2306.10209):
//   qwZ  quantize  (zpq_quant_i8)   INT8 block quantization of a weight shard
//                                   before the forward all-gather
//   qwZ  dequant   (zpq_dequant_i8) the gathered INT8 buffer back to fp16/bf16
//   qgZ  hop send  (zpq_qgz_reorder_quant_i4) tensor-slice reordering fused
//                                   with INT4 block quantization
//   qgZ  hop recv  (zpq_qgz_dequant_reduce_requant_i4) dequantize the chunks
//                                   received in one all-to-all hop, reduce
//                                   them in fp32 in source order, then INT4
//                                   requantize (hop 1) or average (hop 2)
// (ZeRO++ summary page, atlas.scime.ai, "Approach"; mlsanity.com index page,
// "Abstract (arXiv)"; LIT-102 anthology record, "Key takeaways".)
//
// Every kernel streams HBM once: 128-bit loads, one quantization block per
// aligned group of BLOCK/EPL lanes of a wave64 (EPL = elements per lane),
// the block absmax reduced with DPP lane permutes, the division done as a
// correctly rounded multiply-and-correct sequence, codes packed in registers
// and written with 64/128-bit stores.  No LDS and no MFMA: the work is an
// elementwise map with a segmented reduction, bound by HBM bandwidth (and,
// for the hop-receive kernel, by VALU issue).
//
// Bit-exactness: every result equals the plain definition (IEEE binary32
// operations rounded to nearest even, division included) for all finite
// inputs.  Denormals are kept (the gfx950 default f32/f16 denormal mode).

#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>
#include <hip/hip_fp16.h>
#include <stdint.h>
#include <string.h>

#include "zpq.h"

namespace {

constexpr int kThreads = 256;          // 4 waves of 64 per workgroup

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Cross-lane maximum over aligned groups of G lanes (G = 1, 2, 4, ..., 32).
// Values are bit patterns of non-negative floats, which order like unsigned
// integers, so v_max_u32 with a DPP source operand does one step per lane
// permute: quad_perm swaps within 2 and 4 lanes, row_half_mirror within 8,
// row_mirror within 16, ds_swizzle (lane ^ 16) within 32.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

template <int G>
__device__ __forceinline__ uint32_t group_max(uint32_t v) {
    static_assert(G >= 1 && G <= 32 && (G & (G - 1)) == 0, "group of 1..32 lanes");
    if constexpr (G >= 2) v = max(v, dpp<0xB1>(v));     // quad_perm [1,0,3,2]
    if constexpr (G >= 4) v = max(v, dpp<0x4E>(v));     // quad_perm [2,3,0,1]
    if constexpr (G >= 8) v = max(v, dpp<0x141>(v));    // row_half_mirror
    if constexpr (G >= 16) v = max(v, dpp<0x140>(v));   // row_mirror
    if constexpr (G >= 32)
        v = max(v, (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F));  // xor 16
    return v;
}

// ---------------------------------------------------------------------------
// Correctly rounded division fl32(x / s), given r = fl32(1 / s).
// q0 = x*r is within 1.5 ulp of x/s; one residual step (the residual
// x - q*s is exact in an FMA) brings it within 1 ulp; a second step then
// returns the correctly rounded quotient (Markstein's theorem, see Muller et
// al., Handbook of Floating-Point Arithmetic, division with an FMA).
// Preconditions, checked by the callers: 2^-100 <= s (so 1/s is finite and
// no residual underflows while |x/s| >= 1/4; smaller quotients only need to
// stay below 1/2, which they do) and s <= 2^126.
__device__ __forceinline__ float div_cr(float x, float s, float r) {
    float q = x * r;
    float e = __builtin_fmaf(-q, s, x);
    q = __builtin_fmaf(e, r, q);
    e = __builtin_fmaf(-q, s, x);
    return __builtin_fmaf(e, r, q);
}

// Round-half-even to integer and clamp to [-QMAX, QMAX]; the integer lands in
// the low bits of the returned bit pattern (1.5 * 2^23 + k), so its low byte
// is the two's-complement INT8 code and its low nibble the INT4 code.
template <int QMAX>
__device__ __forceinline__ uint32_t round_code(float t) {
    t = __builtin_amdgcn_fmed3f(t, -(float)QMAX, (float)QMAX);
    return __float_as_uint(t + 12582912.0f);
}

// Per-block quantizer state: scale s = fl32(a / QMAX) (IEEE division) and,
// when s >= 2^-100, its correctly rounded reciprocal for div_cr.
template <int QMAX>
struct BlockScale {
    float s, r;
    bool fast;
    __device__ __forceinline__ explicit BlockScale(float a) {
        s = a / (float)QMAX;
        fast = s >= 0x1p-100f;
        r = fast ? 1.0f / s : 0.0f;
    }
    // Codes of N values (in place into bit patterns).  The slow path (tiny
    // or zero scale, block-uniform) divides with the IEEE operator.
    template <int N>
    __device__ __forceinline__ void codes(const float (&v)[N], uint32_t (&out)[N]) const {
        if (fast) {
#pragma unroll
            for (int k = 0; k < N; ++k) out[k] = round_code<QMAX>(div_cr(v[k], s, r));
        } else {
#pragma unroll
            for (int k = 0; k < N; ++k) out[k] = round_code<QMAX>(s != 0.0f ? v[k] / s : 0.0f);
        }
    }
};

// ---------------------------------------------------------------------------
// Byte packing with v_perm_b32.  perm(a, b, sel): selector byte 0..3 picks a
// byte of b, 4..7 a byte of a, 0x0C gives 0x00.
__device__ __forceinline__ uint32_t pack_low_bytes(uint32_t b0, uint32_t b1, uint32_t b2,
                                                   uint32_t b3) {
    uint32_t lo = __builtin_amdgcn_perm(b1, b0, 0x0C0C0400u);
    uint32_t hi = __builtin_amdgcn_perm(b3, b2, 0x0C0C0400u);
    return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

// 8 codes -> one dword of nibbles, element 2k in the low nibble of byte k.
__device__ __forceinline__ uint32_t pack_nibbles(const uint32_t* c) {
    uint32_t even = pack_low_bytes(c[0], c[2], c[4], c[6]);
    uint32_t odd = pack_low_bytes(c[1], c[3], c[5], c[7]);
    return (even & 0x0F0F0F0Fu) | ((odd << 4) & 0xF0F0F0F0u);
}

// EPL/8 dwords of packed nibbles (EPL/2 bytes) to a 8- or 16-byte aligned address.
template <int EPL>
__device__ __forceinline__ void store_nibbles(uint8_t* dst, const uint32_t* packed) {
    if constexpr (EPL == 16) {
        __builtin_nontemporal_store(u32x2{packed[0], packed[1]}, reinterpret_cast<u32x2*>(dst));
    } else {
        static_assert(EPL % 32 == 0, "16-byte stores");
#pragma unroll
        for (int k = 0; k < EPL / 32; ++k)
            __builtin_nontemporal_store(u32x4{packed[4 * k], packed[4 * k + 1], packed[4 * k + 2],
                                              packed[4 * k + 3]},
                                        reinterpret_cast<u32x4*>(dst) + k);
    }
}

// ---------------------------------------------------------------------------
// Input tiles: EPL consecutive elements of type DT held as raw 32-bit words.
template <int DT>
struct ElemBytes { static constexpr int v = DT == ZPQ_F32 ? 4 : 2; };

template <int DT, int EPL>
struct InTile {
    static constexpr int WORDS = EPL * ElemBytes<DT>::v / 4;
    static_assert(WORDS % 4 == 0, "whole 16-byte vectors");
    uint32_t w[WORDS];

    __device__ __forceinline__ void load(const void* base, int64_t elem) {
        const u32x4* p = reinterpret_cast<const u32x4*>(
            static_cast<const char*>(base) + elem * ElemBytes<DT>::v);
#pragma unroll
        for (int i = 0; i < WORDS / 4; ++i) {
            u32x4 t = __builtin_nontemporal_load(p + i);
            w[4 * i] = t.x; w[4 * i + 1] = t.y; w[4 * i + 2] = t.z; w[4 * i + 3] = t.w;
        }
    }
    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int i = 0; i < WORDS; ++i) w[i] = 0;
    }
    __device__ __forceinline__ float get(int k) const {
        if constexpr (DT == ZPQ_F32) {
            return __uint_as_float(w[k]);
        } else if constexpr (DT == ZPQ_F16) {
            uint32_t h = (k & 1) ? (w[k >> 1] >> 16) : (w[k >> 1] & 0xFFFFu);
            return __half2float(__ushort_as_half((unsigned short)h));
        } else {
            return __uint_as_float((k & 1) ? (w[k >> 1] & 0xFFFF0000u) : (w[k >> 1] << 16));
        }
    }
    // bit pattern of max |x| over the tile, as fp32
    __device__ __forceinline__ uint32_t absmax_bits() const {
        if constexpr (DT == ZPQ_F32) {
            uint32_t m = 0;
#pragma unroll
            for (int i = 0; i < WORDS; ++i) m = max(m, w[i] & 0x7FFFFFFFu);
            return m;
        } else {
            // |x| of fp16 and bf16 values orders like its 16-bit pattern:
            // two elements per v_pk_max_u16
            u16x2 m = {0, 0};
#pragma unroll
            for (int i = 0; i < WORDS; ++i) {
                uint32_t a = w[i] & 0x7FFF7FFFu;
                u16x2 v = {(unsigned short)(a & 0xFFFFu), (unsigned short)(a >> 16)};
                m = __builtin_elementwise_max(m, v);
            }
            unsigned short h = m.x > m.y ? m.x : m.y;
            if constexpr (DT == ZPQ_F16)
                return __float_as_uint(__half2float(__ushort_as_half(h)));
            else
                return (uint32_t)h << 16;
        }
    }
};

// ---------------------------------------------------------------------------
// K1: qwZ INT8 block quantize.
// Workgroup covers U * 256 * EPL consecutive elements; its thread t handles
// EPL elements at base + u * 256 * EPL + t * EPL for u < U.
template <int DT, int BLOCK, int EPL, int U>
__global__ __launch_bounds__(kThreads) void k_quant_i8(const void* __restrict__ x, int64_t n,
                                                       int8_t* __restrict__ codes,
                                                       float* __restrict__ scales) {
    constexpr int G = BLOCK / EPL;
    const int64_t wg_base = (int64_t)blockIdx.x * (U * kThreads * EPL);
    InTile<DT, EPL> tile[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t e = wg_base + (int64_t)u * (kThreads * EPL) + threadIdx.x * EPL;
        if (e < n) tile[u].load(x, e); else tile[u].zero();
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t e = wg_base + (int64_t)u * (kThreads * EPL) + threadIdx.x * EPL;
        const float a = __uint_as_float(group_max<G>(tile[u].absmax_bits()));
        BlockScale<127> bs(a);
        float v[EPL];
#pragma unroll
        for (int k = 0; k < EPL; ++k) v[k] = tile[u].get(k);
        uint32_t q[EPL];
        bs.codes(v, q);
        if (e < n) {
            uint32_t packed[EPL / 4];
#pragma unroll
            for (int k = 0; k < EPL / 4; ++k)
                packed[k] = pack_low_bytes(q[4 * k], q[4 * k + 1], q[4 * k + 2], q[4 * k + 3]);
            u32x4* dst = reinterpret_cast<u32x4*>(codes + e);
#pragma unroll
            for (int k = 0; k < EPL / 16; ++k)
                __builtin_nontemporal_store(u32x4{packed[4 * k], packed[4 * k + 1],
                                                  packed[4 * k + 2], packed[4 * k + 3]}, dst + k);
            if ((threadIdx.x & (G - 1)) == 0) scales[e / BLOCK] = bs.s;
        }
    }
}

// ---------------------------------------------------------------------------
// K2: qwZ INT8 dequantize into fp32 / fp16 / bf16.
template <int OT, int EPL>
__device__ __forceinline__ void store_out(void* __restrict__ y, int64_t e, const float (&v)[EPL]) {
    if constexpr (OT == ZPQ_F32) {
        u32x4* dst = reinterpret_cast<u32x4*>(static_cast<float*>(y) + e);
#pragma unroll
        for (int k = 0; k < EPL / 4; ++k)
            __builtin_nontemporal_store(
                u32x4{__float_as_uint(v[4 * k]), __float_as_uint(v[4 * k + 1]),
                      __float_as_uint(v[4 * k + 2]), __float_as_uint(v[4 * k + 3])},
                dst + k);
    } else {
        uint32_t h[EPL / 2];
#pragma unroll
        for (int k = 0; k < EPL / 2; ++k) {
            // The fp32 value must be rounded to fp32 first and then to the
            // 16-bit type.  The empty asm keeps the compiler from fusing the
            // producing multiply into a mixed-precision FMA (v_fma_mixlo_f16
            // with a +0 addend), which rounds once and loses the sign of zero.
            float a = v[2 * k], b = v[2 * k + 1];
            asm("" : "+v"(a), "+v"(b));
            uint32_t lo, hi;
            if constexpr (OT == ZPQ_F16) {
                lo = __half_as_ushort(__float2half_rn(a));
                hi = __half_as_ushort(__float2half_rn(b));
            } else {
                lo = __bfloat16_as_ushort(__float2bfloat16(a));
                hi = __bfloat16_as_ushort(__float2bfloat16(b));
            }
            h[k] = lo | (hi << 16);
        }
        u32x4* dst = reinterpret_cast<u32x4*>(static_cast<uint16_t*>(y) + e);
#pragma unroll
        for (int k = 0; k < EPL / 8; ++k)
            __builtin_nontemporal_store(u32x4{h[4 * k], h[4 * k + 1], h[4 * k + 2], h[4 * k + 3]},
                                        dst + k);
    }
}

template <int OT, int BLOCK, int EPL, int U>
__global__ __launch_bounds__(kThreads) void k_dequant_i8(const int8_t* __restrict__ codes,
                                                         const float* __restrict__ scales,
                                                         int64_t n, void* __restrict__ y) {
    static_assert(EPL == 16, "one 16-byte code vector per lane and tile");
    const int64_t wg_base = (int64_t)blockIdx.x * (U * kThreads * EPL);
    u32x4 cw[U];
    float s[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t e = wg_base + (int64_t)u * (kThreads * EPL) + threadIdx.x * EPL;
        if (e < n) {
            cw[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(codes + e));
            s[u] = scales[e / BLOCK];
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t e = wg_base + (int64_t)u * (kThreads * EPL) + threadIdx.x * EPL;
        if (e < n) {
            const uint32_t w[4] = {cw[u].x, cw[u].y, cw[u].z, cw[u].w};
            float v[EPL];
#pragma unroll
            for (int k = 0; k < EPL; ++k) {
                const int8_t q = (int8_t)(w[k >> 2] >> (8 * (k & 3)));
                v[k] = (float)q * s[u];
            }
            store_out<OT, EPL>(y, e, v);
        }
    }
}

// ---------------------------------------------------------------------------
// K3: qgZ slice reorder + INT4 block quantize.
// Send position p = j*N + m takes slice m*L + j.  Workgroups are laid out
// slice-major (wgs_per_slice per send position), so the source offset is a
// per-workgroup scalar and a tile never straddles two slices.
template <int DT, int BLOCK, int EPL, int U>
__global__ __launch_bounds__(kThreads) void k_reorder_quant_i4(
    const void* __restrict__ grad, int64_t S, int32_t L, int32_t N, uint32_t wgs_per_slice,
    uint8_t* __restrict__ codes, float* __restrict__ scales) {
    constexpr int G = BLOCK / EPL;
    const uint32_t p = blockIdx.x / wgs_per_slice;
    const uint32_t w = blockIdx.x - p * wgs_per_slice;
    const uint32_t j = p / (uint32_t)N;
    const uint32_t m = p - j * (uint32_t)N;
    const int64_t src0 = ((int64_t)m * L + j) * S;      // first element of slice m*L + j
    const int64_t dst0 = (int64_t)p * S;                 // first element of send position p
    const int64_t f0 = (int64_t)w * (U * kThreads * EPL);
    InTile<DT, EPL> tile[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t f = f0 + (int64_t)u * (kThreads * EPL) + threadIdx.x * EPL;
        if (f < S) tile[u].load(grad, src0 + f); else tile[u].zero();
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t f = f0 + (int64_t)u * (kThreads * EPL) + threadIdx.x * EPL;
        const float a = __uint_as_float(group_max<G>(tile[u].absmax_bits()));
        BlockScale<7> bs(a);
        float v[EPL];
#pragma unroll
        for (int k = 0; k < EPL; ++k) v[k] = tile[u].get(k);
        uint32_t q[EPL];
        bs.codes(v, q);
        if (f < S) {
            const int64_t e = dst0 + f;
            uint32_t packed[EPL / 8];
#pragma unroll
            for (int k = 0; k < EPL / 8; ++k) packed[k] = pack_nibbles(q + 8 * k);
            store_nibbles<EPL>(codes + e / 2, packed);
            if ((threadIdx.x & (G - 1)) == 0) scales[e / BLOCK] = bs.s;
        }
    }
}

// ---------------------------------------------------------------------------
// K4: qgZ dequantize -> fp32 reduce in source order -> INT4 requant or average.
//
// Per source and element: d = fl32(q * s) computed as fma(u, s, -8s) with
// u = q + 8 in 0..15 (the nibble with its top bit flipped, converted by
// v_cvt_f32_ubyte): the FMA rounds the exact (u - 8) * s once, which is
// fl32(q * s).  -8s is exact unless 8|s| overflows; then that source's terms
// are -inf and the lane's sums end non-finite, which the lane checks once at
// the end and answers by recomputing with q * s directly (the recomputation
// is the definition itself, so it is also right when a true sum overflows).
// The sum is acc = fl32(acc + d), starting at +0, sources in order 0..K-1.
template <int EPL>
struct SrcCodes {
    static constexpr int W = EPL / 8;     // dwords of nibbles per lane and source
    uint32_t w[W];
    float s;
};

// Source base pointers are wave-uniform (SGPRs); per-lane offsets are 32-bit.
template <int EPL>
__device__ __forceinline__ void load_src(SrcCodes<EPL>& d, const uint8_t* cbase, uint32_t coff,
                                         const float* sbase, uint32_t soff) {
    if constexpr (EPL == 16) {
        u32x2 t = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(cbase + coff));
        d.w[0] = t.x; d.w[1] = t.y;
    } else {
#pragma unroll
        for (int i = 0; i < EPL / 32; ++i) {
            u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(cbase + coff) + i);
            d.w[4 * i] = t.x; d.w[4 * i + 1] = t.y; d.w[4 * i + 2] = t.z; d.w[4 * i + 3] = t.w;
        }
    }
    d.s = sbase[soff];
}

// Byte k of x as a float, one v_cvt_f32_ubyte{k}.  Written as asm so the
// compiler, which can see that each byte holds a nibble, does not replace it
// with a bit-field extract plus a byte-0 conversion (two instructions).
template <int K>
__device__ __forceinline__ float cvt_ubyte(uint32_t x) {
    float r;
    if constexpr (K == 0) asm("v_cvt_f32_ubyte0 %0, %1" : "=v"(r) : "v"(x));
    else if constexpr (K == 1) asm("v_cvt_f32_ubyte1 %0, %1" : "=v"(r) : "v"(x));
    else if constexpr (K == 2) asm("v_cvt_f32_ubyte2 %0, %1" : "=v"(r) : "v"(x));
    else asm("v_cvt_f32_ubyte3 %0, %1" : "=v"(r) : "v"(x));
    return r;
}

template <int EPL>
__device__ __forceinline__ void accumulate(float (&acc)[EPL], const SrcCodes<EPL>& d) {
    const float s = d.s;
    const float c = s * -8.0f;
#pragma unroll
    for (int i = 0; i < SrcCodes<EPL>::W; ++i) {
        const uint32_t b = d.w[i] ^ 0x88888888u;          // nibble q -> q + 8
        const uint32_t lo = b & 0x0F0F0F0Fu;               // byte k: element 8i + 2k
        const uint32_t hi = (b >> 4) & 0x0F0F0F0Fu;        // byte k: element 8i + 2k + 1
        float ul[4], uh[4];
        ul[0] = cvt_ubyte<0>(lo); uh[0] = cvt_ubyte<0>(hi);
        ul[1] = cvt_ubyte<1>(lo); uh[1] = cvt_ubyte<1>(hi);
        ul[2] = cvt_ubyte<2>(lo); uh[2] = cvt_ubyte<2>(hi);
        ul[3] = cvt_ubyte<3>(lo); uh[3] = cvt_ubyte<3>(hi);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            acc[8 * i + 2 * k] = acc[8 * i + 2 * k] + __builtin_fmaf(ul[k], s, c);
            acc[8 * i + 2 * k + 1] = acc[8 * i + 2 * k + 1] + __builtin_fmaf(uh[k], s, c);
        }
    }
}

template <int EPL>
__device__ __forceinline__ void accumulate_direct(float (&acc)[EPL], const SrcCodes<EPL>& d) {
#pragma unroll
    for (int i = 0; i < SrcCodes<EPL>::W; ++i) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int q = ((int)(d.w[i] << (28 - 4 * k))) >> 28;     // sign-extended nibble
            acc[8 * i + k] = acc[8 * i + k] + (float)q * d.s;
        }
    }
}

template <int BLOCK, int EPL, int OUT /* -1: INT4, else a zpq_dtype */, int PF>
__global__ __launch_bounds__(kThreads) void k_dequant_reduce(
    const uint8_t* __restrict__ in_codes, const float* __restrict__ in_scales, int32_t K,
    int64_t c, uint8_t* __restrict__ out_codes, float* __restrict__ out_scales,
    void* __restrict__ out_vals, float divisor, float rdiv, bool div_fast) {
    constexpr int G = BLOCK / EPL;
    const int64_t e = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * EPL;
    if (e >= c) return;            // whole quantization blocks leave together
    const int64_t cstride = c / 2, sstride = c / BLOCK;
    const uint32_t coff = (uint32_t)(e / 2), soff = (uint32_t)(e / BLOCK);   // c < 2^32

    float acc[EPL];
#pragma unroll
    for (int k = 0; k < EPL; ++k) acc[k] = 0.0f;

    // PF sources in flight: slot k holds source i0 + k
    SrcCodes<EPL> buf[PF];
#pragma unroll
    for (int k = 0; k < PF; ++k)
        if (k < K) load_src<EPL>(buf[k], in_codes + k * cstride, coff, in_scales + k * sstride, soff);
    for (int i0 = 0; i0 < K; i0 += PF) {
#pragma unroll
        for (int k = 0; k < PF; ++k) {
            const int i = i0 + k;
            if (i < K) {
                accumulate<EPL>(acc, buf[k]);
                const int nx = i + PF;
                if (nx < K)
                    load_src<EPL>(buf[k], in_codes + (int64_t)nx * cstride, coff,
                                  in_scales + (int64_t)nx * sstride, soff);
            }
        }
    }
    // |acc| as bit patterns: finite values order like unsigned integers and
    // every inf / NaN pattern lies above FLT_MAX's
    uint32_t mbits = 0;
#pragma unroll
    for (int k = 0; k < EPL; ++k) mbits = max(mbits, __float_as_uint(acc[k]) & 0x7FFFFFFFu);
    if (mbits > 0x7F7FFFFFu) {
        // a non-finite sum: redo this lane with q * s directly
#pragma unroll
        for (int k = 0; k < EPL; ++k) acc[k] = 0.0f;
        for (int i = 0; i < K; ++i) {
            SrcCodes<EPL> d;
            load_src<EPL>(d, in_codes + (int64_t)i * cstride, coff, in_scales + (int64_t)i * sstride,
                          soff);
            accumulate_direct<EPL>(acc, d);
        }
        mbits = 0;
#pragma unroll
        for (int k = 0; k < EPL; ++k) mbits = max(mbits, __float_as_uint(acc[k]) & 0x7FFFFFFFu);
    }

    if constexpr (OUT < 0) {
        const float a = __uint_as_float(group_max<G>(mbits));
        BlockScale<7> bs(a);
        uint32_t q[EPL];
        bs.codes(acc, q);
        uint32_t packed[EPL / 8];
#pragma unroll
        for (int k = 0; k < EPL / 8; ++k) packed[k] = pack_nibbles(q + 8 * k);
        store_nibbles<EPL>(out_codes + e / 2, packed);
        if ((threadIdx.x & (G - 1)) == 0) out_scales[e / BLOCK] = bs.s;
    } else {
        // y = fl32(acc / divisor): div_cr is exact when the divisor is in
        // [1, 2^40] (checked on the host: the quotient cannot overflow) and
        // |acc| >= 2^-60 or acc == 0 (the quotient is normal and no residual
        // underflows); otherwise the IEEE operator.
        bool fast = div_fast && mbits <= 0x7F7FFFFFu;
#pragma unroll
        for (int k = 0; k < EPL; ++k)
            fast = fast && (fabsf(acc[k]) >= 0x1p-60f || acc[k] == 0.0f);
        float y[EPL];
        if (fast) {
#pragma unroll
            for (int k = 0; k < EPL; ++k) y[k] = div_cr(acc[k], divisor, rdiv);
        } else {
#pragma unroll
            for (int k = 0; k < EPL; ++k) y[k] = acc[k] / divisor;
        }
        store_out<OUT, EPL>(out_vals, e, y);
    }
}

// ---------------------------------------------------------------------------
// Host side.

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline bool overlaps(const void* a, uint64_t na, const void* b, uint64_t nb) {
    if (na == 0 || nb == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + nb && b0 < a0 + na;
}

inline bool block_ok(int32_t b) {
    return b == 32 || b == 64 || b == 128 || b == 256 || b == 512;
}

inline int64_t dtype_bytes(int32_t t) {
    return t == ZPQ_F32 ? 4 : (t == ZPQ_F16 || t == ZPQ_BF16) ? 2 : 0;
}

inline zpq_status after_launch() {
    return hipGetLastError() == hipSuccess ? ZPQ_OK : ZPQ_ERR_LAUNCH;
}

inline unsigned grid_for(int64_t elems, int64_t per_wg) {
    return (unsigned)((elems + per_wg - 1) / per_wg);
}

// Launch shapes (elements per lane, tiles per lane, sources in flight).
constexpr int kEplQuant = 16, kUQuant = 2;
constexpr int kEplDequant = 16, kUDequant = 2;
constexpr int kEplQgz = 16, kUQgz = 2;
constexpr int kEplReduce = 16, kPfReduce = 4;

template <int BLOCK>
zpq_status launch_quant_i8(const void* x, int32_t dt, int64_t n, int8_t* codes, float* scales,
                           hipStream_t st) {
    const unsigned grid = grid_for(n, (int64_t)kUQuant * kThreads * kEplQuant);
    switch (dt) {
    case ZPQ_F32:
        hipLaunchKernelGGL((k_quant_i8<ZPQ_F32, BLOCK, kEplQuant, kUQuant>), dim3(grid),
                           dim3(kThreads), 0, st, x, n, codes, scales);
        break;
    case ZPQ_F16:
        hipLaunchKernelGGL((k_quant_i8<ZPQ_F16, BLOCK, kEplQuant, kUQuant>), dim3(grid),
                           dim3(kThreads), 0, st, x, n, codes, scales);
        break;
    default:
        hipLaunchKernelGGL((k_quant_i8<ZPQ_BF16, BLOCK, kEplQuant, kUQuant>), dim3(grid),
                           dim3(kThreads), 0, st, x, n, codes, scales);
        break;
    }
    return after_launch();
}

template <int BLOCK>
zpq_status launch_dequant_i8(const int8_t* codes, const float* scales, int64_t n, void* y,
                             int32_t dt, hipStream_t st) {
    const unsigned grid = grid_for(n, (int64_t)kUDequant * kThreads * kEplDequant);
    switch (dt) {
    case ZPQ_F32:
        hipLaunchKernelGGL((k_dequant_i8<ZPQ_F32, BLOCK, kEplDequant, kUDequant>), dim3(grid),
                           dim3(kThreads), 0, st, codes, scales, n, y);
        break;
    case ZPQ_F16:
        hipLaunchKernelGGL((k_dequant_i8<ZPQ_F16, BLOCK, kEplDequant, kUDequant>), dim3(grid),
                           dim3(kThreads), 0, st, codes, scales, n, y);
        break;
    default:
        hipLaunchKernelGGL((k_dequant_i8<ZPQ_BF16, BLOCK, kEplDequant, kUDequant>), dim3(grid),
                           dim3(kThreads), 0, st, codes, scales, n, y);
        break;
    }
    return after_launch();
}

template <int BLOCK>
zpq_status launch_qgz_quant(const void* g, int32_t dt, int64_t n, int32_t L, int32_t N,
                            uint8_t* codes, float* scales, hipStream_t st) {
    const int64_t W = (int64_t)L * N;
    const int64_t S = n / W;
    const int64_t per_wg = (int64_t)kUQgz * kThreads * kEplQgz;
    const int64_t wps = (S + per_wg - 1) / per_wg;
    if (wps * W > 0x7FFFFFFFLL) return ZPQ_ERR_SIZE;
    const unsigned grid = (unsigned)(wps * W);
    switch (dt) {
    case ZPQ_F32:
        hipLaunchKernelGGL((k_reorder_quant_i4<ZPQ_F32, BLOCK, kEplQgz, kUQgz>), dim3(grid),
                           dim3(kThreads), 0, st, g, S, L, N, (uint32_t)wps, codes, scales);
        break;
    case ZPQ_F16:
        hipLaunchKernelGGL((k_reorder_quant_i4<ZPQ_F16, BLOCK, kEplQgz, kUQgz>), dim3(grid),
                           dim3(kThreads), 0, st, g, S, L, N, (uint32_t)wps, codes, scales);
        break;
    default:
        hipLaunchKernelGGL((k_reorder_quant_i4<ZPQ_BF16, BLOCK, kEplQgz, kUQgz>), dim3(grid),
                           dim3(kThreads), 0, st, g, S, L, N, (uint32_t)wps, codes, scales);
        break;
    }
    return after_launch();
}

template <int BLOCK>
zpq_status launch_reduce(const uint8_t* ic, const float* is, int32_t K, int64_t c, uint8_t* oc,
                         float* os, void* ov, int32_t odt, float divisor, hipStream_t st) {
    const unsigned grid = grid_for(c, (int64_t)kThreads * kEplReduce);
    const bool div_fast = divisor >= 1.0f && divisor <= 0x1p40f;
    const float rdiv = 1.0f / divisor;
    if (oc != nullptr) {
        hipLaunchKernelGGL((k_dequant_reduce<BLOCK, kEplReduce, -1, kPfReduce>), dim3(grid),
                           dim3(kThreads), 0, st, ic, is, K, c, oc, os, ov, divisor, rdiv,
                           div_fast);
    } else if (odt == ZPQ_F32) {
        hipLaunchKernelGGL((k_dequant_reduce<BLOCK, kEplReduce, ZPQ_F32, kPfReduce>), dim3(grid),
                           dim3(kThreads), 0, st, ic, is, K, c, oc, os, ov, divisor, rdiv,
                           div_fast);
    } else if (odt == ZPQ_F16) {
        hipLaunchKernelGGL((k_dequant_reduce<BLOCK, kEplReduce, ZPQ_F16, kPfReduce>), dim3(grid),
                           dim3(kThreads), 0, st, ic, is, K, c, oc, os, ov, divisor, rdiv,
                           div_fast);
    } else {
        hipLaunchKernelGGL((k_dequant_reduce<BLOCK, kEplReduce, ZPQ_BF16, kPfReduce>),
                           dim3(grid), dim3(kThreads), 0, st, ic, is, K, c, oc, os, ov, divisor,
                           rdiv, div_fast);
    }
    return after_launch();
}

#define ZPQ_DISPATCH_BLOCK(block, fn, args) \
    switch (block) {                           \
    case 32: return fn<32> args;               \
    case 64: return fn<64> args;               \
    case 128: return fn<128> args;             \
    case 256: return fn<256> args;             \
    default: return fn<512> args;              \
    }

}  // namespace

extern "C" {

zpq_status zpq_quant_i8(const void* x, int32_t x_dtype, int64_t n, int32_t block, int8_t* codes,
                        float* scales, zpq_stream stream) {
    if (!block_ok(block)) return ZPQ_ERR_BLOCK;
    if (n < 0 || n % block != 0) return ZPQ_ERR_SIZE;
    const int64_t eb = dtype_bytes(x_dtype);
    if (eb == 0) return ZPQ_ERR_DTYPE;
    if (n == 0) return ZPQ_OK;
    if (!x || !codes || !scales) return ZPQ_ERR_NULL;
    if (!aligned16(x) || !aligned16(codes) || !aligned16(scales)) return ZPQ_ERR_ALIGN;
    const uint64_t nb = (uint64_t)(n / block) * 4;
    if (overlaps(x, n * eb, codes, n) || overlaps(x, n * eb, scales, nb) ||
        overlaps(codes, n, scales, nb))
        return ZPQ_ERR_ALIAS;
    hipStream_t st = static_cast<hipStream_t>(stream);
    ZPQ_DISPATCH_BLOCK(block, launch_quant_i8, (x, x_dtype, n, codes, scales, st))
}

zpq_status zpq_dequant_i8(const int8_t* codes, const float* scales, int64_t n, int32_t block,
                          void* y, int32_t y_dtype, zpq_stream stream) {
    if (!block_ok(block)) return ZPQ_ERR_BLOCK;
    if (n < 0 || n % block != 0) return ZPQ_ERR_SIZE;
    const int64_t eb = dtype_bytes(y_dtype);
    if (eb == 0) return ZPQ_ERR_DTYPE;
    if (n == 0) return ZPQ_OK;
    if (!codes || !scales || !y) return ZPQ_ERR_NULL;
    if (!aligned16(codes) || !aligned16(scales) || !aligned16(y)) return ZPQ_ERR_ALIGN;
    const uint64_t nb = (uint64_t)(n / block) * 4;
    if (overlaps(y, n * eb, codes, n) || overlaps(y, n * eb, scales, nb)) return ZPQ_ERR_ALIAS;
    hipStream_t st = static_cast<hipStream_t>(stream);
    ZPQ_DISPATCH_BLOCK(block, launch_dequant_i8, (codes, scales, n, y, y_dtype, st))
}

zpq_status zpq_qgz_reorder_quant_i4(const void* grad, int32_t g_dtype, int64_t n,
                                    int32_t local_ranks, int32_t nodes, int32_t block,
                                    uint8_t* codes, float* scales, zpq_stream stream) {
    if (!block_ok(block)) return ZPQ_ERR_BLOCK;
    if (local_ranks < 1 || nodes < 1) return ZPQ_ERR_ARG;
    const int64_t W = (int64_t)local_ranks * nodes;
    if (W > 0x7FFFFFFF) return ZPQ_ERR_ARG;
    if (n < 0 || n % (W * block) != 0) return ZPQ_ERR_SIZE;
    const int64_t eb = dtype_bytes(g_dtype);
    if (eb == 0) return ZPQ_ERR_DTYPE;
    if (n == 0) return ZPQ_OK;
    if (!grad || !codes || !scales) return ZPQ_ERR_NULL;
    if (!aligned16(grad) || !aligned16(codes) || !aligned16(scales)) return ZPQ_ERR_ALIGN;
    const uint64_t nb = (uint64_t)(n / block) * 4;
    if (overlaps(grad, n * eb, codes, n / 2) || overlaps(grad, n * eb, scales, nb) ||
        overlaps(codes, n / 2, scales, nb))
        return ZPQ_ERR_ALIAS;
    hipStream_t st = static_cast<hipStream_t>(stream);
    ZPQ_DISPATCH_BLOCK(block, launch_qgz_quant,
                       (grad, g_dtype, n, local_ranks, nodes, codes, scales, st))
}

zpq_status zpq_qgz_dequant_reduce_requant_i4(const uint8_t* in_codes, const float* in_scales,
                                             int32_t n_src, int64_t chunk_elems, int32_t block,
                                             uint8_t* out_codes, float* out_scales,
                                             void* out_vals, int32_t out_dtype, float divisor,
                                             zpq_stream stream) {
    if (!block_ok(block)) return ZPQ_ERR_BLOCK;
    if (n_src < 1) return ZPQ_ERR_ARG;
    if (chunk_elems < 0 || chunk_elems % block != 0 || chunk_elems >= (1LL << 32))
        return ZPQ_ERR_SIZE;
    const bool mode_i4 = out_codes && out_scales && !out_vals;
    const bool mode_fl = !out_codes && !out_scales && out_vals;
    if (mode_i4 == mode_fl) return ZPQ_ERR_MODE;
    int64_t ob = 0;
    if (mode_fl) {
        ob = dtype_bytes(out_dtype);
        if (ob == 0) return ZPQ_ERR_DTYPE;
        if (!(divisor > 0.0f && divisor <= 3.4028234663852886e38f)) return ZPQ_ERR_ARG;
    }
    if (chunk_elems == 0) return ZPQ_OK;
    if (!in_codes || !in_scales) return ZPQ_ERR_NULL;
    if (!aligned16(in_codes) || !aligned16(in_scales) ||
        (mode_i4 && (!aligned16(out_codes) || !aligned16(out_scales))) ||
        (mode_fl && !aligned16(out_vals)))
        return ZPQ_ERR_ALIGN;
    const uint64_t in_cb = (uint64_t)n_src * (uint64_t)(chunk_elems / 2);
    const uint64_t in_sb = (uint64_t)n_src * (uint64_t)(chunk_elems / block) * 4;
    if (mode_i4) {
        const uint64_t cb = chunk_elems / 2, sb = (uint64_t)(chunk_elems / block) * 4;
        if (overlaps(out_codes, cb, in_codes, in_cb) || overlaps(out_codes, cb, in_scales, in_sb) ||
            overlaps(out_scales, sb, in_codes, in_cb) || overlaps(out_scales, sb, in_scales, in_sb) ||
            overlaps(out_codes, cb, out_scales, sb))
            return ZPQ_ERR_ALIAS;
    } else {
        const uint64_t vb = (uint64_t)chunk_elems * ob;
        if (overlaps(out_vals, vb, in_codes, in_cb) || overlaps(out_vals, vb, in_scales, in_sb))
            return ZPQ_ERR_ALIAS;
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    ZPQ_DISPATCH_BLOCK(block, launch_reduce,
                       (in_codes, in_scales, n_src, chunk_elems, out_codes, out_scales, out_vals,
                        out_dtype, divisor, st))
}

const char* zpq_status_str(zpq_status s) {
    switch (s) {
    case ZPQ_OK: return "ok";
    case ZPQ_ERR_NULL: return "null pointer";
    case ZPQ_ERR_SIZE: return "size is negative or not a whole number of blocks/slices";
    case ZPQ_ERR_BLOCK: return "block must be 32, 64, 128, 256 or 512";
    case ZPQ_ERR_ALIGN: return "pointer not 16-byte aligned";
    case ZPQ_ERR_DTYPE: return "unsupported element type";
    case ZPQ_ERR_MODE: return "select exactly one output mode";
    case ZPQ_ERR_LAUNCH: return "kernel launch failed";
    case ZPQ_ERR_ARG: return "invalid argument";
    case ZPQ_ERR_ALIAS: return "output overlaps an input";
    }
    return "unknown status";
}

int32_t zpq_abi_version(void) { return ZPQ_ABI_VERSION; }

}  // extern "C"
