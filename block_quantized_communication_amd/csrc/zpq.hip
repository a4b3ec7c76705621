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
// "Abstract (arXiv)"; LIT-102 anthology record, "Key takeaways".)  Plus the
// non-blocked ablation (zpq_quant_i8_tensor: one scale per tensor, the
// summary page's "Measured effects" table and "Surprising findings").
//
// Every kernel streams HBM once (the per-tensor quantizer twice: it needs the
// tensor's maximum before the first code): wide vector loads, one quantization block per
// aligned group of BLOCK/EPL lanes of a wave64 (EPL = elements per lane),
// the block absmax reduced with DPP lane permutes, the division done without
// the IEEE divide (a multiply and one residual correction for 16-bit inputs,
// one binary64 product for binary32 operands, both equal to the IEEE
// quotient where it matters), codes packed in registers and written with
// 64/128-bit stores.  No MFMA: the work is an elementwise map with a
// segmented reduction, bound by HBM bandwidth (and, for the hop-receive
// kernel, by VALU issue).  LDS only stages a wave's averaged outputs so that
// they leave as coalesced 1 KB stores.
//
// Bit-exactness: every result equals the plain definition (IEEE binary32
// operations rounded to nearest even, division included) for all finite
// inputs, except that a NaN the definition produces (a sum meeting +inf and
// -inf) may differ in sign and payload, and requantized blocks whose sums are
// not all finite are unspecified.  Denormals are kept (the gfx950 default
// f32/f16 denormal mode).

#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>
#include <hip/hip_fp16.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <atomic>

#include "zpq.h"

// Launch shapes.  Defaults are the measured best on MI355X; each can be
// overridden at build time (-DZPQ_...) to compare variants.
#ifndef ZPQ_QUANT_EPL
#define ZPQ_QUANT_EPL 8        // elements per lane, INT8 quantize of fp16/bf16 (block <= 256)
#endif
#ifndef ZPQ_QUANT_U
#define ZPQ_QUANT_U 2          // tiles per lane, INT8 quantize
#endif
#ifndef ZPQ_DEQUANT_EPL
#define ZPQ_DEQUANT_EPL 8      // elements per lane, INT8 dequantize
#endif
#ifndef ZPQ_DEQUANT_U
#define ZPQ_DEQUANT_U 1
#endif
#ifndef ZPQ_QGZ_EPL
#define ZPQ_QGZ_EPL 8          // elements per lane, reorder + INT4 quantize of fp16/bf16
#endif
#ifndef ZPQ_QGZ_U
#define ZPQ_QGZ_U 2            // tiles per lane, reorder + INT4 quantize
#endif
#ifndef ZPQ_REDUCE_EPL_I4
#define ZPQ_REDUCE_EPL_I4 32   // elements per lane, hop-1 receive (INT4 out)
#endif
#ifndef ZPQ_REDUCE_EPL_FL
#define ZPQ_REDUCE_EPL_FL 16   // elements per lane, hop-2 receive (float out)
#endif
#ifndef ZPQ_REDUCE_PF_I4
#define ZPQ_REDUCE_PF_I4 2     // received sources in flight per lane (hop 1)
#endif
#ifndef ZPQ_REDUCE_PF_FL
#define ZPQ_REDUCE_PF_FL 2     // received sources in flight per lane (hop 2)
#endif
#ifndef ZPQ_REDUCE_PF_FL_NARROW
#define ZPQ_REDUCE_PF_FL_NARROW 4  // the same with 8 elements per lane (short chunks)
#endif
#ifndef ZPQ_REDUCE_NARROW_WAVES
#define ZPQ_REDUCE_NARROW_WAVES 8  // hop 2: 8 elements per lane below this many waves per SIMD
#endif
#ifndef ZPQ_REDUCE_WG3
#define ZPQ_REDUCE_WG3 0           // receive: 3-wave workgroups where they spread waves more evenly
#endif
// Measurement builds only (never the shipped library): the receive kernel
// records each wave's start and end time (the 100 MHz constant clock) into a
// buffer set by zpq_timeline_set; ZPQ_TIMELINE_WAVES > 0 also fixes its
// occupancy target, so that the recording code does not change the number of
// waves per SIMD the shipped kernel gets.
#ifndef ZPQ_TIMELINE
#define ZPQ_TIMELINE 0
#endif
#ifndef ZPQ_TIMELINE_WAVES
#define ZPQ_TIMELINE_WAVES 0
#endif
// Persistent grids: workgroups per compute unit (0 = one workgroup per
// virtual block, no loop).
#ifndef ZPQ_PERSIST_QUANT
#define ZPQ_PERSIST_QUANT 0
#endif
#ifndef ZPQ_PERSIST_DEQUANT
#define ZPQ_PERSIST_DEQUANT 0
#endif
#ifndef ZPQ_PERSIST_QGZ
#define ZPQ_PERSIST_QGZ 0
#endif
#ifndef ZPQ_PERSIST_REDUCE
#define ZPQ_PERSIST_REDUCE 0
#endif
// Give each XCD a contiguous range of tiles, per kernel.
#ifndef ZPQ_XCD_QUANT
#define ZPQ_XCD_QUANT 0
#endif
#ifndef ZPQ_XCD_DEQUANT
#define ZPQ_XCD_DEQUANT 1
#endif
#ifndef ZPQ_XCD_QGZ
#define ZPQ_XCD_QGZ 0
#endif
#ifndef ZPQ_XCD_REDUCE
#define ZPQ_XCD_REDUCE 0
#endif
#ifndef ZPQ_THREADS
#define ZPQ_THREADS 256
#endif

// Non-temporal hints on streamed loads (L) and stores (S), per kernel.
#ifndef ZPQ_NTL_QUANT
#define ZPQ_NTL_QUANT 1
#endif
#ifndef ZPQ_NTS_QUANT
#define ZPQ_NTS_QUANT 1
#endif
#ifndef ZPQ_NTL_DEQUANT
#define ZPQ_NTL_DEQUANT 1
#endif
#ifndef ZPQ_NTS_DEQUANT
#define ZPQ_NTS_DEQUANT 1
#endif
#ifndef ZPQ_NTL_QGZ
#define ZPQ_NTL_QGZ 1
#endif
#ifndef ZPQ_NTS_QGZ
#define ZPQ_NTS_QGZ 1
#endif
// Cache-policy bits of the qgZ quantizer's code stores, issued as buffer
// stores through a descriptor based at the workgroup's codes (19: sc0 sc1 nt);
// -1: global stores with the ZPQ_NTS_QGZ hint instead.
#ifndef ZPQ_CPOL_QGZ
#define ZPQ_CPOL_QGZ 19
#endif
#ifndef ZPQ_NTL_REDUCE
#define ZPQ_NTL_REDUCE 1
#endif
#ifndef ZPQ_NTS_REDUCE
#define ZPQ_NTS_REDUCE 1
#endif

#if ZPQ_TIMELINE
__device__ uint64_t* zpq_tl_buf = nullptr;     // 2 words per wave: start, end
__device__ uint32_t zpq_tl_waves = 0;
#endif

namespace {

constexpr int kThreads = ZPQ_THREADS;  // 4 waves of 64 per workgroup by default

// Streamed (read-once / write-once) accesses, with or without the
// non-temporal hint.
template <bool NT, class T>
__device__ __forceinline__ T ld_stream(const T* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}
template <bool NT, class T>
__device__ __forceinline__ void st_stream(T v, T* p) {
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

// Buffer descriptor over `bytes` bytes from the wave-uniform address `base`
// (held in SGPRs); lanes supply 32-bit byte offsets, and an access past
// `bytes` reads zeros or is dropped instead of faulting.  Word 3 0x00020000
// is the raw-buffer format for the gfx9 family.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// A store through a descriptor at byte offset `off`, with the cache-policy
// bits CPOL (bit 0 sc0, bit 1 nt, bit 4 sc1).
template <int CPOL, class T>
__device__ __forceinline__ void st_desc(T v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
    static_assert(sizeof(T) == 4 || sizeof(T) == 8 || sizeof(T) == 16, "4, 8 or 16 bytes");
    if constexpr (sizeof(T) == 16) __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, CPOL);
    else if constexpr (sizeof(T) == 8) __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, CPOL);
    else __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, CPOL);
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Tile processed by workgroup k of n.  Workgroups are dispatched round-robin
// over the 8 XCDs (k mod 8); with the remap XCD x takes the contiguous tiles
// [x*q + min(x, r), ...) where n = 8q + r: a bijection on [0, n).
template <bool REMAP>
__device__ __forceinline__ uint32_t tile_of(uint32_t k, uint32_t n) {
    if constexpr (REMAP) {
        const uint32_t x = k & 7u, i = k >> 3, q = n >> 3, r = n & 7u;
        return x * q + (x < r ? x : r) + i;
    } else {
        return k;
    }
}

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
// fl32(x / d) for binary32 x and d > 0, through binary64.  rd = RN64(1/d) is
// within 2^-53 (relatively) of 1/d, so the binary64 product x * rd is within
// 2^-52 of x / d.  A binary32 rounding boundary (a midpoint m between two
// binary32 numbers, 25 significant bits) cannot be closer than 2^-49
// (relatively) to a quotient x / d of binary32 numbers that is itself in the
// normal binary32 range: x - m*d is a nonzero multiple of ulp(m)*ulp(d)/2 (the
// odd part of m*d has at least 25 bits, x at most 24, so they differ).  The
// product therefore lies on the same side of every boundary as x / d, and one
// rounding to binary32 gives the IEEE quotient (the double-rounding argument of
// Figueroa, 1995, with the product's error in place of the first rounding).
// Quotients below 2^-126 are not covered (the boundaries of the subnormal
// grid can be hit exactly); callers route those elsewhere or do not depend
// on them.
__device__ __forceinline__ float div_f64(float x, double rd) {
    return (float)((double)x * rd);
}

// Round-half-even to integer and clamp to [-QMAX, QMAX]; the integer lands in
// the low bits of the returned bit pattern (1.5 * 2^23 + k), so its low byte
// is the two's-complement INT8 code and its low nibble the INT4 code.
template <int QMAX>
__device__ __forceinline__ uint32_t round_code(float t) {
    t = __builtin_amdgcn_fmed3f(t, -(float)QMAX, (float)QMAX);
    return __float_as_uint(t + 12582912.0f);
}

// fl32(x / s) after ONE residual correction, r within one ulp of 1/s.  For
// fp16 and bf16 inputs (x and the block absmax both 16-bit values, s their
// scale) this rounds to the same integer code as the IEEE quotient: checked by
// exhaustion over every absmax, every |x| <= absmax of both types and both
// floats next to 1/s, for qmax 127 and 7.
__device__ __forceinline__ float div_1c(float x, float s, float r) {
    const float q = x * r;
    return __builtin_fmaf(__builtin_fmaf(-q, s, x), r, q);
}

// Round-half-even without the clamp, for the fast path: with a normal scale
// s = fl32(a/QMAX) every |x| <= a has |fl32(x/s)| <= fl32(a/s) <= QMAX(1 + 2^-23),
// which rounds to at most QMAX.
__device__ __forceinline__ uint32_t round_code_fast(float t) {
    return __float_as_uint(t + 12582912.0f);
}

// Codes of N values for a known scale s, as rounded bit patterns.
//  16-bit inputs: fast when s >= 2^-100, with r within one ulp of 1/s
//  (div_1c, exhaustively checked); otherwise the IEEE operator, clamped
//  (s == 0 gives codes 0).
template <int QMAX, int N>
__device__ __forceinline__ void codes16(float s, float r, bool fast, const float (&v)[N],
                                        uint32_t (&out)[N]) {
    if (fast) {
#pragma unroll
        for (int k = 0; k < N; ++k) out[k] = round_code_fast(div_1c(v[k], s, r));
    } else {
#pragma unroll
        for (int k = 0; k < N; ++k) out[k] = round_code<QMAX>(s != 0.0f ? v[k] / s : 0.0f);
    }
}

//  fp32 values: rd = RN64(1/s) (0 when s == 0); the code is rint(div_f64(x, rd)),
//  exact for every s > 0: a quotient below 2^-126, which div_f64 does not
//  cover, is below 1/2 and gives code 0 either way.  normal = (s >= 2^-126):
//  then no code exceeds QMAX and the clamp is skipped.
template <int QMAX, int N>
__device__ __forceinline__ void codes32(double rd, bool normal, const float (&v)[N],
                                        uint32_t (&out)[N]) {
    if (normal) {
#pragma unroll
        for (int k = 0; k < N; ++k) out[k] = round_code_fast(div_f64(v[k], rd));
    } else {
#pragma unroll
        for (int k = 0; k < N; ++k) out[k] = round_code<QMAX>(div_f64(v[k], rd));
    }
}

// Per-block quantizer state from the block absmax a: scale s = fl32(a / QMAX)
// and a reciprocal for the codes.
//  * 16-bit inputs (ONE_STEP true), branch-free: s = fl32(a * k) plus one
//    residual correction (k = fl32(1/QMAX)), and r = the hardware reciprocal
//    of s refined by one Newton step, which leaves r within one ulp of 1/s.
//    For every fp16 and bf16 absmax a >= 2^-90 that s is exactly
//    fl32(a / QMAX), and div_1c with either float next to 1/s gives the IEEE
//    codes: both checked by exhaustion over all (a, x) pairs of both types
//    and both QMAX.  fast = (a >= 2^-90); a slower block's exact scale
//    a / QMAX (possibly subnormal) is computed on its slow path.
//  * fp32 inputs (ONE_STEP false): s = div_f64(a, RN64(1/QMAX)) when a/QMAX is
//    a normal binary32 number (a >= 2^-118), else the IEEE operator; then
//    rd = RN64(1/s) (0 for s == 0) and every code is rint(div_f64(x, rd)),
//    exact for any s > 0 (a quotient too small for div_f64 rounds to code 0
//    either way).  The clamp is needed only when s is subnormal.
template <int QMAX, bool ONE_STEP>
struct BlockScale {
    float a, s, r;
    double rd;
    bool fast;
    BlockScale() = default;
    __device__ __forceinline__ explicit BlockScale(float a_) : a(a_) {
        constexpr float kQ = (float)QMAX;
        constexpr float kInvQ = 1.0f / (float)QMAX;      // fl32(1/QMAX), folded by the compiler
        if constexpr (ONE_STEP) {
            const float s0 = a * kInvQ;
            s = __builtin_fmaf(__builtin_fmaf(-s0, kQ, a), kInvQ, s0);
            const float r0 = __builtin_amdgcn_rcpf(s);
            r = __builtin_fmaf(__builtin_fmaf(-s, r0, 1.0f), r0, r0);
            fast = a >= 0x1p-90f;
        } else {
            constexpr double kInvQ64 = 1.0 / (double)QMAX;
            s = a >= 0x1p-118f ? div_f64(a, kInvQ64) : a / kQ;
            rd = s > 0.0f ? 1.0 / (double)s : 0.0;
            fast = s >= 0x1p-126f;
        }
    }
    // Codes of N values (as rounded bit patterns); afterwards s is the
    // block's scale on every path.
    template <int N>
    __device__ __forceinline__ void codes(const float (&v)[N], uint32_t (&out)[N]) {
        if constexpr (ONE_STEP) {
            if (fast) {
                codes16<QMAX>(s, r, true, v, out);
            } else {
                s = a / (float)QMAX;
                codes16<QMAX>(s, r, false, v, out);
            }
        } else {
            codes32<QMAX>(rd, fast, v, out);
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
template <int EPL, bool NT>
__device__ __forceinline__ void store_nibbles(uint8_t* dst, const uint32_t* packed) {
    if constexpr (EPL == 8) {
        st_stream<NT>(packed[0], reinterpret_cast<uint32_t*>(dst));
    } else if constexpr (EPL == 16) {
        st_stream<NT>(u32x2{packed[0], packed[1]}, reinterpret_cast<u32x2*>(dst));
    } else {
        static_assert(EPL % 32 == 0, "16-byte stores");
#pragma unroll
        for (int k = 0; k < EPL / 32; ++k)
            st_stream<NT>(u32x4{packed[4 * k], packed[4 * k + 1], packed[4 * k + 2],
                                packed[4 * k + 3]},
                          reinterpret_cast<u32x4*>(dst) + k);
    }
}

// The same through a descriptor, from byte offset `off`, cache-policy bits CPOL.
template <int EPL, int CPOL>
__device__ __forceinline__ void store_nibbles(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                              const uint32_t* packed) {
    if constexpr (EPL == 8) {
        st_desc<CPOL>(packed[0], r, off);
    } else if constexpr (EPL == 16) {
        st_desc<CPOL>(u32x2{packed[0], packed[1]}, r, off);
    } else {
        static_assert(EPL % 32 == 0, "16-byte stores");
#pragma unroll
        for (int k = 0; k < EPL / 32; ++k)
            st_desc<CPOL>(u32x4{packed[4 * k], packed[4 * k + 1], packed[4 * k + 2],
                                packed[4 * k + 3]}, r, off + 16 * k);
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

    template <bool NT>
    __device__ __forceinline__ void load(const void* base, int64_t elem) {
        const u32x4* p = reinterpret_cast<const u32x4*>(
            static_cast<const char*>(base) + elem * ElemBytes<DT>::v);
#pragma unroll
        for (int i = 0; i < WORDS / 4; ++i) {
            u32x4 t = ld_stream<NT>(p + i);
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
    // The block's quantizer state; every lane of the aligned group of G lanes
    // holding the block gets the same one.
    template <int QMAX, int G>
    __device__ __forceinline__ BlockScale<QMAX, DT != ZPQ_F32> block_scale() const {
        return BlockScale<QMAX, DT != ZPQ_F32>(__uint_as_float(group_max<G>(absmax_bits())));
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
            for (int i = 0; i < WORDS; ++i)
                m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w[i] & 0x7FFF7FFFu));
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
                                                       float* __restrict__ scales, uint32_t nvb) {
    constexpr int G = BLOCK / EPL;
    for (uint32_t k = blockIdx.x; k < nvb; k += gridDim.x) {
    const uint32_t vb = tile_of<ZPQ_XCD_QUANT>(k, nvb);
    const int64_t wg_base = (int64_t)vb * (U * kThreads * EPL);
    InTile<DT, EPL> tile[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t e = wg_base + (int64_t)u * (kThreads * EPL) + threadIdx.x * EPL;
        if (e < n) tile[u].template load<ZPQ_NTL_QUANT>(x, e); else tile[u].zero();
    }
    // Every tile's block scale first (the divisions of the tiles are
    // independent and interleave), then the codes.
    BlockScale<127, DT != ZPQ_F32> bss[U];
#pragma unroll
    for (int u = 0; u < U; ++u) bss[u] = tile[u].template block_scale<127, G>();
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t e = wg_base + (int64_t)u * (kThreads * EPL) + threadIdx.x * EPL;
        auto& bs = bss[u];
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
            if constexpr (EPL == 8) {
                st_stream<ZPQ_NTS_QUANT>(u32x2{packed[0], packed[1]},
                                         reinterpret_cast<u32x2*>(codes + e));
            }
            u32x4* dst = reinterpret_cast<u32x4*>(codes + e);
#pragma unroll
            for (int k = 0; k < EPL / 16; ++k)
                st_stream<ZPQ_NTS_QUANT>(u32x4{packed[4 * k], packed[4 * k + 1],
                                                  packed[4 * k + 2], packed[4 * k + 3]}, dst + k);
            if ((threadIdx.x & (G - 1)) == 0) scales[e / BLOCK] = bs.s;
        }
    }
    }
}

// ---------------------------------------------------------------------------
// Per-tensor INT8 quantization (non-blocked ablation): three passes.
//  1. at most kTensorPartials workgroups loop over the tiles; each writes the
//     bit pattern of its max |x| into its slot of a uint32 array that
//     overlays the codes buffer (overwritten in pass 3);
//  2. one workgroup reduces those maxima (all loads issued at once) and
//     writes s = fl32(a/127);
//  3. the codes, with that one scale (the block quantizer's code path).
constexpr int kTensorEpl = 8, kTensorU = 2;
constexpr int64_t kTensorTile = (int64_t)kTensorU * kThreads * kTensorEpl;
constexpr int kTensorPartials = 2048;
static_assert(kTensorPartials % kThreads == 0, "whole loads per thread");

// max over a workgroup of per-lane values (bit patterns of non-negative floats)
__device__ __forceinline__ uint32_t workgroup_max(uint32_t v) {
    __shared__ uint32_t part[kThreads / 64];
    v = group_max<32>(v);
    v = max(v, (uint32_t)__builtin_amdgcn_readlane((int)v, 32));
    v = max(v, (uint32_t)__builtin_amdgcn_readlane((int)v, 0));
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
    __syncthreads();
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < kThreads / 64; ++i) m = max(m, part[i]);
    return m;
}

template <int DT>
__global__ __launch_bounds__(kThreads) void k_tensor_absmax(const void* __restrict__ x, int64_t n,
                                                            int64_t ntiles,
                                                            uint32_t* __restrict__ partial) {
    uint32_t m = 0;
    for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        const int64_t base = tile * kTensorTile;
#pragma unroll
        for (int u = 0; u < kTensorU; ++u) {
            const int64_t e = base + (int64_t)u * (kThreads * kTensorEpl) + threadIdx.x * kTensorEpl;
            if (e < n) {
                InTile<DT, kTensorEpl> t;
                t.template load<true>(x, e);
                m = max(m, t.absmax_bits());
            }
        }
    }
    m = workgroup_max(m);
    if (threadIdx.x == 0) partial[blockIdx.x] = m;
}

__global__ __launch_bounds__(kThreads) void k_tensor_scale(const uint32_t* __restrict__ partial,
                                                           int32_t count, float* __restrict__ scale) {
    uint32_t m = 0;
#pragma unroll
    for (int k = 0; k < kTensorPartials / kThreads; ++k) {
        const int i = k * kThreads + threadIdx.x;
        if (i < count) m = max(m, partial[i]);
    }
    m = workgroup_max(m);
    if (threadIdx.x == 0) scale[0] = __uint_as_float(m) / 127.0f;
}

template <int DT>
__global__ __launch_bounds__(kThreads) void k_tensor_codes(const void* __restrict__ x, int64_t n,
                                                           const float* __restrict__ scale,
                                                           int8_t* __restrict__ codes,
                                                           uint32_t nvb) {
    constexpr int EPL = kTensorEpl;
    const float s = scale[0];
    const bool fast16 = s >= 0x1p-100f;
    const float r = fast16 ? 1.0f / s : 0.0f;
    const double rd = s > 0.0f ? 1.0 / (double)s : 0.0;
    for (uint32_t t = blockIdx.x; t < nvb; t += gridDim.x) {
    const int64_t base = (int64_t)t * kTensorTile;
    InTile<DT, EPL> tile[kTensorU];
#pragma unroll
    for (int u = 0; u < kTensorU; ++u) {
        const int64_t e = base + (int64_t)u * (kThreads * EPL) + threadIdx.x * EPL;
        if (e < n) tile[u].template load<true>(x, e); else tile[u].zero();
    }
#pragma unroll
    for (int u = 0; u < kTensorU; ++u) {
        const int64_t e = base + (int64_t)u * (kThreads * EPL) + threadIdx.x * EPL;
        float v[EPL];
#pragma unroll
        for (int k = 0; k < EPL; ++k) v[k] = tile[u].get(k);
        uint32_t q[EPL];
        if constexpr (DT == ZPQ_F32) codes32<127>(rd, s >= 0x1p-126f, v, q);
        else codes16<127>(s, r, fast16, v, q);
        if (e < n)
            st_stream<false>(u32x2{pack_low_bytes(q[0], q[1], q[2], q[3]),
                                   pack_low_bytes(q[4], q[5], q[6], q[7])},
                             reinterpret_cast<u32x2*>(codes + e));
    }
    }
}

// ---------------------------------------------------------------------------
// K2: qwZ INT8 dequantize into fp32 / fp16 / bf16.
template <int OT>
struct OutBytes { static constexpr int v = OT == ZPQ_F32 ? 4 : 2; };

// EPL values in the output type, as EPL * size / 16 16-byte vectors.
template <int OT, int EPL>
__device__ __forceinline__ void pack_out(const float (&v)[EPL], u32x4 (&o)[EPL * OutBytes<OT>::v / 16]) {
    if constexpr (OT == ZPQ_F32) {
#pragma unroll
        for (int k = 0; k < EPL / 4; ++k)
            o[k] = u32x4{__float_as_uint(v[4 * k]), __float_as_uint(v[4 * k + 1]),
                         __float_as_uint(v[4 * k + 2]), __float_as_uint(v[4 * k + 3])};
    } else {
        uint32_t h[EPL / 2];
#pragma unroll
        for (int k = 0; k < EPL / 2; ++k) {
            // The fp32 value must be rounded to fp32 first and then to the
            // 16-bit type.  The empty asm keeps the compiler from fusing the
            // producing operation into a mixed-precision FMA (v_fma_mixlo_f16
            // with a +0 addend), which rounds once and loses the sign of zero.
            // One v_cvt_pk_{f16,bf16}_f32 rounds both values to nearest even.
            f32x2 ab = {v[2 * k], v[2 * k + 1]};
            asm("" : "+v"(ab));
            if constexpr (OT == ZPQ_F16)
                h[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(ab, f16x2));
            else
                h[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(ab, bf16x2));
        }
#pragma unroll
        for (int k = 0; k < EPL / 8; ++k) o[k] = u32x4{h[4 * k], h[4 * k + 1], h[4 * k + 2], h[4 * k + 3]};
    }
}

// The lane's EPL output values (elements e .. e+EPL-1) as consecutive 16-byte stores.
template <int OT, int EPL, bool NT>
__device__ __forceinline__ void store_out(void* __restrict__ y, int64_t e, const float (&v)[EPL]) {
    constexpr int V = EPL * OutBytes<OT>::v / 16;
    u32x4 o[V];
    pack_out<OT, EPL>(v, o);
    u32x4* dst = reinterpret_cast<u32x4*>(static_cast<char*>(y) + e * OutBytes<OT>::v);
#pragma unroll
    for (int k = 0; k < V; ++k) st_stream<NT>(o[k], dst + k);
}

// The same values written by the whole wave as V coalesced 1 KB stores: the
// lanes' vectors pass through the wave's own LDS slice (V * 64 vectors,
// lane-major in, store-major out), so store k of lane L writes the wave's
// 16-byte vector 64k + L.  Needs every lane of the wave active, holding
// elements wbase + EPL*lane .. (wbase = the wave's first element).  With more
// than one vector per lane the plain stores of neighbouring lanes are V*16
// bytes apart and each store instruction covers its 64 lanes' share of
// V KB; these cover 1 KB each.
template <int OT, int EPL, bool NT>
__device__ __forceinline__ void store_out_wave(void* __restrict__ y, int64_t e, const float (&v)[EPL],
                                               u32x4* __restrict__ slice) {
    constexpr int V = EPL * OutBytes<OT>::v / 16;
    u32x4 o[V];
    pack_out<OT, EPL>(v, o);
    const int lane = (int)(threadIdx.x & 63);
#pragma unroll
    for (int k = 0; k < V; ++k) slice[lane * V + k] = o[k];
    __builtin_amdgcn_wave_barrier();        // the reads below take other lanes' writes
#pragma unroll
    for (int k = 0; k < V; ++k) o[k] = slice[k * 64 + lane];
    __builtin_amdgcn_wave_barrier();        // a later use of the slice comes after these reads
    u32x4* dst = reinterpret_cast<u32x4*>(static_cast<char*>(y) + (e - (int64_t)lane * EPL) *
                                                                    OutBytes<OT>::v);
#pragma unroll
    for (int k = 0; k < V; ++k) st_stream<NT>(o[k], dst + k * 64 + lane);
}

template <int OT, int BLOCK, int EPL, int U>
__global__ __launch_bounds__(kThreads) void k_dequant_i8(const int8_t* __restrict__ codes,
                                                         const float* __restrict__ scales,
                                                         int64_t n, void* __restrict__ y,
                                                         uint32_t nvb) {
    static_assert((EPL == 8 || EPL % 16 == 0) && EPL <= BLOCK, "code vectors inside a block");
    constexpr int V = EPL >= 16 ? EPL / 16 : 1;
    for (uint32_t k = blockIdx.x; k < nvb; k += gridDim.x) {
    const uint32_t vb = tile_of<ZPQ_XCD_DEQUANT>(k, nvb);
    const int64_t wg_base = (int64_t)vb * (U * kThreads * EPL);
    u32x4 cw[U][V];
    float s[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t e = wg_base + (int64_t)u * (kThreads * EPL) + threadIdx.x * EPL;
        if (e < n) {
            if constexpr (EPL == 8) {
                const u32x2 t = ld_stream<ZPQ_NTL_DEQUANT>(reinterpret_cast<const u32x2*>(codes + e));
                cw[u][0] = u32x4{t.x, t.y, 0u, 0u};
            } else {
#pragma unroll
                for (int v = 0; v < V; ++v)
                    cw[u][v] = ld_stream<ZPQ_NTL_DEQUANT>(reinterpret_cast<const u32x4*>(codes + e) + v);
            }
            s[u] = scales[e / BLOCK];
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t e = wg_base + (int64_t)u * (kThreads * EPL) + threadIdx.x * EPL;
        if (e < n) {
            float v[EPL];
#pragma unroll
            for (int k = 0; k < EPL; ++k) {
                const u32x4 c = cw[u][k >> 4];
                const uint32_t w = c[(k >> 2) & 3];
                const int8_t q = (int8_t)(w >> (8 * (k & 3)));
                v[k] = (float)q * s[u];
            }
            store_out<OT, EPL, ZPQ_NTS_DEQUANT>(y, e, v);
        }
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
    uint8_t* __restrict__ codes, float* __restrict__ scales, uint32_t nvb) {
    constexpr int G = BLOCK / EPL;
    for (uint32_t k = blockIdx.x; k < nvb; k += gridDim.x) {
    const uint32_t vb = tile_of<ZPQ_XCD_QGZ>(k, nvb);
    const uint32_t p = vb / wgs_per_slice;
    const uint32_t w = vb - p * wgs_per_slice;
    const uint32_t j = p / (uint32_t)N;
    const uint32_t m = p - j * (uint32_t)N;
    const int64_t src0 = ((int64_t)m * L + j) * S;      // first element of slice m*L + j
    const int64_t dst0 = (int64_t)p * S;                 // first element of send position p
    const int64_t f0 = (int64_t)w * (U * kThreads * EPL);
    // The workgroup's codes (U * kThreads * EPL / 2 contiguous bytes) go out
    // as buffer stores with cache policy sc0 sc1 nt: measured 2-3% faster
    // than non-temporal global stores on the 2^28 and 1.06G workloads (sc1
    // alone, or nt alone, equal or slower once the outputs rotate so that
    // none stays in the last-level cache).
    const __amdgpu_buffer_rsrc_t rc = rsrc(codes + (dst0 + f0) / 2, U * kThreads * EPL / 2);
    InTile<DT, EPL> tile[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t f = f0 + (int64_t)u * (kThreads * EPL) + threadIdx.x * EPL;
        if (f < S) tile[u].template load<ZPQ_NTL_QGZ>(grad, src0 + f); else tile[u].zero();
    }
    // Every tile's block scale first (the divisions of the tiles are
    // independent and interleave), then the codes.
    BlockScale<7, DT != ZPQ_F32> bss[U];
#pragma unroll
    for (int u = 0; u < U; ++u) bss[u] = tile[u].template block_scale<7, G>();
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t f = f0 + (int64_t)u * (kThreads * EPL) + threadIdx.x * EPL;
        auto& bs = bss[u];
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
            if constexpr (ZPQ_CPOL_QGZ >= 0)
                store_nibbles<EPL, ZPQ_CPOL_QGZ>(rc, (uint32_t)(f - f0) / 2, packed);
            else
                store_nibbles<EPL, ZPQ_NTS_QGZ>(codes + e / 2, packed);
            if ((threadIdx.x & (G - 1)) == 0) scales[e / BLOCK] = bs.s;
        }
    }
    }
}

// ---------------------------------------------------------------------------
// K4: qgZ dequantize -> fp32 reduce in source order -> INT4 requant or average.
//
// Per source and element: d = fl32(q * s), as ONE rounding of an exact
// expression in u = q + 8 in 0..15 (the nibble with its top bit flipped):
//  * INT4 output (hop 1): u converted by v_cvt_f32_ubyte, d = fma(u, s, -8s);
//  * float output (hop 2, wide launches): one XOR flips the top bit of a dword's eight
//    nibbles, a mask puts two of them into the two 16-bit halves of a
//    register, and v_fma_mix_f32 reads a half as the fp16 number u * 2^-24:
//    d = fma(u * 2^-24, s * 2^24, -8s).
// (Measured per launch shape: the mixed-precision form is faster for the
// float-output launches with 16 or more elements per lane, the conversion
// form for the INT4-output ones; at 8 per lane the two trade places from one
// box to the next, and the conversion form stays.)
// The scaled constants are exact unless they overflow (|s| > FLT_MAX/8 for
// -8s, |s| > FLT_MAX/2^24 for s * 2^24); then that source's term is +-inf or
// NaN (u * inf, 0 * inf or inf - inf) for every element of the lane, since
// all of them share the source's scale, while a term made with finite
// constants is finite.  A non-finite sum never becomes finite again, so the
// lane checks one sum at the end and, if it is not finite, recomputes with
// q * s directly, which is the definition itself and so also right when true
// sums overflow.  The sum is acc = fl32(acc + d), starting at +0, sources in
// order 0..K-1.
template <int EPL>
struct SrcCodes {
    static constexpr int W = EPL / 8;     // dwords of nibbles per lane and source
    uint32_t w[W];
    float s;
};

// Received sources are read through buffer descriptors (rsrc): the source's
// base address lives in SGPRs (advanced per source by scalar adds) and each
// lane supplies only a 32-bit byte offset, so the source loop spends no
// vector instructions on addresses.  A descriptor covers exactly one source's
// chunk (codes) or scale vector; an offset past it would read zeros, not fault.
// Cache-policy operand of the code loads: 2 is the non-temporal bit.
constexpr int kAuxReduce = ZPQ_NTL_REDUCE ? 2 : 0;

template <int EPL>
__device__ __forceinline__ void load_src(SrcCodes<EPL>& d, const uint8_t* cbase, uint32_t cbytes,
                                         uint32_t coff, const float* sbase, uint32_t sbytes,
                                         uint32_t soff) {
    const __amdgpu_buffer_rsrc_t rc = rsrc(cbase, cbytes);
    if constexpr (EPL == 8) {
        d.w[0] = __builtin_amdgcn_raw_buffer_load_b32(rc, coff, 0, kAuxReduce);
    } else if constexpr (EPL == 16) {
        const auto t = __builtin_amdgcn_raw_buffer_load_b64(rc, coff, 0, kAuxReduce);
        d.w[0] = t[0]; d.w[1] = t[1];
    } else {
#pragma unroll
        for (int i = 0; i < EPL / 32; ++i) {
            const auto t = __builtin_amdgcn_raw_buffer_load_b128(rc, coff + 16 * i, 0, kAuxReduce);
            d.w[4 * i] = t[0]; d.w[4 * i + 1] = t[1]; d.w[4 * i + 2] = t[2]; d.w[4 * i + 3] = t[3];
        }
    }
    d.s = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsrc(sbase, sbytes), soff * 4, 0, 0));
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

// fl32(h * s24 + c) where h is the 16-bit half H of x read as an fp16
// number: one v_fma_mix_f32.
template <int H>
__device__ __forceinline__ float fma_mix_half(uint32_t x, float s24, float c) {
    float r;
    if constexpr (H == 0)
        asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[0,0,0] op_sel_hi:[1,0,0]"
            : "=v"(r) : "v"(x), "v"(s24), "v"(c));
    else
        asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
            : "=v"(r) : "v"(x), "v"(s24), "v"(c));
    return r;
}

// acc[e] = fl32(acc[e] + fl32(q_e * s)) for the EPL elements of one source;
// MIX selects the v_fma_mix_f32 form (see above).
template <int EPL, bool MIX>
__device__ __forceinline__ void accumulate(float (&acc)[EPL], const SrcCodes<EPL>& d) {
    if constexpr (MIX) {
        const float s24 = d.s * 0x1p24f;
        const float c8 = d.s * -8.0f;
#pragma unroll
        for (int i = 0; i < SrcCodes<EPL>::W; ++i) {
            const uint32_t x = d.w[i] ^ 0x88888888u;          // every nibble q -> q + 8
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                // nibble k (element 8i+k) in the low half, nibble k+4 in the high half
                const uint32_t h = (x >> (4 * k)) & 0x000F000Fu;
                acc[8 * i + k] = acc[8 * i + k] + fma_mix_half<0>(h, s24, c8);
                acc[8 * i + k + 4] = acc[8 * i + k + 4] + fma_mix_half<1>(h, s24, c8);
            }
        }
        return;
    }
    const float s = d.s;
    const float c = s * -8.0f;
#pragma unroll
    for (int i = 0; i < SrcCodes<EPL>::W; ++i) {
        // nibble q -> q + 8 by flipping its top bit (one 3-input bit op each)
        const uint32_t lo = (d.w[i] & 0x0F0F0F0Fu) ^ 0x08080808u;          // byte k: element 8i+2k
        const uint32_t hi = ((d.w[i] >> 4) & 0x0F0F0F0Fu) ^ 0x08080808u;   // byte k: element 8i+2k+1
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

// max(m, |a|, |b|) and min(m, |a|, |b|) in one v_max3_f32 / v_min3_f32 with
// |.| source modifiers.  Written as asm: the compiler would otherwise
// canonicalize each loop-carried operand first (an extra instruction per
// element).  Quiet NaN operands are ignored (IEEE mode), which the callers
// allow for.
__device__ __forceinline__ float max3_abs(float m, float a, float b) {
    float r;
    asm("v_max3_f32 %0, |%1|, |%2|, %3" : "=v"(r) : "v"(a), "v"(b), "v"(m));
    return r;
}
__device__ __forceinline__ float min3_abs(float m, float a, float b) {
    float r;
    asm("v_min3_f32 %0, |%1|, |%2|, %3" : "=v"(r) : "v"(a), "v"(b), "v"(m));
    return r;
}

// max |v| (mx) or min |v| over N values, in two independent chains so that
// consecutive instructions do not wait on each other.
template <bool MAX, int N>
__device__ __forceinline__ float reduce_abs(const float (&v)[N]) {
    static_assert(N % 2 == 0, "pairs");
    float m0 = MAX ? 0.0f : __builtin_inff(), m1 = m0;
#pragma unroll
    for (int k = 0; k < N; k += 4) {
        m0 = MAX ? max3_abs(m0, v[k], v[k + 1]) : min3_abs(m0, v[k], v[k + 1]);
        if (k + 3 < N)
            m1 = MAX ? max3_abs(m1, v[k + 2], v[k + 3]) : min3_abs(m1, v[k + 2], v[k + 3]);
    }
    return MAX ? fmaxf(m0, m1) : fminf(m0, m1);
}

// acc[e] = fl32(acc[e] + q_e * s) with the product formed directly; the
// first source sets acc[e] = fl32(+0 + q_e * s) (the sum starts at +0).
template <int EPL, bool FIRST>
__device__ __forceinline__ void accumulate_direct(float (&acc)[EPL], const SrcCodes<EPL>& d) {
#pragma unroll
    for (int i = 0; i < SrcCodes<EPL>::W; ++i) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int q = ((int)(d.w[i] << (28 - 4 * k))) >> 28;     // sign-extended nibble
            acc[8 * i + k] = (FIRST ? 0.0f : acc[8 * i + k]) + (float)q * d.s;
        }
    }
}

// The average of the float-output mode, fl32(acc / divisor), set up on the
// host: rdiv = RN64(1/divisor) for the binary64 route, thr its lower bound
// (below), and p2 = 1/divisor when the divisor is a power of two 2^k (then
// 2^-k is a binary32 number and fl32(acc * 2^-k) is the IEEE quotient for
// every acc: the product is exact before its one rounding), else 0.
struct Avg {
    double rdiv;
    float divisor, thr, p2;
};

template <int BLOCK, int EPL, int OUT, int PF>
__device__ __forceinline__ void reduce_tile(
    const uint8_t* __restrict__ in_codes, const float* __restrict__ in_scales, int32_t K,
    int64_t c, uint8_t* __restrict__ out_codes, float* __restrict__ out_scales,
    void* __restrict__ out_vals, Avg avg, int64_t e,
    u32x4* __restrict__ slice);

// 16-byte vectors per lane of the float output; with two or more, the
// output goes through an LDS slice of V * 64 vectors per wave.
template <int OUT, int EPL>
struct OutVectors { static constexpr int v = OUT < 0 ? 0 : EPL * (OUT == ZPQ_F32 ? 4 : 2) / 16; };

#if ZPQ_TIMELINE && ZPQ_TIMELINE_WAVES > 0
#define ZPQ_REDUCE_ATTR __attribute__((amdgpu_waves_per_eu(ZPQ_TIMELINE_WAVES, ZPQ_TIMELINE_WAVES)))
#else
#define ZPQ_REDUCE_ATTR
#endif

// Wave timeline (measurement builds): lane 0 of each wave stores the clock.
__device__ __forceinline__ void timeline_mark(int which) {
#if ZPQ_TIMELINE
    if (zpq_tl_buf != nullptr && (threadIdx.x & 63) == 0) {
        const uint32_t w = blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64;
        if (w < zpq_tl_waves)
            __builtin_nontemporal_store(__builtin_amdgcn_s_memrealtime(), zpq_tl_buf + 2 * w + which);
    }
#else
    (void)which;
#endif
}

// Waves per SIMD on gfx950 also depend on scalar registers, beyond what the
// compiler's occupancy report counts: 8 up to 80 (its count), 7 up to 96, 6
// up to 112 (800 per SIMD, a wave taking its count plus 16, rounded up to 16;
// measured with residency probes).  The INT4 kernel (92) runs 7 waves per
// SIMD; the 16-per-lane average (80) is at the edge of 8.
template <int BLOCK, int EPL, int OUT /* -1: INT4, else a zpq_dtype */, int PF>
__global__ __launch_bounds__(kThreads) ZPQ_REDUCE_ATTR void k_dequant_reduce(
    const uint8_t* __restrict__ in_codes, const float* __restrict__ in_scales, int32_t K,
    int64_t c, uint8_t* __restrict__ out_codes, float* __restrict__ out_scales,
    void* __restrict__ out_vals, Avg avg, uint32_t nvb) {
    constexpr int V = OutVectors<OUT, EPL>::v;
    __shared__ u32x4 stage[V >= 2 ? kThreads / 64 : 1][V >= 2 ? V * 64 : 1];
    u32x4* const slice = &stage[V >= 2 ? threadIdx.x / 64 : 0][0];
    // kThreads threads per workgroup, or kThreads - 64 where a build with
    // ZPQ_REDUCE_WG3 picks 3-wave workgroups (reduce_threads).
    timeline_mark(0);
    for (uint32_t k = blockIdx.x; k < nvb; k += gridDim.x) {
    const uint32_t vb = tile_of<ZPQ_XCD_REDUCE>(k, nvb);
        const int64_t e = ((int64_t)vb * blockDim.x + threadIdx.x) * EPL;
        if (e < c)                 // whole quantization blocks leave together
            reduce_tile<BLOCK, EPL, OUT, PF>(in_codes, in_scales, K, c, out_codes, out_scales,
                                             out_vals, avg, e, slice);
    }
    timeline_mark(1);
}

// The epilogue of a tile: requantize the sums to INT4 codes and block
// scales (OUT < 0) or average them and store them as OUT.
template <int BLOCK, int EPL, int OUT>
__device__ __forceinline__ void finish_tile(const float (&acc)[EPL], int64_t e,
                                            uint8_t* __restrict__ out_codes,
                                            float* __restrict__ out_scales,
                                            void* __restrict__ out_vals, Avg avg,
                                            u32x4* __restrict__ slice) {
    constexpr int G = BLOCK / EPL;
    if constexpr (OUT < 0) {
        // Requantize the sums (sums that are not finite lie outside the
        // quantizer's domain: their block's output is unspecified).
        const float m = reduce_abs<true>(acc);
        const float a = __uint_as_float(group_max<G>(__float_as_uint(m)));
        // The scale s = fl32(a / 7) by the binary64 route (the IEEE operator
        // below 2^-118, where a/7 is no longer a normal binary32 number).
        const float s = a >= 0x1p-118f ? div_f64(a, 1.0 / 7.0) : a / 7.0f;
        uint32_t packed[EPL / 8];
        {
            // Codes from the exact product x * r.  With a normal scale s, r
            // within one ulp of 1/s (the hardware reciprocal refined by one
            // Newton step) and |x| <= a <= 7.0000009 s, x * r lies within
            // 2^-20.1 of x / s, and fl32(x / s) within 2^-22 of x / s: unless
            // x * r is within 2^-19 of a half-integer, rint_even(x * r) and
            // rint_even(fl32(x / s)) are the same integer.  One fused
            // multiply-add with 1.5 * 2^23 rounds the product to that integer
            // (in the low bits of y), a second gives the residual x * r - q.
            // A lane holding a value that close (or a scale below 2^-126)
            // takes the binary64 route for all its codes.  Checked on the
            // CPU, with both floats next to 1/s, for every value within 16
            // ulp of every rounding boundary of quantizer-produced scales in
            // every binade.
            const float r0 = __builtin_amdgcn_rcpf(s);
            const float r = __builtin_fmaf(__builtin_fmaf(-s, r0, 1.0f), r0, r0);
            bool near = !(s >= 0x1p-126f);
#pragma unroll
            for (int k = 0; k < EPL / 8; ++k) {
                uint32_t q[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float y = __builtin_fmaf(acc[8 * k + j], r, 12582912.0f);
                    const float d = __builtin_fmaf(acc[8 * k + j], r, -(y - 12582912.0f));
                    near |= fabsf(d) > 0.5f - 0x1p-19f;
                    q[j] = __float_as_uint(y);
                }
                packed[k] = pack_nibbles(q);
            }
            if (near) {
                BlockScale<7, false> bs(a);               // the same s, and RN64(1/s)
#pragma unroll
                for (int k = 0; k < EPL / 8; ++k) {       // 8 codes at a time: few live registers
                    float v[8];
                    uint32_t q[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) v[j] = acc[8 * k + j];
                    bs.codes(v, q);
                    packed[k] = pack_nibbles(q);
                }
            }
        }
        store_nibbles<EPL, ZPQ_NTS_REDUCE>(out_codes + e / 2, packed);
        if ((threadIdx.x & (G - 1)) == 0) out_scales[e / BLOCK] = s;
    } else {
        // y = fl32(acc / divisor) = div_f64(acc, RN64(1/divisor)) whenever the
        // quotient is a normal binary32 number or overflows, i.e. for
        // |acc| >= thr = 2^-126 * divisor (rounded up; set on the host), and
        // for acc == 0, infinities and NaN.  A lane with a smaller nonzero sum
        // divides those with the IEEE operator.
        // With 16 or more sums per lane a power-of-two divisor takes one
        // multiply per sum (measured 1.4% faster for the 16-source average by
        // 16; at 8 per lane the extra branch cost as much as it saved).
        float y[EPL];
        if (EPL >= 16 && avg.p2 != 0.0f) {
#pragma unroll
            for (int k = 0; k < EPL; ++k) y[k] = acc[k] * avg.p2;
        } else if (reduce_abs<false>(acc) >= avg.thr) {
#pragma unroll
            for (int k = 0; k < EPL; ++k) y[k] = div_f64(acc[k], avg.rdiv);
        } else {
#pragma unroll
            for (int k = 0; k < EPL; ++k)
                y[k] = (fabsf(acc[k]) >= avg.thr || acc[k] == 0.0f) ? div_f64(acc[k], avg.rdiv)
                                                                     : acc[k] / avg.divisor;
        }
        if constexpr (OutVectors<OUT, EPL>::v >= 2) {
            if (__builtin_amdgcn_read_exec() == ~0ull)      // a whole wave: coalesced stores
                store_out_wave<OUT, EPL, ZPQ_NTS_REDUCE>(out_vals, e, y, slice);
            else
                store_out<OUT, EPL, ZPQ_NTS_REDUCE>(out_vals, e, y);
        } else {
            store_out<OUT, EPL, ZPQ_NTS_REDUCE>(out_vals, e, y);
        }
    }
}

template <int BLOCK, int EPL, int OUT, int PF>
__device__ __forceinline__ void reduce_tile(
    const uint8_t* __restrict__ in_codes, const float* __restrict__ in_scales, int32_t K,
    int64_t c, uint8_t* __restrict__ out_codes, float* __restrict__ out_scales,
    void* __restrict__ out_vals, Avg avg, int64_t e,
    u32x4* __restrict__ slice) {
    const int64_t cstride = c / 2, sstride = c / BLOCK;
    const uint32_t coff = (uint32_t)(e / 2), soff = (uint32_t)(e / BLOCK);   // c < 2^32
    const uint32_t cbytes = (uint32_t)cstride, sbytes = (uint32_t)(sstride * 4);

    float acc[EPL];
#pragma unroll
    for (int k = 0; k < EPL; ++k) acc[k] = 0.0f;

    // Sources in flight.  The steady-state loop refills every slot without a
    // condition (a whole group of PF sources always remains), so the
    // compiler can wait for exactly the oldest load instead of all of them.
    auto src_load = [&](SrcCodes<EPL>& d, int i) {
        load_src<EPL>(d, in_codes + (int64_t)i * cstride, cbytes, coff,
                      in_scales + (int64_t)i * sstride, sbytes, soff);
    };
    if (K >= PF) {
        SrcCodes<EPL> buf[PF];
#pragma unroll
        for (int k = 0; k < PF; ++k) src_load(buf[k], k);
        int i0 = 0;
        for (; i0 + 2 * PF <= K; i0 += PF) {
#pragma unroll
            for (int k = 0; k < PF; ++k) {
                accumulate<EPL, (OUT >= 0 && EPL >= 16)>(acc, buf[k]);
                src_load(buf[k], i0 + PF + k);
            }
        }
#pragma unroll
        for (int k = 0; k < PF; ++k) accumulate<EPL, (OUT >= 0 && EPL >= 16)>(acc, buf[k]);
        for (int i = i0 + PF; i < K; ++i) {          // fewer than PF left
            SrcCodes<EPL> d;
            src_load(d, i);
            accumulate<EPL, (OUT >= 0 && EPL >= 16)>(acc, d);
        }
    } else {
        for (int i = 0; i < K; ++i) {
            SrcCodes<EPL> d;
            src_load(d, i);
            accumulate<EPL, (OUT >= 0 && EPL >= 16)>(acc, d);
        }
    }
    // An overflowed -8s leaves every sum of the lane -inf or NaN (see above):
    // one sum decides whether the lane recomputes its sums with q * s
    // directly.  For INT4 output the recomputation sets the sums from source
    // 0 instead of clearing them first: the compiler merges a cleared start
    // into the usual path as one select per sum (32 instructions per tile,
    // measured 1-2% of the hop-1 time).  The float-output kernels keep the
    // cleared start: there the other form measured 3% slower (16 per lane)
    // or needs more scalar registers than 8 waves per SIMD leave (8 per lane).
    if (!(fabsf(acc[0]) <= 3.4028234663852886e38f)) {
        if constexpr (OUT < 0) {
            SrcCodes<EPL> d;
            src_load(d, 0);
            accumulate_direct<EPL, true>(acc, d);
        } else {
#pragma unroll
            for (int k = 0; k < EPL; ++k) acc[k] = 0.0f;
        }
        for (int i = OUT < 0 ? 1 : 0; i < K; ++i) {
            SrcCodes<EPL> d;
            src_load(d, i);
            accumulate_direct<EPL, false>(acc, d);
        }
    }
    finish_tile<BLOCK, EPL, OUT>(acc, e, out_codes, out_scales, out_vals, avg, slice);
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

// Compute units of the current device (cached per device id; host threads
// may race to fill an entry, with the same value).
inline int cu_count() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Element counts above 2^40 are refused (ZPQ_ERR_SIZE): grid sizes stay
// within 32 bits and byte counts within 64.
constexpr int64_t kMaxElems = 1LL << 40;

// A dispatch holds at most 2^32 - 1 work-items per dimension, so at most
// kMaxGrid workgroups; every kernel loops over its virtual blocks with a
// stride of the grid size, so a capped grid still covers them all.
constexpr unsigned kMaxGrid = 0xFFFFFFFFu / kThreads;

// Launch grid for nvb virtual blocks: all of them (up to kMaxGrid), or a
// persistent grid of per_cu workgroups per compute unit that loops over them.
inline unsigned launch_grid(uint64_t nvb, int per_cu) {
    uint64_t g = nvb;
    if (per_cu > 0 && (uint64_t)per_cu * (uint64_t)cu_count() < g)
        g = (uint64_t)per_cu * (uint64_t)cu_count();
    return (unsigned)(g < kMaxGrid ? g : kMaxGrid);
}

// Launch shapes (elements per lane, tiles per lane, sources in flight).
// fp16/bf16 inputs use 8 elements per lane (one 16-byte load, so each load
// instruction of a wave covers 1 KB contiguous) when the block fits in 32
// lanes; fp32 inputs and block 512 use 16.
template <int DT, int BLOCK, int EPL16>
constexpr int epl_in() { return (DT != ZPQ_F32 && BLOCK / EPL16 <= 32) ? EPL16 : 16; }
constexpr int kEplQuant = ZPQ_QUANT_EPL, kUQuant = ZPQ_QUANT_U;
constexpr int kEplDequant = ZPQ_DEQUANT_EPL, kUDequant = ZPQ_DEQUANT_U;
constexpr int kEplQgz = ZPQ_QGZ_EPL, kUQgz = ZPQ_QGZ_U;
constexpr int kEplI4 = ZPQ_REDUCE_EPL_I4, kEplFl = ZPQ_REDUCE_EPL_FL;
constexpr int kPfI4 = ZPQ_REDUCE_PF_I4, kPfFl = ZPQ_REDUCE_PF_FL;
constexpr int kPfFlNarrow = ZPQ_REDUCE_PF_FL_NARROW;

template <int DT, int BLOCK>
void launch_quant_dt(const void* x, int64_t n, int8_t* codes, float* scales, hipStream_t st) {
    constexpr int E = epl_in<DT, BLOCK, kEplQuant>();
    const unsigned nvb = grid_for(n, (int64_t)kUQuant * kThreads * E);
    hipLaunchKernelGGL((k_quant_i8<DT, BLOCK, E, kUQuant>), dim3(launch_grid(nvb, ZPQ_PERSIST_QUANT)),
                       dim3(kThreads), 0, st, x, n, codes, scales, nvb);
}

template <int BLOCK>
zpq_status launch_quant_i8(const void* x, int32_t dt, int64_t n, int8_t* codes, float* scales,
                           hipStream_t st) {
    switch (dt) {
    case ZPQ_F32: launch_quant_dt<ZPQ_F32, BLOCK>(x, n, codes, scales, st); break;
    case ZPQ_F16: launch_quant_dt<ZPQ_F16, BLOCK>(x, n, codes, scales, st); break;
    default: launch_quant_dt<ZPQ_BF16, BLOCK>(x, n, codes, scales, st); break;
    }
    return after_launch();
}

template <int BLOCK>
zpq_status launch_dequant_i8(const int8_t* codes, const float* scales, int64_t n, void* y,
                             int32_t dt, hipStream_t st) {
    constexpr int E = kEplDequant <= BLOCK ? kEplDequant : 16;
    const unsigned nvb = grid_for(n, (int64_t)kUDequant * kThreads * E);
    const unsigned grid = launch_grid(nvb, ZPQ_PERSIST_DEQUANT);
    switch (dt) {
    case ZPQ_F32:
        hipLaunchKernelGGL((k_dequant_i8<ZPQ_F32, BLOCK, E, kUDequant>), dim3(grid),
                           dim3(kThreads), 0, st, codes, scales, n, y, nvb);
        break;
    case ZPQ_F16:
        hipLaunchKernelGGL((k_dequant_i8<ZPQ_F16, BLOCK, E, kUDequant>), dim3(grid),
                           dim3(kThreads), 0, st, codes, scales, n, y, nvb);
        break;
    default:
        hipLaunchKernelGGL((k_dequant_i8<ZPQ_BF16, BLOCK, E, kUDequant>), dim3(grid),
                           dim3(kThreads), 0, st, codes, scales, n, y, nvb);
        break;
    }
    return after_launch();
}

template <int DT, int BLOCK>
zpq_status launch_qgz_dt(const void* g, int64_t n, int32_t L, int32_t N, uint8_t* codes,
                         float* scales, hipStream_t st) {
    constexpr int E = epl_in<DT, BLOCK, kEplQgz>();
    const int64_t W = (int64_t)L * N;
    const int64_t S = n / W;
    const int64_t per_wg = (int64_t)kUQgz * kThreads * E;
    const int64_t wps = (S + per_wg - 1) / per_wg;
    if (wps * W > 0x7FFFFFFFLL) return ZPQ_ERR_SIZE;
    const unsigned nvb = (unsigned)(wps * W);
    hipLaunchKernelGGL((k_reorder_quant_i4<DT, BLOCK, E, kUQgz>),
                       dim3(launch_grid(nvb, ZPQ_PERSIST_QGZ)), dim3(kThreads), 0, st, g, S, L, N,
                       (uint32_t)wps, codes, scales, nvb);
    return after_launch();
}

template <int BLOCK>
zpq_status launch_qgz_quant(const void* g, int32_t dt, int64_t n, int32_t L, int32_t N,
                            uint8_t* codes, float* scales, hipStream_t st) {
    switch (dt) {
    case ZPQ_F32: return launch_qgz_dt<ZPQ_F32, BLOCK>(g, n, L, N, codes, scales, st);
    case ZPQ_F16: return launch_qgz_dt<ZPQ_F16, BLOCK>(g, n, L, N, codes, scales, st);
    default: return launch_qgz_dt<ZPQ_BF16, BLOCK>(g, n, L, N, codes, scales, st);
    }
}

template <int BLOCK, int EPL>
constexpr int epl_for() {
    return EPL > BLOCK ? BLOCK : (BLOCK / EPL <= 32 ? EPL : BLOCK / 32);   // a block spans <= 32 lanes
}

// Threads per workgroup of a receive launch over c elements at EPL per lane:
// kThreads (4 waves), or, built with ZPQ_REDUCE_WG3, one wave fewer where
// that leaves fewer waves on the busiest compute unit (the dispatcher spreads
// workgroups evenly over the CUs).  For example, the 48-source hop 2 of a
// 138B-model layer has 5376 waves: 1344 workgroups of 4 put 24 waves on 64 of
// the 256 CUs and 20 on the rest, 1792 of 3 put 21 on every CU.  Measured
// against 4-wave workgroups: faster on two boards, 4-7% slower on four, so
// it is off by default.
inline unsigned reduce_threads(int64_t c, int epl) {
    constexpr int64_t wmax = kThreads / 64;
    if (wmax < 2 || !ZPQ_REDUCE_WG3) return kThreads;
    const int64_t waves = (c + 64LL * epl - 1) / (64LL * epl);
    const int64_t n = cu_count();
    auto busiest = [&](int64_t w) { return ((waves + w - 1) / w + n - 1) / n * w; };
    return (unsigned)(64 * (busiest(wmax - 1) < busiest(wmax) ? wmax - 1 : wmax));
}

template <int BLOCK, int EPL, int PF>
void launch_reduce_fl(const uint8_t* ic, const float* is, int32_t K, int64_t c, void* ov,
                      int32_t odt, Avg avg, hipStream_t st) {
    const unsigned nt = reduce_threads(c, EPL);
    const unsigned nvb = grid_for(c, (int64_t)nt * EPL);
    const dim3 grid(launch_grid(nvb, ZPQ_PERSIST_REDUCE));
    if (odt == ZPQ_F32)
        hipLaunchKernelGGL((k_dequant_reduce<BLOCK, EPL, ZPQ_F32, PF>), grid, dim3(nt), 0,
                           st, ic, is, K, c, nullptr, nullptr, ov, avg, nvb);
    else if (odt == ZPQ_F16)
        hipLaunchKernelGGL((k_dequant_reduce<BLOCK, EPL, ZPQ_F16, PF>), grid, dim3(nt), 0,
                           st, ic, is, K, c, nullptr, nullptr, ov, avg, nvb);
    else
        hipLaunchKernelGGL((k_dequant_reduce<BLOCK, EPL, ZPQ_BF16, PF>), grid, dim3(nt), 0,
                           st, ic, is, K, c, nullptr, nullptr, ov, avg, nvb);
}

template <int BLOCK>
zpq_status launch_reduce(const uint8_t* ic, const float* is, int32_t K, int64_t c, uint8_t* oc,
                         float* os, void* ov, int32_t odt, float divisor, hipStream_t st) {
    constexpr int EI = epl_for<BLOCK, kEplI4>(), EF = epl_for<BLOCK, kEplFl>();
    // FLOAT mode: the smallest binary32 thr with thr / divisor >= 2^-126 for
    // the exact quotient (2^-126 * divisor is exact in binary64; round up).
    Avg avg;
    avg.divisor = divisor;
    avg.rdiv = 1.0 / (double)divisor;
    const double t64 = ldexp((double)divisor, -126);
    avg.thr = (float)t64;
    if ((double)avg.thr < t64) avg.thr = nextafterf(avg.thr, __builtin_inff());
    int ex = 0;
    // divisor = 2^(ex-1) when its significand is 1/2; 2^(1-ex) is finite for ex >= -126
    avg.p2 = (frexpf(divisor, &ex) == 0.5f && ex >= -126) ? ldexpf(1.0f, 1 - ex) : 0.0f;
    if (oc != nullptr) {
        const unsigned nt = reduce_threads(c, EI);
        const unsigned nvb = grid_for(c, (int64_t)nt * EI);
        hipLaunchKernelGGL((k_dequant_reduce<BLOCK, EI, -1, kPfI4>),
                           dim3(launch_grid(nvb, ZPQ_PERSIST_REDUCE)), dim3(nt), 0, st, ic,
                           is, K, c, oc, os, ov, avg, nvb);
        return after_launch();
    }
    // A short chunk gives few waves at 16 elements per lane (the fused
    // workload's hop 2: 2.6 per SIMD); halving the lane's share doubles them.
    const int64_t waves16 = (c + 16 * 64 - 1) / (16 * 64);
    if (BLOCK <= 256 && waves16 < (int64_t)ZPQ_REDUCE_NARROW_WAVES * 4 * cu_count())
        launch_reduce_fl<BLOCK, 8, kPfFlNarrow>(ic, is, K, c, ov, odt, avg, st);
    else
        launch_reduce_fl<BLOCK, EF, kPfFl>(ic, is, K, c, ov, odt, avg, st);
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
    if (n < 0 || n > kMaxElems || n % block != 0) return ZPQ_ERR_SIZE;
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

zpq_status zpq_quant_i8_tensor(const void* x, int32_t x_dtype, int64_t n, int8_t* codes,
                               float* scale, zpq_stream stream) {
    if (n < 0 || n > kMaxElems || n % 16 != 0) return ZPQ_ERR_SIZE;
    const int64_t eb = dtype_bytes(x_dtype);
    if (eb == 0) return ZPQ_ERR_DTYPE;
    if (!scale) return ZPQ_ERR_NULL;
    if (n > 0 && (!x || !codes)) return ZPQ_ERR_NULL;
    if (!aligned16(scale) || (n > 0 && (!aligned16(x) || !aligned16(codes)))) return ZPQ_ERR_ALIGN;
    if (overlaps(x, n * eb, codes, n) || overlaps(x, n * eb, scale, 4) ||
        overlaps(codes, n, scale, 4))
        return ZPQ_ERR_ALIAS;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t nwg = (n + kTensorTile - 1) / kTensorTile;           // tiles of the codes pass
    const int32_t np = (int32_t)(nwg < kTensorPartials ? nwg : kTensorPartials);
    uint32_t* partial = reinterpret_cast<uint32_t*>(codes);     // np * 4 <= n bytes
    if (np > 0) {
        switch (x_dtype) {
        case ZPQ_F32:
            hipLaunchKernelGGL(k_tensor_absmax<ZPQ_F32>, dim3(np), dim3(kThreads), 0, st, x, n,
                               nwg, partial);
            break;
        case ZPQ_F16:
            hipLaunchKernelGGL(k_tensor_absmax<ZPQ_F16>, dim3(np), dim3(kThreads), 0, st, x, n,
                               nwg, partial);
            break;
        default:
            hipLaunchKernelGGL(k_tensor_absmax<ZPQ_BF16>, dim3(np), dim3(kThreads), 0, st, x, n,
                               nwg, partial);
            break;
        }
    }
    hipLaunchKernelGGL(k_tensor_scale, dim3(1), dim3(kThreads), 0, st, partial, np, scale);
    if (nwg > 0) {
        const unsigned g = launch_grid((uint64_t)nwg, 0);
        const uint32_t nvb = (uint32_t)nwg;                 // n <= 2^40: nwg <= 2^28
        switch (x_dtype) {
        case ZPQ_F32:
            hipLaunchKernelGGL(k_tensor_codes<ZPQ_F32>, dim3(g), dim3(kThreads), 0, st, x, n,
                               scale, codes, nvb);
            break;
        case ZPQ_F16:
            hipLaunchKernelGGL(k_tensor_codes<ZPQ_F16>, dim3(g), dim3(kThreads), 0, st, x, n,
                               scale, codes, nvb);
            break;
        default:
            hipLaunchKernelGGL(k_tensor_codes<ZPQ_BF16>, dim3(g), dim3(kThreads), 0, st, x, n,
                               scale, codes, nvb);
            break;
        }
    }
    return after_launch();
}

zpq_status zpq_dequant_i8(const int8_t* codes, const float* scales, int64_t n, int32_t block,
                          void* y, int32_t y_dtype, zpq_stream stream) {
    if (!block_ok(block)) return ZPQ_ERR_BLOCK;
    if (n < 0 || n > kMaxElems || n % block != 0) return ZPQ_ERR_SIZE;
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
    if (n < 0 || n > kMaxElems || n % (W * block) != 0) return ZPQ_ERR_SIZE;
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

#if ZPQ_TIMELINE
// Measurement builds: where the receive kernel records wave times (2 words
// per wave, for the first `waves` waves of each launch; NULL stops it).
int32_t zpq_timeline_set(void* buf, uint32_t waves) {
    if (hipMemcpyToSymbol(HIP_SYMBOL(zpq_tl_buf), &buf, sizeof(buf)) != hipSuccess) return 1;
    if (hipMemcpyToSymbol(HIP_SYMBOL(zpq_tl_waves), &waves, sizeof(waves)) != hipSuccess) return 2;
    return 0;
}
#endif

}  // extern "C"
