// bench_patterns.hip -- measurement kernels for bench.py --patterns (not part
// of libzpq; built into libbench_patterns.so beside bench.py).
//
// Two kinds:
//  * ceilings: read-only, write-only and copy streams, 16 bytes per lane and
//    tile, non-temporal, two tiles per lane, one-shot grids of 256-thread
//    workgroups -- what plain streaming reaches on this GPU;
//  * access patterns: for each libzpq kernel, the same per-lane loads and
//    stores (widths, cache hints, lane layout, tiles per lane, sources in
//    flight, grid and workgroup shape, the slice reorder of the qgZ
//    quantizer, the LDS-staged stores of averaged outputs) with the
//    arithmetic replaced by XOR -- what the kernel's memory traffic alone
//    costs.  Their outputs are meaningless;
//  * VALU issue rates: one instruction kind (or one per-element instruction
//    sequence of the hop-receive loop) repeated on registers, eight
//    independent chains per lane, no memory traffic inside the loop -- what
//    the vector ALU sustains per SIMD for that kind.
//
// Every entry point takes device pointers and a hipStream_t, checks nothing
// beyond what its caller (bench.py) guarantees (whole tiles / blocks, the
// sizes of the workloads), and returns the hipGetLastError code.
#include <hip/hip_runtime.h>
#include <stdint.h>

// Wave timeline of the receive pattern (pat_receive with parts bit 2): lane 0
// of each wave stores the 100 MHz constant clock at its start and end.
__device__ uint64_t* pat_tl_buf = nullptr;
__device__ uint32_t pat_tl_waves = 0;

namespace {

constexpr int kThreads = 256;

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <class T>
__device__ __forceinline__ T ldnt(const T* p) { return __builtin_nontemporal_load(p); }
template <class T>
__device__ __forceinline__ void stnt(T v, T* p) { __builtin_nontemporal_store(v, p); }

__device__ __forceinline__ uint32_t fold(u32x4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

// Raw-buffer descriptor over `bytes` bytes from a wave-uniform `base`.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// ---------------------------------------------------------------------------
// Ceilings.  n16 = number of 16-byte units; tile = 256 lanes x 16 bytes.
__global__ __launch_bounds__(kThreads) void k_read(const u32x4* __restrict__ src, int64_t n16,
                                                   uint32_t* __restrict__ sink) {
    const int64_t base = (int64_t)blockIdx.x * (2 * kThreads);
    uint32_t x = 0;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int64_t i = base + u * kThreads + threadIdx.x;
        if (i < n16) x ^= fold(ldnt(src + i));
    }
    if (x == 0x9E3779B9u) sink[threadIdx.x] = x;      // keeps the loads; practically never taken
}

__global__ __launch_bounds__(kThreads) void k_write(u32x4* __restrict__ dst, int64_t n16) {
    const int64_t base = (int64_t)blockIdx.x * (2 * kThreads);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int64_t i = base + u * kThreads + threadIdx.x;
        if (i < n16) stnt(u32x4{(uint32_t)i, 1u, 2u, 3u}, dst + i);
    }
}

__global__ __launch_bounds__(kThreads) void k_copy(const u32x4* __restrict__ src,
                                                   u32x4* __restrict__ dst, int64_t n16) {
    const int64_t base = (int64_t)blockIdx.x * (2 * kThreads);
    u32x4 v[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int64_t i = base + u * kThreads + threadIdx.x;
        v[u] = i < n16 ? ldnt(src + i) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int64_t i = base + u * kThreads + threadIdx.x;
        if (i < n16) stnt(v[u], dst + i);
    }
}

// The same streams with every cache-policy value of the buffer loads and
// stores (AUX: bit 0 sc0, bit 1 nt, bit 4 sc1; the copy's loads keep nt) and
// TPL 16-byte tiles per lane; `bytes` a multiple of 4096 * TPL, below 4 GiB.
template <int AUX, int TPL>
__global__ __launch_bounds__(kThreads) void k_write_pol(void* dst, uint32_t bytes) {
    const auto r = rsrc(dst, bytes);
    const uint32_t base = blockIdx.x * (TPL * kThreads) + threadIdx.x;
#pragma unroll
    for (int u = 0; u < TPL; ++u) {
        const uint32_t off = (base + u * kThreads) * 16;
        __builtin_amdgcn_raw_buffer_store_b128(u32x4{off, 1u, 2u, 3u}, r, off, 0, AUX);
    }
}
template <int AUX, int TPL>
__global__ __launch_bounds__(kThreads) void k_read_pol(const void* src, uint32_t bytes,
                                                       uint32_t* __restrict__ sink) {
    const auto r = rsrc(src, bytes);
    const uint32_t base = blockIdx.x * (TPL * kThreads) + threadIdx.x;
    uint32_t x = 0;
#pragma unroll
    for (int u = 0; u < TPL; ++u)
        x ^= fold(__builtin_amdgcn_raw_buffer_load_b128(r, (base + u * kThreads) * 16, 0, AUX));
    if (x == 0x9E3779B9u) sink[threadIdx.x] = x;
}
template <int AUX, int TPL>
__global__ __launch_bounds__(kThreads) void k_copy_pol(const void* src, void* dst, uint32_t bytes) {
    const auto rs = rsrc(src, bytes), rd = rsrc(dst, bytes);
    const uint32_t base = blockIdx.x * (TPL * kThreads) + threadIdx.x;
    u32x4 v[TPL];
#pragma unroll
    for (int u = 0; u < TPL; ++u)
        v[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, (base + u * kThreads) * 16, 0, 2);
#pragma unroll
    for (int u = 0; u < TPL; ++u)
        __builtin_amdgcn_raw_buffer_store_b128(v[u], rd, (base + u * kThreads) * 16, 0, AUX);
}
constexpr int kPolicies[8] = {0, 1, 2, 3, 16, 17, 18, 19};

// ---------------------------------------------------------------------------
// qwZ quantize (fp16 in, block 256): per lane and tile one 16-byte load (8
// elements), one 8-byte code store, one scale store per 32 lanes; two tiles
// per lane.
__global__ __launch_bounds__(kThreads) void k_pat_quant_i8(const u32x4* __restrict__ x, int64_t n,
                                                           u32x2* __restrict__ codes,
                                                           uint32_t* __restrict__ scales) {
    const int64_t base = (int64_t)blockIdx.x * (2 * kThreads * 8);
    u32x4 v[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int64_t e = base + u * (kThreads * 8) + threadIdx.x * 8;
        v[u] = e < n ? ldnt(x + e / 8) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int64_t e = base + u * (kThreads * 8) + threadIdx.x * 8;
        if (e < n) {
            stnt(u32x2{v[u].x ^ v[u].y, v[u].z ^ v[u].w}, codes + e / 8);
            if ((threadIdx.x & 31) == 0) scales[e / 256] = fold(v[u]);
        }
    }
}

// qwZ dequantize (block 256, fp16 out): per lane one 8-byte code load, one
// scale load, one 16-byte store; workgroups in the XCD-contiguous tile order.
__global__ __launch_bounds__(kThreads) void k_pat_dequant_i8(const u32x2* __restrict__ codes,
                                                             const uint32_t* __restrict__ scales,
                                                             int64_t n, u32x4* __restrict__ y,
                                                             uint32_t nvb) {
    const uint32_t k = blockIdx.x, xcd = k & 7u, i = k >> 3, q = nvb >> 3, r = nvb & 7u;
    const uint32_t vb = xcd * q + (xcd < r ? xcd : r) + i;
    const int64_t e = (int64_t)vb * (kThreads * 8) + threadIdx.x * 8;
    if (e < n) {
        const u32x2 c = ldnt(codes + e / 8);
        const uint32_t s = scales[e / 256];
        stnt(u32x4{c.x ^ s, c.y, c.x, c.y ^ s}, y + e / 8);
    }
}

// qgZ reorder + INT4 quantize (fp16/bf16 in, block 64 or 128): slice-major
// workgroups (send position p = j*N + m reads slice m*L + j), two tiles per
// lane, one 16-byte load and one 4-byte code store per lane and tile (a
// buffer store with cache policy sc0 sc1 nt through a descriptor based at the
// workgroup's codes, as libzpq), one scale store per block.
// CPOL: the code stores' cache-policy bits (19 as libzpq), or -1 for
// non-temporal global stores.
template <int CPOL>
__global__ __launch_bounds__(kThreads) void k_pat_reorder_quant_i4(
    const u32x4* __restrict__ g, int64_t S, int32_t L, int32_t N, uint32_t wgs_per_slice,
    int32_t block, uint32_t* __restrict__ codes, uint32_t* __restrict__ scales) {
    const uint32_t vb = blockIdx.x;
    const uint32_t p = vb / wgs_per_slice, w = vb - p * wgs_per_slice;
    const uint32_t j = p / (uint32_t)N, m = p - j * (uint32_t)N;
    const int64_t src0 = ((int64_t)m * L + j) * S, dst0 = (int64_t)p * S;
    const int64_t f0 = (int64_t)w * (2 * kThreads * 8);
    const uint32_t lanes_per_block = (uint32_t)block / 8;
    const __amdgpu_buffer_rsrc_t rc = rsrc(codes + (dst0 + f0) / 8, 2 * kThreads * 8 / 2);
    u32x4 v[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int64_t f = f0 + u * (kThreads * 8) + threadIdx.x * 8;
        v[u] = f < S ? ldnt(g + (src0 + f) / 8) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int64_t f = f0 + u * (kThreads * 8) + threadIdx.x * 8;
        if (f < S) {
            const int64_t e = dst0 + f;
            if constexpr (CPOL >= 0)
                __builtin_amdgcn_raw_buffer_store_b32(fold(v[u]), rc, (uint32_t)(f - f0) / 2, 0, CPOL);
            else
                stnt(fold(v[u]), codes + e / 8);
            if ((threadIdx.x & (lanes_per_block - 1)) == 0) scales[e / block] = v[u].x;
        }
    }
}

// qgZ hop receive: per lane EPL nibbles (EPL/2 bytes) and one scale from each
// of K sources, PF sources in flight, through buffer descriptors that cover
// one source each (as the kernel reads them); then EPL/2 bytes of codes and a
// scale per block (INT4 output) or EPL 16-bit values (float output).
constexpr int kAux = 2;        // non-temporal loads


template <int EPL>
struct Src {
    uint32_t w[EPL / 8];
    uint32_t s;
};

template <int EPL, bool SC>
__device__ __forceinline__ void load(Src<EPL>& d, const uint8_t* c, uint32_t cb, uint32_t coff,
                                     const uint32_t* s, uint32_t sb, uint32_t soff) {
    const __amdgpu_buffer_rsrc_t rc = rsrc(c, cb);
    if constexpr (EPL == 8) {
        d.w[0] = __builtin_amdgcn_raw_buffer_load_b32(rc, coff, 0, kAux);
    } else if constexpr (EPL == 16) {
        const auto t = __builtin_amdgcn_raw_buffer_load_b64(rc, coff, 0, kAux);
        d.w[0] = t[0]; d.w[1] = t[1];
    } else {
#pragma unroll
        for (int i = 0; i < EPL / 32; ++i) {
            const auto t = __builtin_amdgcn_raw_buffer_load_b128(rc, coff + 16 * i, 0, kAux);
            d.w[4 * i] = t[0]; d.w[4 * i + 1] = t[1]; d.w[4 * i + 2] = t[2]; d.w[4 * i + 3] = t[3];
        }
    }
    d.s = SC ? __builtin_amdgcn_raw_buffer_load_b32(rsrc(s, sb), soff * 4, 0, 0) : soff;
}

template <int EPL>
__device__ __forceinline__ void mix(uint32_t (&acc)[EPL / 8], const Src<EPL>& d) {
#pragma unroll
    for (int i = 0; i < EPL / 8; ++i) acc[i] ^= d.w[i] ^ d.s;
}

__device__ __forceinline__ void pat_mark(int which) {
    if (pat_tl_buf != nullptr && (threadIdx.x & 63) == 0) {
        const uint32_t w = blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64;
        if (w < pat_tl_waves)
            __builtin_nontemporal_store(__builtin_amdgcn_s_memrealtime(), pat_tl_buf + 2 * w + which);
    }
}

// SC: the per-source scale loads; ST: the output stores (both true for the
// pattern proper; the others decompose its time); TL: record the wave timeline.
template <int EPL, int PF, bool I4, bool SC, bool ST, bool TL = false>
__global__ __launch_bounds__(kThreads) void k_pat_receive(
    const uint8_t* __restrict__ in_codes, const uint32_t* __restrict__ in_scales, int32_t K,
    int64_t c, int32_t block, uint8_t* __restrict__ out_codes, uint32_t* __restrict__ out_scales,
    uint16_t* __restrict__ out_vals) {
    constexpr int V = I4 ? 1 : EPL / 8;          // 16-byte output vectors per lane (float output)
    __shared__ u32x4 stage[V >= 2 ? kThreads / 64 : 1][V >= 2 ? V * 64 : 1];
    if constexpr (TL) pat_mark(0);
    const int64_t e = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * EPL;
    if (e >= c) return;
    const int64_t cs = c / 2, ss = c / block;
    const uint32_t coff = (uint32_t)(e / 2), soff = (uint32_t)(e / block);
    const uint32_t cb = (uint32_t)cs, sb = (uint32_t)(ss * 4);
    uint32_t acc[EPL / 8] = {};
    auto ld = [&](Src<EPL>& d, int i) {
        load<EPL, SC>(d, in_codes + (int64_t)i * cs, cb, coff, in_scales + (int64_t)i * ss, sb, soff);
    };
    Src<EPL> buf[PF];
#pragma unroll
    for (int k = 0; k < PF; ++k) ld(buf[k], k);            // K >= PF (bench.py's workloads)
    int i0 = 0;
    for (; i0 + 2 * PF <= K; i0 += PF) {
#pragma unroll
        for (int k = 0; k < PF; ++k) {
            mix<EPL>(acc, buf[k]);
            ld(buf[k], i0 + PF + k);
        }
    }
#pragma unroll
    for (int k = 0; k < PF; ++k) mix<EPL>(acc, buf[k]);
    for (int i = i0 + PF; i < K; ++i) {
        Src<EPL> d;
        ld(d, i);
        mix<EPL>(acc, d);
    }
    if constexpr (!ST) {
        // Keeps the loads: the sum of every lane would have to hit one value.
        if (acc[0] == 0x9E3779B9u && e == 0) {
            if constexpr (I4) out_scales[0] = acc[0];
            else out_vals[0] = 1;
        }
        return;
    }
    if constexpr (I4) {
        uint32_t* dst = reinterpret_cast<uint32_t*>(out_codes + e / 2);
#pragma unroll
        for (int i = 0; i < EPL / 8; i += 4) {
            if constexpr (EPL >= 32)
                stnt(u32x4{acc[i], acc[i + 1], acc[i + 2], acc[i + 3]},
                     reinterpret_cast<u32x4*>(dst + i));
        }
        if constexpr (EPL == 16) stnt(u32x2{acc[0], acc[1]}, reinterpret_cast<u32x2*>(dst));
        if constexpr (EPL == 8) stnt(acc[0], dst);
        const uint32_t lanes_per_block = (uint32_t)block / EPL;
        if ((threadIdx.x & (lanes_per_block - 1)) == 0) out_scales[e / block] = acc[0];
    } else {
        u32x4 o[V];
#pragma unroll
        for (int k = 0; k < V; ++k) o[k] = u32x4{acc[k], acc[k] + 1, acc[k] + 2, acc[k] + 3};
        if (V >= 2 && __builtin_amdgcn_read_exec() == ~0ull) {
            // A whole wave, as libzpq: lane-major into the wave's LDS slice, read
            // back store-major, so that each store covers 1 KB contiguous.
            const int lane = (int)(threadIdx.x & 63);
            u32x4* slice = &stage[V >= 2 ? threadIdx.x / 64 : 0][0];
#pragma unroll
            for (int k = 0; k < V; ++k) slice[lane * V + k] = o[k];
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int k = 0; k < V; ++k) o[k] = slice[k * 64 + lane];
            __builtin_amdgcn_wave_barrier();
            u32x4* dst = reinterpret_cast<u32x4*>(out_vals + (e - (int64_t)lane * EPL));
#pragma unroll
            for (int k = 0; k < V; ++k) stnt(o[k], dst + k * 64 + lane);
        } else {
            u32x4* dst = reinterpret_cast<u32x4*>(out_vals + e);
#pragma unroll
            for (int k = 0; k < V; ++k) stnt(o[k], dst + k);
        }
    }
    if constexpr (TL) pat_mark(1);
}

// ---------------------------------------------------------------------------
// VALU issue rates.  Each kernel runs `iters` iterations of 4 x 8 copies of
// one instruction (or one per-element sequence) on 8 independent register
// chains per lane; an empty asm statement on the inputs each iteration keeps
// the compiler from hoisting anything.  The instructions are written as asm
// so that exactly the named encoding issues.  One store per lane at the end.
#define ZPQB_VALU1(name, text)                                                             \
    __global__ __launch_bounds__(kThreads) void name(uint32_t* out, int iters, float b) {  \
        float a[8];                                                                        \
        for (int i = 0; i < 8; ++i) a[i] = threadIdx.x * 0.001f + i;                        \
        for (int it = 0; it < iters; ++it) {                                                \
            asm volatile("" : "+v"(b));                                                     \
            _Pragma("unroll") for (int r = 0; r < 4; ++r) {                                 \
                _Pragma("unroll") for (int i = 0; i < 8; ++i)                               \
                    asm volatile(text : "+v"(a[i]) : "v"(b));                               \
            }                                                                               \
        }                                                                                   \
        float t = 0.0f;                                                                     \
        for (int i = 0; i < 8; ++i) t += a[i];                                              \
        out[blockIdx.x * kThreads + threadIdx.x] = __float_as_uint(t);                      \
    }
ZPQB_VALU1(k_valu_add, "v_add_f32 %0, %0, %1")
ZPQB_VALU1(k_valu_mul, "v_mul_f32 %0, %0, %1")
ZPQB_VALU1(k_valu_fma, "v_fma_f32 %0, %0, %1, %1")
ZPQB_VALU1(k_valu_cvt_ubyte, "v_cvt_f32_ubyte1 %0, %0")
ZPQB_VALU1(k_valu_cvt_off, "v_cvt_off_f32_i4 %0, %0")
ZPQB_VALU1(k_valu_cvt_sdwa,
           "v_cvt_f32_i32_sdwa %0, sext(%0) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1")
ZPQB_VALU1(k_valu_and, "v_and_b32 %0, %0, %1")
ZPQB_VALU1(k_valu_shift, "v_lshrrev_b32 %0, 4, %0")
ZPQB_VALU1(k_valu_bitop3, "v_bitop3_b32 %0, %0, %1, %1 bitop3:0x6c")
ZPQB_VALU1(k_valu_perm, "v_perm_b32 %0, %0, %1, %1")
ZPQB_VALU1(k_valu_max3, "v_max3_f32 %0, %0, %1, %1")
ZPQB_VALU1(k_valu_fma_mix, "v_fma_mix_f32 %0, %0, %1, %1")
// two-result conversion (two fp8 bytes to two floats) and a binary64 multiply
__global__ __launch_bounds__(kThreads) void k_valu_cvt_pk_fp8(uint32_t* out, int iters, float b) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    uint32_t x[8];
    f32x2 p[8];
    for (int i = 0; i < 8; ++i) x[i] = threadIdx.x * 0x9E3779B9u + i;
    for (int it = 0; it < iters; ++it) {
        _Pragma("unroll") for (int i = 0; i < 8; ++i) asm volatile("" : "+v"(x[i]));
        _Pragma("unroll") for (int r = 0; r < 4; ++r) {
            _Pragma("unroll") for (int i = 0; i < 8; ++i)
                asm volatile("v_cvt_pk_f32_fp8 %0, %1" : "=v"(p[i]) : "v"(x[i]));
        }
    }
    float t = b;
    for (int i = 0; i < 8; ++i) t += p[i].x + p[i].y;
    out[blockIdx.x * kThreads + threadIdx.x] = __float_as_uint(t);
}
__global__ __launch_bounds__(kThreads) void k_valu_mul_f64(uint32_t* out, int iters, float b) {
    double d[8];
    double db = (double)b;
    for (int i = 0; i < 8; ++i) d[i] = threadIdx.x * 0.001 + i;
    for (int it = 0; it < iters; ++it) {
        asm volatile("" : "+v"(db));
        _Pragma("unroll") for (int r = 0; r < 4; ++r) {
            _Pragma("unroll") for (int i = 0; i < 8; ++i)
                asm volatile("v_mul_f64 %0, %0, %1" : "+v"(d[i]) : "v"(db));
        }
    }
    double t = 0.0;
    for (int i = 0; i < 8; ++i) t += d[i];
    out[blockIdx.x * kThreads + threadIdx.x] = __float_as_uint((float)t);
}

// Per-element sequences of a dequantize-and-add loop: a nibble (in byte 1 of
// w) becomes a float, is scaled and added to the element's sum.
#define ZPQB_VALU_SEQ(name, body)                                                          \
    __global__ __launch_bounds__(kThreads) void name(uint32_t* out, int iters, float b) {  \
        float a[8];                                                                        \
        uint32_t w[8];                                                                     \
        const float c = -8.0f * b;                                                         \
        (void)c;                                                                           \
        for (int i = 0; i < 8; ++i) {                                                      \
            a[i] = 0.0f;                                                                    \
            w[i] = (threadIdx.x * 0x9E3779B9u + i) & 0x0F0F0F0Fu;                            \
        }                                                                                   \
        for (int it = 0; it < iters; ++it) {                                                \
            _Pragma("unroll") for (int i = 0; i < 8; ++i) asm volatile("" : "+v"(w[i]));    \
            _Pragma("unroll") for (int r = 0; r < 4; ++r) {                                 \
                _Pragma("unroll") for (int i = 0; i < 8; ++i) {                             \
                    float u;                                                                \
                    body                                                                    \
                }                                                                           \
            }                                                                               \
        }                                                                                   \
        float t = 0.0f;                                                                     \
        for (int i = 0; i < 8; ++i) t += a[i];                                              \
        out[blockIdx.x * kThreads + threadIdx.x] = __float_as_uint(t);                      \
    }
// the receive loop's form: byte conversion, rounding FMA (u - 8) * s, add
ZPQB_VALU_SEQ(k_seq_cvt_fma_add,
              asm volatile("v_cvt_f32_ubyte1 %0, %1" : "=v"(u) : "v"(w[i]));
              asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(u) : "v"(b), "v"(c));
              asm volatile("v_add_f32 %0, %0, %1" : "+v"(a[i]) : "v"(u));)
// the same with a plain multiply (needs a signed value; shown for its rate)
ZPQB_VALU_SEQ(k_seq_cvt_mul_add,
              asm volatile("v_cvt_f32_ubyte1 %0, %1" : "=v"(u) : "v"(w[i]));
              asm volatile("v_mul_f32 %0, %0, %1" : "+v"(u) : "v"(b));
              asm volatile("v_add_f32 %0, %0, %1" : "+v"(a[i]) : "v"(u));)
// signed conversion of a nibble with an SDWA byte select, multiply, add
ZPQB_VALU_SEQ(k_seq_sdwa_mul_add,
              asm volatile("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD "
                           "src0_sel:BYTE_1" : "=v"(u) : "v"(w[i]));
              asm volatile("v_mul_f32 %0, %0, %1" : "+v"(u) : "v"(b));
              asm volatile("v_add_f32 %0, %0, %1" : "+v"(a[i]) : "v"(u));)
// mixed-precision FMA on a 16-bit operand (conversion folded in), add
ZPQB_VALU_SEQ(k_seq_fmamix_add,
              asm volatile("v_fma_mix_f32 %0, %1, %2, %3 op_sel_hi:[1,0,0]"
                           : "=v"(u) : "v"(w[i]), "v"(b), "v"(c));
              asm volatile("v_add_f32 %0, %0, %1" : "+v"(a[i]) : "v"(u));)
// no conversion at all: copy, multiply, add (a lower bound for any form)
ZPQB_VALU_SEQ(k_seq_mov_mul_add,
              asm volatile("v_mov_b32 %0, %1" : "=v"(u) : "v"(w[i]));
              asm volatile("v_mul_f32 %0, %0, %1" : "+v"(u) : "v"(b));
              asm volatile("v_add_f32 %0, %0, %1" : "+v"(a[i]) : "v"(u));)

typedef void (*valu_kernel_t)(uint32_t*, int, float);
struct ValuKind {
    valu_kernel_t fn;
    int instr_per_step;     // instructions per chain and inner step
};
const ValuKind kValuKinds[] = {
    {k_valu_add, 1}, {k_valu_mul, 1}, {k_valu_fma, 1}, {k_valu_cvt_ubyte, 1},
    {k_valu_cvt_off, 1}, {k_valu_cvt_sdwa, 1}, {k_valu_and, 1}, {k_valu_shift, 1},
    {k_valu_bitop3, 1}, {k_valu_perm, 1}, {k_valu_max3, 1}, {k_valu_fma_mix, 1},
    {k_valu_cvt_pk_fp8, 1}, {k_valu_mul_f64, 1},
    {k_seq_cvt_fma_add, 3}, {k_seq_cvt_mul_add, 3}, {k_seq_sdwa_mul_add, 3},
    {k_seq_fmamix_add, 2}, {k_seq_mov_mul_add, 3},
};
constexpr int kNumValuKinds = sizeof(kValuKinds) / sizeof(kValuKinds[0]);

inline unsigned grid_for(int64_t units, int64_t per_wg) {
    return (unsigned)((units + per_wg - 1) / per_wg);
}

template <int EPL, int PF, bool I4>
int launch_pat_receive(unsigned g, unsigned nt, hipStream_t s, const uint8_t* ic,
                       const uint32_t* is, int32_t K, int64_t c, int32_t block, uint8_t* oc,
                       uint32_t* os, uint16_t* ov, int parts) {
    switch (parts) {
    case 3: hipLaunchKernelGGL((k_pat_receive<EPL, PF, I4, true, true>), dim3(g), dim3(nt), 0, s,
                               ic, is, K, c, block, oc, os, ov); break;
    case 2: hipLaunchKernelGGL((k_pat_receive<EPL, PF, I4, false, true>), dim3(g), dim3(nt), 0, s,
                               ic, is, K, c, block, oc, os, ov); break;
    case 1: hipLaunchKernelGGL((k_pat_receive<EPL, PF, I4, true, false>), dim3(g), dim3(nt), 0, s,
                               ic, is, K, c, block, oc, os, ov); break;
    case 0: hipLaunchKernelGGL((k_pat_receive<EPL, PF, I4, false, false>), dim3(g), dim3(nt), 0, s,
                               ic, is, K, c, block, oc, os, ov); break;
    case 7: hipLaunchKernelGGL((k_pat_receive<EPL, PF, I4, true, true, true>), dim3(g), dim3(nt), 0,
                               s, ic, is, K, c, block, oc, os, ov); break;
    default: return (int)hipErrorInvalidValue;
    }
    return hipGetLastError();
}


// ---------------------------------------------------------------------------
// Residency: how many waves of a kernel a SIMD holds at once, by the kernel's
// scalar register count.  Each probe kernel reserves 64 VGPRs and the SGPRs up
// to a given one (empty asm clobbers: the compiler then reports that many plus
// 7 more in use), then sleeps a fixed number of times; lane 0 of each wave
// records its start and end in the timeline buffer (2 words per wave).
#define ZPQ_RES_BODY(CLOB)                                                        \
    const uint32_t w = blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64;          \
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();                          \
    asm volatile("" ::: CLOB, "v63");                                            \
    for (int i = 0; i < iters; ++i) __builtin_amdgcn_s_sleep(64);                  \
    const uint64_t t1 = __builtin_amdgcn_s_memrealtime();                          \
    if ((threadIdx.x & 63) == 0 && w < n) { ts[2 * w] = t0; ts[2 * w + 1] = t1; }
__global__ __launch_bounds__(kThreads) void k_res76(uint64_t* ts, uint32_t n, int iters) { ZPQ_RES_BODY("s69") }
__global__ __launch_bounds__(kThreads) void k_res78(uint64_t* ts, uint32_t n, int iters) { ZPQ_RES_BODY("s71") }
__global__ __launch_bounds__(kThreads) void k_res80(uint64_t* ts, uint32_t n, int iters) { ZPQ_RES_BODY("s73") }
__global__ __launch_bounds__(kThreads) void k_res81(uint64_t* ts, uint32_t n, int iters) { ZPQ_RES_BODY("s74") }
__global__ __launch_bounds__(kThreads) void k_res82(uint64_t* ts, uint32_t n, int iters) { ZPQ_RES_BODY("s75") }
__global__ __launch_bounds__(kThreads) void k_res96(uint64_t* ts, uint32_t n, int iters) { ZPQ_RES_BODY("s89") }
__global__ __launch_bounds__(kThreads) void k_res97(uint64_t* ts, uint32_t n, int iters) { ZPQ_RES_BODY("s90") }
__global__ __launch_bounds__(kThreads) void k_res98(uint64_t* ts, uint32_t n, int iters) { ZPQ_RES_BODY("s91") }
__global__ __launch_bounds__(kThreads) void k_res104(uint64_t* ts, uint32_t n, int iters) { ZPQ_RES_BODY("s97") }
#undef ZPQ_RES_BODY
typedef void (*res_fn)(uint64_t*, uint32_t, int);
const res_fn kResKernels[] = {k_res76, k_res78, k_res80, k_res81, k_res82, k_res96, k_res97, k_res98, k_res104};
const int kResSgprs[] = {76, 78, 80, 81, 82, 96, 97, 98, 104};   // as the compiler reports them
constexpr int kNumRes = sizeof(kResSgprs) / sizeof(kResSgprs[0]);

}  // namespace

extern "C" {

int pat_read(const void* src, int64_t bytes, void* sink, void* st) {
    const int64_t n16 = bytes / 16;
    hipLaunchKernelGGL(k_read, dim3(grid_for(n16, 2 * kThreads)), dim3(kThreads), 0,
                       (hipStream_t)st, (const u32x4*)src, n16, (uint32_t*)sink);
    return hipGetLastError();
}

int pat_write(void* dst, int64_t bytes, void* st) {
    const int64_t n16 = bytes / 16;
    hipLaunchKernelGGL(k_write, dim3(grid_for(n16, 2 * kThreads)), dim3(kThreads), 0,
                       (hipStream_t)st, (u32x4*)dst, n16);
    return hipGetLastError();
}

int pat_copy(const void* src, void* dst, int64_t bytes, void* st) {
    const int64_t n16 = bytes / 16;
    hipLaunchKernelGGL(k_copy, dim3(grid_for(n16, 2 * kThreads)), dim3(kThreads), 0,
                       (hipStream_t)st, (const u32x4*)src, (u32x4*)dst, n16);
    return hipGetLastError();
}

// n fp16 elements, block 256
int pat_quant_i8(const void* x, int64_t n, void* codes, void* scales, void* st) {
    hipLaunchKernelGGL(k_pat_quant_i8, dim3(grid_for(n, 2 * kThreads * 8)), dim3(kThreads), 0,
                       (hipStream_t)st, (const u32x4*)x, n, (u32x2*)codes, (uint32_t*)scales);
    return hipGetLastError();
}

// n elements, block 256, fp16 out
int pat_dequant_i8(const void* codes, const void* scales, int64_t n, void* y, void* st) {
    const unsigned nvb = grid_for(n, kThreads * 8);
    hipLaunchKernelGGL(k_pat_dequant_i8, dim3(nvb), dim3(kThreads), 0, (hipStream_t)st,
                       (const u32x2*)codes, (const uint32_t*)scales, n, (u32x4*)y, nvb);
    return hipGetLastError();
}

// n fp16/bf16 elements, L x N slices, block 64 or 128
int pat_reorder_quant_i4(const void* g, int64_t n, int32_t L, int32_t N, int32_t block,
                         void* codes, void* scales, void* st) {
    const int64_t S = n / ((int64_t)L * N);
    const unsigned wps = grid_for(S, 2 * kThreads * 8);
    hipLaunchKernelGGL(k_pat_reorder_quant_i4<19>, dim3(wps * (unsigned)(L * N)), dim3(kThreads), 0,
                       (hipStream_t)st, (const u32x4*)g, S, L, N, wps, block, (uint32_t*)codes,
                       (uint32_t*)scales);
    return hipGetLastError();
}

// The same with the code stores' cache policy `pol` (0 .. 7: the bits of
// kPolicies[pol]) or non-temporal global stores (pol = -1).
int pat_reorder_quant_i4_pol(int32_t pol, const void* g, int64_t n, int32_t L, int32_t N,
                             int32_t block, void* codes, void* scales, void* st) {
    typedef void (*kf)(const u32x4*, int64_t, int32_t, int32_t, uint32_t, int32_t, uint32_t*,
                       uint32_t*);
    static const kf tab[9] = {k_pat_reorder_quant_i4<-1>, k_pat_reorder_quant_i4<0>,
                              k_pat_reorder_quant_i4<1>, k_pat_reorder_quant_i4<2>,
                              k_pat_reorder_quant_i4<3>, k_pat_reorder_quant_i4<16>,
                              k_pat_reorder_quant_i4<17>, k_pat_reorder_quant_i4<18>,
                              k_pat_reorder_quant_i4<19>};
    if (pol < -1 || pol > 7) return (int)hipErrorInvalidValue;
    const int64_t S = n / ((int64_t)L * N);
    const unsigned wps = grid_for(S, 2 * kThreads * 8);
    hipLaunchKernelGGL(tab[pol + 1], dim3(wps * (unsigned)(L * N)), dim3(kThreads), 0,
                       (hipStream_t)st, (const u32x4*)g, S, L, N, wps, block, (uint32_t*)codes,
                       (uint32_t*)scales);
    return hipGetLastError();
}

// Policy streams: kind 0 read, 1 write, 2 copy; pol 0 .. 7 (kPolicies); tpl 1 or 2.
int pat_stream_pol(int32_t kind, int32_t pol, int32_t tpl, const void* src, void* dst,
                   int64_t bytes, void* sink, void* st) {
#define ZPQ_POL_ROW(T)                                                                          \
    {k_read_pol<0, T>, k_read_pol<1, T>, k_read_pol<2, T>, k_read_pol<3, T>, k_read_pol<16, T>,  \
     k_read_pol<17, T>, k_read_pol<18, T>, k_read_pol<19, T>}
    typedef void (*rf)(const void*, uint32_t, uint32_t*);
    typedef void (*wf)(void*, uint32_t);
    typedef void (*cf)(const void*, void*, uint32_t);
    static const rf rd[2][8] = {ZPQ_POL_ROW(1), ZPQ_POL_ROW(2)};
#undef ZPQ_POL_ROW
    static const wf wr[2][8] = {
        {k_write_pol<0, 1>, k_write_pol<1, 1>, k_write_pol<2, 1>, k_write_pol<3, 1>,
         k_write_pol<16, 1>, k_write_pol<17, 1>, k_write_pol<18, 1>, k_write_pol<19, 1>},
        {k_write_pol<0, 2>, k_write_pol<1, 2>, k_write_pol<2, 2>, k_write_pol<3, 2>,
         k_write_pol<16, 2>, k_write_pol<17, 2>, k_write_pol<18, 2>, k_write_pol<19, 2>}};
    static const cf cp[2][8] = {
        {k_copy_pol<0, 1>, k_copy_pol<1, 1>, k_copy_pol<2, 1>, k_copy_pol<3, 1>,
         k_copy_pol<16, 1>, k_copy_pol<17, 1>, k_copy_pol<18, 1>, k_copy_pol<19, 1>},
        {k_copy_pol<0, 2>, k_copy_pol<1, 2>, k_copy_pol<2, 2>, k_copy_pol<3, 2>,
         k_copy_pol<16, 2>, k_copy_pol<17, 2>, k_copy_pol<18, 2>, k_copy_pol<19, 2>}};
    if (kind < 0 || kind > 2 || pol < 0 || pol > 7 || (tpl != 1 && tpl != 2) || bytes <= 0 ||
        bytes >= (1LL << 32) || bytes % (16LL * kThreads * tpl) != 0)
        return (int)hipErrorInvalidValue;
    const dim3 grid((unsigned)(bytes / (16LL * kThreads * tpl)));
    const hipStream_t s = (hipStream_t)st;
    const uint32_t b = (uint32_t)bytes;
    if (kind == 0) hipLaunchKernelGGL(rd[tpl - 1][pol], grid, dim3(kThreads), 0, s, src, b, (uint32_t*)sink);
    else if (kind == 1) hipLaunchKernelGGL(wr[tpl - 1][pol], grid, dim3(kThreads), 0, s, dst, b);
    else hipLaunchKernelGGL(cp[tpl - 1][pol], grid, dim3(kThreads), 0, s, src, dst, b);
    return hipGetLastError();
}

int pat_policy_bits(int32_t pol) { return (pol >= 0 && pol < 8) ? kPolicies[pol] : -1; }

// K sources x c elements; I4 output (out_codes, out_scales) when out_vals is
// NULL, else 16-bit values.  epl / pf: the launch shape libzpq picks.  parts:
// bit 0 the scale loads, bit 1 the stores (3: the kernel's whole pattern);
// 7: the whole pattern, recording the wave timeline (pat_timeline_set).
int pat_receive(const void* in_codes, const void* in_scales, int32_t K, int64_t c, int32_t block,
                void* out_codes, void* out_scales, void* out_vals, int32_t epl, int32_t pf,
                int32_t parts, void* st) {
    const unsigned nt = kThreads;                // libzpq's receive workgroups: 4 waves
    const unsigned g = grid_for(c, (int64_t)nt * epl);
    const hipStream_t s = (hipStream_t)st;
    const uint8_t* ic = (const uint8_t*)in_codes;
    const uint32_t* is = (const uint32_t*)in_scales;
    uint8_t* oc = (uint8_t*)out_codes;
    uint32_t* os = (uint32_t*)out_scales;
    uint16_t* ov = (uint16_t*)out_vals;
    if (!out_vals && epl == 32 && pf == 2)
        return launch_pat_receive<32, 2, true>(g, nt, s, ic, is, K, c, block, oc, os, ov, parts);
    if (out_vals && epl == 16 && pf == 2)
        return launch_pat_receive<16, 2, false>(g, nt, s, ic, is, K, c, block, oc, os, ov, parts);
    if (out_vals && epl == 8 && pf == 4)
        return launch_pat_receive<8, 4, false>(g, nt, s, ic, is, K, c, block, oc, os, ov, parts);
    return (int)hipErrorInvalidValue;
}

// Where pat_receive with parts 7 records wave times: 2 words per wave for
// the first `waves` waves (NULL: nowhere).
int pat_timeline_set(void* buf, uint32_t waves) {
    if (hipMemcpyToSymbol(HIP_SYMBOL(pat_tl_buf), &buf, sizeof(buf)) != hipSuccess) return 1;
    if (hipMemcpyToSymbol(HIP_SYMBOL(pat_tl_waves), &waves, sizeof(waves)) != hipSuccess) return 2;
    return 0;
}

// Residency probe `i` (0 .. pat_residency_count() - 1): `waves` waves (a
// multiple of 4) in 256-thread workgroups, each sleeping `iters` (1..4096)
// times 64 x 64 cycles; times into `ts` (2 words per wave).
int pat_residency_count(void) { return kNumRes; }
int pat_residency_sgprs(int i) { return (i >= 0 && i < kNumRes) ? kResSgprs[i] : -1; }
int pat_residency(int i, void* ts, uint32_t waves, int32_t iters, void* st) {
    if (i < 0 || i >= kNumRes || waves == 0 || waves % 4 != 0 || iters < 1 || iters > 4096)
        return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(kResKernels[i], dim3(waves / 4), dim3(kThreads), 0, (hipStream_t)st,
                       (uint64_t*)ts, waves, iters);
    return hipGetLastError();
}

// VALU issue-rate kernel `kind` (0 .. pat_valu_kinds() - 1) on `wgs`
// workgroups of 256 threads, `iters` iterations; `out` holds wgs * 256 words.
// Instructions issued per wave: iters * 32 * instr_per_step.
int pat_valu_kinds(void) { return kNumValuKinds; }

int pat_valu_instr_per_step(int kind) {
    return (kind >= 0 && kind < kNumValuKinds) ? kValuKinds[kind].instr_per_step : 0;
}

int pat_valu(int kind, int32_t wgs, int32_t iters, void* out, void* st) {
    if (kind < 0 || kind >= kNumValuKinds || wgs <= 0 || iters <= 0)
        return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(kValuKinds[kind].fn, dim3((unsigned)wgs), dim3(kThreads), 0,
                       (hipStream_t)st, (uint32_t*)out, iters, 1.0001f);
    return hipGetLastError();
}

}  // extern "C"
