// Device helpers shared by the gfx950 kernels: element formats, 16-byte
// vectors, MFMA operand types and the fused epilogue.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "../tlgemm_internal.h"

namespace tlg {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---- element formats ------------------------------------------------------------
// Storage: fp32 as float, fp16 and bf16 as their 16-bit patterns.
template <int DT> struct Elem;
template <> struct Elem<TLG_F32> {
    using storage = float;
    static constexpr int per16 = 4;  // elements per 16-byte vector
    __device__ static float to_f32(float v) { return v; }
};
template <> struct Elem<TLG_F16> {
    using storage = uint16_t;
    static constexpr int per16 = 8;
    __device__ static float to_f32(uint16_t v) { return (float)__builtin_bit_cast(_Float16, v); }
};
template <> struct Elem<TLG_BF16> {
    using storage = uint16_t;
    static constexpr int per16 = 8;
    __device__ static float to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }
};

// fp32 -> bf16, round to nearest even (gfx950's conversion instruction,
// v_cvt_pk_bf16_f32, under the default rounding mode); NaN stays NaN.  Two
// values at a time where they are packed together: one instruction for the
// pair, where rounding in integer arithmetic took five per value (measured on
// the square 4096³ bf16 -> bf16 GEMM, whose epilogue converts 16.8 M values).
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ inline uint16_t f32_to_bf16_rne(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
__device__ inline uint32_t f32x2_to_bf16x2_rne(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}
// fp32 pair -> fp16 pair, round to nearest even (v_cvt_pk_f16_f32).
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
__device__ inline uint32_t f32x2_to_f16x2_rne(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, f16x2_t));
}
// Two fp32 values as the packed 16-bit pair of the output type.
template <int DT> __device__ inline uint32_t pack2(float lo, float hi) {
    static_assert(DT != TLG_F32, "16-bit types only");
    if constexpr (DT == TLG_F16) return f32x2_to_f16x2_rne(lo, hi);
    else return f32x2_to_bf16x2_rne(lo, hi);
}

template <int DT> __device__ inline void store_out(void* Y, int64_t idx, float v) {
    if constexpr (DT == TLG_F32) {
        static_cast<float*>(Y)[idx] = v;
    } else if constexpr (DT == TLG_F16) {
        static_cast<_Float16*>(Y)[idx] = (_Float16)v;  // v_cvt_f16_f32: round to nearest even
    } else {
        static_cast<uint16_t*>(Y)[idx] = f32_to_bf16_rne(v);
    }
}

// 16 bytes of output from 16 / sizeof(element) fp32 values (same rounding as store_out).
template <int DT> __device__ inline u32x4 pack16(const float* v) {
    u32x4 o;
    if constexpr (DT == TLG_F32) {
#pragma unroll
        for (int u = 0; u < 4; ++u) o[u] = __float_as_uint(v[u]);
    } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) o[u] = pack2<DT>(v[2 * u], v[2 * u + 1]);
    }
    return o;
}

template <int DT> __device__ inline float load_elem(const void* p, int64_t idx) {
    return Elem<DT>::to_f32(static_cast<const typename Elem<DT>::storage*>(p)[idx]);
}

// EPC consecutive bias values from n on (n a multiple of EPC, the pointer
// 16-byte aligned) as fp32, in one 8- or 16-byte load.
template <int DT, int EPC> __device__ inline void load_bias_run(const void* bias, int n, float* b) {
    using St = typename Elem<DT>::storage;
    constexpr int BYTES = EPC * (int)sizeof(St);
    const St* p = static_cast<const St*>(bias) + n;
    if constexpr (BYTES == 16 && DT == TLG_F32) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
        for (int u = 0; u < 4; ++u) b[u] = __uint_as_float(w[u]);
    } else if constexpr (DT != TLG_F32 && (BYTES == 16 || BYTES == 8)) {
        constexpr int NW = BYTES / 4;
        uint32_t w[NW];
        if constexpr (NW == 4) {
            const u32x4 x = *reinterpret_cast<const u32x4*>(p);
            w[0] = x[0], w[1] = x[1], w[2] = x[2], w[3] = x[3];
        } else {
            const u32x2 x = *reinterpret_cast<const u32x2*>(p);
            w[0] = x[0], w[1] = x[1];
        }
#pragma unroll
        for (int u = 0; u < NW; ++u) {
            b[2 * u] = Elem<DT>::to_f32((uint16_t)(w[u] & 0xffffu));
            b[2 * u + 1] = Elem<DT>::to_f32((uint16_t)(w[u] >> 16));
        }
    } else {
#pragma unroll
        for (int u = 0; u < EPC; ++u) b[u] = load_elem<DT>(bias, n + u);
    }
}

// The inverse of pack16: 16 bytes of stored output as 16 / sizeof(element) fp32 values.
template <int DT> __device__ inline void unpack16(u32x4 w, float* v) {
    if constexpr (DT == TLG_F32) {
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = __uint_as_float(w[u]);
    } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            v[2 * u] = Elem<DT>::to_f32((uint16_t)(w[u] & 0xffffu));
            v[2 * u + 1] = Elem<DT>::to_f32((uint16_t)(w[u] >> 16));
        }
    }
}

// ---- fused epilogue ----------------------------------------------------------------
// Bias first, then the tanh form of GELU, evaluated in fp32.
// tanh from its exponential identity tanh(u) = 1 - 2 / (e^(2u) + 1), with the
// hardware base-2 exponential and reciprocal (each within about 1 ulp): e^(2u)
// overflows to +inf or underflows to 0 for large |u|, which gives exactly ±1,
// and NaN propagates.  Near u = 0 the subtraction cancels, leaving an absolute
// error of a few 1e-8, which GELU's factor y/2 keeps far below fp32 parity.
__device__ inline float tanh_fast(float u) {
    const float e = __builtin_amdgcn_exp2f(u * 2.8853900817779268f);  // 2/ln(2): 2^(2u·log2 e) = e^(2u)
    return 1.0f - 2.0f * __builtin_amdgcn_rcpf(e + 1.0f);
}

__device__ inline float gelu_tanh(float y) {
    const float c = 0.7978845608028654f;  // sqrt(2/pi)
    const float u = c * (y + 0.044715f * y * y * y);
    return 0.5f * y * (1.0f + tanh_fast(u));
}

template <uint32_t EPI> __device__ inline float epilogue(float acc, float b) {
    float y = acc;
    if constexpr ((EPI & TLG_EPI_BIAS) != 0) y += b;
    if constexpr ((EPI & TLG_EPI_GELU_TANH) != 0) y = gelu_tanh(y);
    return y;
}

// ---- 16-byte global loads --------------------------------------------------------
__device__ inline u32x4 ldg16(const void* p) { return *static_cast<const u32x4*>(p); }

// Raw buffer loads: a uniform 128-bit descriptor (base, byte count) in scalar
// registers, a per-lane 32-bit byte offset and a uniform 32-bit offset.  A
// kernel that issues many loads from one operand then holds one vector
// register of address instead of a 64-bit address per load.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ u32x4 buffer_load16(i32x4 rsrc, uint32_t voffset, int soffset, int aux) __asm(
    "llvm.amdgcn.raw.buffer.load.v4i32");
__device__ void buffer_store16(u32x4 v, i32x4 rsrc, uint32_t voffset, int soffset, int aux) __asm(
    "llvm.amdgcn.raw.buffer.store.v4i32");
// Cache-policy operand of the buffer accesses: device scope (sc1).  A store
// with it writes through this XCD's L2, and a load with it does not take a
// line this XCD's L2 may hold from before, so the two exchange data between
// workgroups on different XCDs without an L2 write-back or invalidate (the
// access form of a relaxed device-scope atomic on gfx950).
constexpr int kAuxDevice = 16;
// Descriptor for the bytes [p, p + bytes), bytes < 2^31: every field is read
// from the first lane (the arguments are uniform by construction, and this
// keeps the descriptor in scalar registers), stride 0, 32-bit data format.
__device__ inline i32x4 buffer_rsrc(const void* p, int64_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));
    r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
    r[3] = 0x00020000;
    return r;
}

// ---- LDS transpose reads (ds_read_b64_tr_b16) ----------------------------------------
// Every lane names 8 bytes (four 16-bit elements) of LDS; within each group of
// 16 lanes, lane l receives element l % 4 of the 8 bytes named by lanes
// 4j + l/4, j = 0..3 (layout measured on gfx950).  Pointed at four rows of a
// row-major tile, four lanes per row and four elements apart, the group reads
// a 4×16 block and each lane receives one column of it: four consecutive rows.
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ inline u32x2 lds_read_tr16(const void* p) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(const_cast<void*>(p))));
}

// ---- MFMA wrappers -----------------------------------------------------------------
// 16x16 output block, fp32 accumulate.
__device__ inline f32x4 mfma16_f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
template <int DT> __device__ inline f32x4 mfma16_16bit(u32x4 a, u32x4 b, f32x4 c) {
    if constexpr (DT == TLG_F16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
// 32x32 output block.
__device__ inline f32x16 mfma32_f32(float a, float b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}
template <int DT> __device__ inline f32x16 mfma32_16bit(u32x4 a, u32x4 b, f32x16 c) {
    if constexpr (DT == TLG_F16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// ---- host-side dispatch helpers ----------------------------------------------------
template <int V> using ic = std::integral_constant<int, V>;

// Only the compile-time part of the flags selects a kernel; the residual is a
// run-time argument.
template <class F> inline int with_epi(uint32_t epi, F&& f) {
    switch (epi & kEpiKernel) {
    case 0: return f(ic<0>{});
    case TLG_EPI_BIAS: return f(ic<TLG_EPI_BIAS>{});
    case TLG_EPI_GELU_TANH: return f(ic<TLG_EPI_GELU_TANH>{});
    default: return f(ic<TLG_EPI_BIAS | TLG_EPI_GELU_TANH>{});
    }
}

// The five supported (in, out) pairs.
template <class F> inline int with_types(int in_dt, int out_dt, F&& f) {
    if (in_dt == TLG_F32) return f(ic<TLG_F32>{}, ic<TLG_F32>{});
    if (in_dt == TLG_F16) {
        if (out_dt == TLG_F16) return f(ic<TLG_F16>{}, ic<TLG_F16>{});
        return f(ic<TLG_F16>{}, ic<TLG_F32>{});
    }
    if (out_dt == TLG_BF16) return f(ic<TLG_BF16>{}, ic<TLG_BF16>{});
    return f(ic<TLG_BF16>{}, ic<TLG_F32>{});
}

template <class F> inline int with_layout(int layout, F&& f) {
    switch (layout) {
    case TLG_NK: return f(ic<TLG_NK>{});
    case TLG_KN: return f(ic<TLG_KN>{});
    case TLG_AT_NK: return f(ic<TLG_AT_NK>{});
    default: return f(ic<TLG_AT_KN>{});
    }
}

int check_launch(const char* what);

}  // namespace tlg
