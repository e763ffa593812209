// common.h -- element types, conversions and MFMA wrappers for gfx950.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lmoe {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Element loads/stores for the two storage types.  bf16 <-> f32 conversion
// rounds to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }
template <class E> __device__ __forceinline__ E from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// D[32x32] += A[32x16] * B[16x32].  Lane l holds A[l%32][8*(l/32) .. +7] and
// B[8*(l/32) .. +7][l%32]; the result register r of lane l is
// D[8*(r/4) + 4*(l/32) + r%4][l%32].
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// D[16x16] += A[16x32] * B[32x16].  Lane l holds A[l%16][8*(l/16) .. +7] and
// B[8*(l/16) .. +7][l%16]; register r of lane l is D[4*(l/16) + r][l%16].
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint4 ldg16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ uint2 ldg8(const void* p) { return *reinterpret_cast<const uint2*>(p); }
__device__ __forceinline__ uint32_t ldg4(const void* p) { return *reinterpret_cast<const uint32_t*>(p); }
__device__ __forceinline__ uint32_t ldg1(const void* p) { return *static_cast<const uint8_t*>(p); }

// 8 OCP FP8 E4M3 codes (bytes 0..7 of v) -> the 8 equal bfloat16 values
// (every E4M3 value is exact in bfloat16), with gfx950's
// v_cvt_scalef32_pk_bf16_fp8 at scale 1.  Device code only.
__device__ __forceinline__ uint4 e4m3x8_to_bf16x8(uint2 v) {
#if defined(__HIP_DEVICE_COMPILE__)
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, 1.0f, false);
    const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, 1.0f, true);
    const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, 1.0f, false);
    const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, 1.0f, true);
    return uint4{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                 __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3)};
#else
    (void)v;
    return uint4{0u, 0u, 0u, 0u};
#endif
}

// An OCP E8M0 block scale byte b (1 .. 254) as the float32 2^(b - 127).
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) { return __uint_as_float(b << 23); }

// 8 OCP E2M1 (FP4) codes -- the nibbles of v, element 0 in the low nibble of
// byte 0 -- times the block scale sc, as 8 bfloat16 (exact: an E2M1 value
// times a power of two), with gfx950's v_cvt_scalef32_pk_bf16_fp4.  Device
// code only.
__device__ __forceinline__ uint4 fp4x8_to_bf16x8(uint32_t v, float sc) {
#if defined(__HIP_DEVICE_COMPILE__)
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, sc, 0);
    const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, sc, 1);
    const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, sc, 2);
    const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, sc, 3);
    return uint4{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                 __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3)};
#else
    (void)v;
    (void)sc;
    return uint4{0u, 0u, 0u, 0u};
#endif
}

// Streaming (non-temporal) vector stores, for outputs that the kernel does
// not read back.  A GEMM tile's stores are issued in a burst at its end, and
// loads issued after them are counted behind them (one in-order vector
// memory counter): non-temporal stores are acknowledged sooner, so the next
// tile's operand loads wait less.
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void st_nt8(void* p, uint2 v) {
    __builtin_nontemporal_store(u32x2{v.x, v.y}, static_cast<u32x2*>(p));
}
__device__ __forceinline__ void st_nt16(void* p, uint4 v) {
    __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, static_cast<u32x4*>(p));
}

constexpr uint4 kZero16 = {0u, 0u, 0u, 0u};

// 4 floats as 4 bfloat16 (round to nearest even), packed in 8 bytes.
__device__ __forceinline__ uint2 pack4_bf16(const f32x4& v) {
    const bf16 b[4] = {(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
    return *reinterpret_cast<const uint2*>(b);
}

// The tiled path keeps the gate-scaled expert outputs g * y in HBM as
// IEEE half precision scaled by 2^-8: 11 significant bits (a rounding error
// of at most 2^-12 relative, 8x below bfloat16's) in the same two bytes.
// The scale moves half precision's range to [2^-6, 1.7e7] for normal values
// (below it the absolute error is at most 2^-17 / 2); larger magnitudes
// saturate at 65504 * 2^8 instead of becoming infinite.  NaN stays NaN.
constexpr float kYScale = 0x1p-8f, kYUnscale = 0x1p8f;
__device__ __forceinline__ uint2 pack4_f16_sat(f32x4 v) {
    f16 h[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float c = fabsf(v[i]) > 65504.0f ? copysignf(65504.0f, v[i]) : v[i];
        h[i] = (f16)c;
    }
    return *reinterpret_cast<const uint2*>(h);
}

__host__ __device__ constexpr int cdiv(int a, int b) { return (a + b - 1) / b; }

}  // namespace lmoe
