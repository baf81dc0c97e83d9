// 16-bit element types of the kernels: fp16 (_Float16) and bf16 (__bf16).
// Tensors travel as 16-bit storage (_Float16 pointers and vectors); the
// element type E says how the bits are read.  The conversions and the MFMA
// below are the only places that depend on it.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

namespace c3d {

typedef _Float16 e16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float e32x16_t __attribute__((ext_vector_type(16)));

template <typename E>
__device__ __forceinline__ float to_f32(_Float16 raw) {
    if constexpr (std::is_same_v<E, __bf16>)
        return (float)__builtin_bit_cast(__bf16, raw);
    else
        return (float)raw;
}

// fp32 -> E with round-to-nearest-even
template <typename E>
__device__ __forceinline__ _Float16 from_f32(float v) {
    if constexpr (std::is_same_v<E, __bf16>)
        return __builtin_bit_cast(_Float16, (__bf16)v);
    else
        return (_Float16)v;
}

// v_mfma_f32_32x32x16_{f16,bf16}: 32x32 fp32 accumulator += A (32x16) * B (16x32)
template <typename E>
__device__ __forceinline__ e32x16_t mfma_32x32x16(e16x8_t a, e16x8_t b, e32x16_t c) {
#if defined(__HIP_DEVICE_COMPILE__)
    if constexpr (std::is_same_v<E, __bf16>)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                       0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
#else
    (void)a;
    (void)b;
    return c;
#endif
}

}  // namespace c3d
