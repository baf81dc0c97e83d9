// Device helpers shared by the implicit-GEMM conv kernels (conv3d_igemm.hip,
// conv3d_ps.hip): vector types, the LDS bank swizzle, buffer resources with
// range-checked loads, direct global->LDS loads, and the fused epilogue.
#pragma once

#include "c3d_internal.h"
#include "elem16.h"

#include <type_traits>

namespace c3d {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;


// Calls f(std::integral_constant<int, i>{}) for i = 0..N-1 (compile-time indices).
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<N, I + 1>(f);
    }
}

// Bank swizzle of 16-byte chunks within an LDS row of BK halves.  Chosen so
// that 32 consecutive rows read at one logical chunk by ds_read_b128 hit
// distinct banks in every group of 8 (128-byte) and 16 (256-byte) lanes.  It
// depends on row & 15 only, so 32-row MFMA sub-tiles share one pattern.
template <int BK>
__device__ __forceinline__ int swz(int row) {
    if constexpr (BK == 64) {
        return (row ^ ((row >> 3) & 1)) & 7;
    } else {
        static_assert(BK == 32, "BK must be 32 or 64");
        return ((row >> 1) ^ (row >> 3)) & 3;
    }
}

// Wait until at most N global->LDS loads of this wave are in flight and all of
// its LDS reads have returned, then meet the other waves.  Loads retire in
// order, so "at most N" means every older stage has landed.
template <int N>
__device__ __forceinline__ void wait_lds_and_loads() {
    static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit counter");
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Buffer resources: the device pass uses the gfx950 128-bit descriptor type;
// the host pass (which never runs these functions) sees a placeholder.
#if defined(__HIP_DEVICE_COMPILE__)
typedef __amdgpu_buffer_rsrc_t buf_rsrc;
#else
struct buf_rsrc {
    uint32_t w[4];
};
#endif

// Raw (unswizzled, stride 0) buffer over `bytes` bytes at `base`.  Loads whose
// voffset + soffset reach past `bytes` return zeros, dword by dword.
__device__ __forceinline__ buf_rsrc make_rsrc(const void *base, uint32_t bytes) {
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
#else
    (void)base;
    (void)bytes;
    return buf_rsrc{};
#endif
}

// 16 bytes per lane from base + voff + soff straight into LDS: lane i writes
// lds + 16*i (lds must be wave-uniform).  Only the device pass sees the builtin.
__device__ __forceinline__ void dma16(buf_rsrc r, char *lds, uint32_t voff, uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)lds, 16, voff, soff, 0, 0);
#else
    (void)r;
    (void)lds;
    (void)voff;
    (void)soff;
#endif
}

// Offset that is always past a buffer's record count (records stay below 2^31,
// and the scalar offsets added to it below 2^31 too, so the sum cannot wrap).
constexpr uint32_t kOOB = 0x80000000u;

// 8-byte buffer load / store (four fp16); out-of-range loads read zeros and
// out-of-range stores are dropped by the buffer unit's range check.
__device__ __forceinline__ half4_t load8(buf_rsrc r, uint32_t off) {
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_bit_cast(half4_t, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
#else
    (void)r;
    (void)off;
    return half4_t{};
#endif
}
__device__ __forceinline__ void store8(buf_rsrc r, uint32_t off, half4_t v) {
#if defined(__HIP_DEVICE_COMPILE__)
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, off, 0, 0);
#else
    (void)r;
    (void)off;
    (void)v;
#endif
}

// Epilogue of one tile: + bias (+ residual) in fp32, one RNE rounding, NDHWC
// store.  Lane holds, for sub-tile (i, j) and register 4g+e: channel
// co = 8g + 4*(lane/32) + e of the sub-tile, voxel m = lane % 32.
// Branch-free, through buffer resources over this tile's output rows (and the
// same rows of the residual, and the bias): rows past M lie past the records,
// channels past Cout get an out-of-range offset, a missing bias or residual is
// a resource of zero records; out-of-range loads read zeros and such stores
// are dropped.  The bias and residual of sub-tile row i+1 are loaded before
// the stores of row i: y aliases neither input, but the compiler cannot know
// that, and loads queued behind stores would each wait out a round trip.
template <typename E, int TN, int TM, int WN, int WM>
__device__ __forceinline__ void store_tile(const ConvParams &p, const f32x16 (&acc)[TN][TM], int m0, int bm, int n0,
                                           int wmi, int wni, int rrow, int rhi) {
    const int M = (int)p.M;
    const int rows = M - m0 < bm ? M - m0 : bm;
    const uint32_t tile_bytes = (uint32_t)rows * (uint32_t)p.Cout * 2u;
    const buf_rsrc ry = make_rsrc(p.y + (int64_t)m0 * p.Cout, tile_bytes);
    const buf_rsrc rr = make_rsrc(p.res ? p.res + (int64_t)m0 * p.Cout : p.y, p.res ? tile_bytes : 0u);
    const buf_rsrc rb = make_rsrc(p.bias ? p.bias : p.y, p.bias ? (uint32_t)p.Cout * 2u : 0u);
    auto offset = [&](int i, int g, int j) {
        const int co = n0 + wni * WN + i * 32 + 8 * g + 4 * rhi;
        const int mr = wmi * WM + j * 32 + rrow;  // row within the tile
        return co < p.Cout ? ((uint32_t)mr * (uint32_t)p.Cout + (uint32_t)co) * 2u : kOOB;
    };
    half4_t bv[2][4], rv[2][4][TM];
    auto fetch = [&](int i, int slot) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int co = n0 + wni * WN + i * 32 + 8 * g + 4 * rhi;
            bv[slot][g] = load8(rb, (uint32_t)co * 2u);
#pragma unroll
            for (int j = 0; j < TM; ++j) rv[slot][g][j] = load8(rr, offset(i, g, j));
        }
    };
    fetch(0, 0);
#pragma unroll
    for (int i = 0; i < TN; ++i) {
        if (i + 1 < TN) fetch(i + 1, (i + 1) & 1);
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int j = 0; j < TM; ++j) {
                half4_t h;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    h[e] = from_f32<E>(acc[i][j][4 * g + e] + to_f32<E>(bv[i & 1][g][e]) + to_f32<E>(rv[i & 1][g][j][e]));
                store8(ry, offset(i, g, j), h);
            }
    }
}

}  // namespace c3d
