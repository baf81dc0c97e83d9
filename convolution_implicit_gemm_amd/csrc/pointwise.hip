// 1x1x1 convolution (a plain GEMM over voxels) as an HBM-bound stream on gfx950.
//
// y[m][co] = bias[co] (+ res[m][co]) + sum_ci x[m][ci] * w[co][ci] with no
// padding: every output voxel reads exactly its own input row.  At 256 -> 128
// channels the arithmetic intensity is ~85 flop/byte, far below the MI355X
// ridge, so the kernel is designed around moving bytes:
//  * persistent blocks, each streaming tiles of input rows through a
//    bank-swizzled LDS ring with buffer_load ... lds (no VGPR staging): up to
//    128 output channels, 4 waves and two or more blocks per CU with 64-row
//    tiles in a 64 KB ring; above, 8 waves and one block per CU; at 512
//    input channels 32-row tiles in a 128 KB ring;
//  * each wave keeps its 32 output channels x all Cin of weights in VGPRs as
//    MFMA A-fragments, loaded once per block;
//  * every tile gets its own buffer resource spanning exactly its valid rows,
//    so rows past M read as zeros through the range check;
//  * fp16 MFMA 32x32x16 with fp32 accumulation; bias / residual added in fp32,
//    one RNE rounding; the rounded tile is staged in LDS so that every store
//    is a 16-byte piece of a whole output row.
// Loads and stores share one counter on gfx9; the per-tile wait counts only
// the loads issued after the tile's own, which loads retire in order.
#include "c3d_internal.h"
#include "elem16.h"

namespace c3d {

typedef _Float16 pw_half8 __attribute__((ext_vector_type(8)));
typedef _Float16 pw_half4 __attribute__((ext_vector_type(4)));
typedef float pw_f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void pw_lds_void;

#if defined(__HIP_DEVICE_COMPILE__)
typedef __amdgpu_buffer_rsrc_t pw_rsrc;
#else
struct pw_rsrc {
    uint32_t w[4];
};
#endif

namespace {

__device__ __forceinline__ pw_rsrc pw_make_rsrc(const void *base, uint32_t bytes) {
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
#else
    (void)base;
    (void)bytes;
    return pw_rsrc{};
#endif
}

// Cache policy 2 (nt): the input is streamed once.  Measured on the 256 -> 128
// stage: 0.283 ms against 0.300 ms with the default policy; non-temporal
// output stores, by contrast, measured 4% slower and are not used.
__device__ __forceinline__ void pw_dma16(pw_rsrc r, char *lds, uint32_t voff) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (pw_lds_void *)lds, 16, voff, 0, 0, 2);
#else
    (void)r;
    (void)lds;
    (void)voff;
#endif
}

// Wait until at most N vector-memory operations of this wave are in flight and
// its LDS traffic is done, then meet the other waves.  Loads retire in issue
// order among themselves, so "at most N" with N counting only the loads issued
// after a tile's loads guarantees that tile has landed, whatever the order in
// which the stores in between complete.
template <int N>
__device__ __forceinline__ void pw_wait_and_barrier() {
    static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit counter");
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// 16-byte chunk swizzle within a row of CPR chunks: 32 consecutive rows read at
// one logical chunk land on distinct banks in every 8- and 16-lane group.
template <int CPR>
__device__ __forceinline__ int pw_swz(int row) {
    if constexpr (CPR >= 16)
        return row & 15;
    else
        return (row ^ ((row >> 3) & 1)) & 7;
}

// Voxels per tile: 64, or 32 at 512 input channels, where a 64-row tile is
// 64 KiB and only two would fit the ring.
template <int CIN>
constexpr int pw_rows() {
    return CIN == 512 ? 32 : 64;
}
// Waves per block, each owning 32 output channels: 4 up to 128 output
// channels, 8 above, so that one block row covers up to 256 channels and the
// input is streamed once (with 4 waves a 512 -> 256 conv streamed it twice and
// ran at a third of the HBM rate).
constexpr int pw_waves(int32_t cout) { return cout > 128 ? 8 : 4; }

// Input ring depth: about 64 KB of tiles per block, at most 8; 128 KB at 512
// input channels (one block per CU).
template <int CIN>
constexpr int pw_ring() {
    if constexpr (CIN == 512) return 4;
    constexpr int tile = pw_rows<CIN>() * CIN * 2;
    constexpr int nb = 64 * 1024 / tile;
    return nb > 8 ? 8 : (nb < 2 ? 2 : nb);
}

// Whether a block waits for the tile it just prefetched before computing the
// current one.  Measured on 33 frames of 256x256 (identical outputs): at
// 256 -> 128, with two blocks per CU and a two-tile ring, computing only
// after the prefetch has landed runs at 0.287-0.295 ms against 0.304-0.315 ms
// with the prefetch in flight during the MFMAs; every other configuration is
// 7-21% faster with it in flight.
template <int CIN, int NWV>
constexpr bool pw_serial() {
    return CIN == 256 && NWV == 4;
}

template <int CIN, int NWV, typename E>
__global__ __launch_bounds__(64 * NWV, NWV == 4 ? 2 : 1) void pointwise_kernel(PwParams p) {
    constexpr int RB = CIN * 2;                 // bytes per input row
    constexpr int CPR = CIN / 8;                // 16-byte chunks per row
    constexpr int BM = pw_rows<CIN>();          // rows per tile
    constexpr int NB = pw_ring<CIN>();          // ring depth
    constexpr int TILE_BYTES = BM * RB;
    constexpr int RPI = 1024 / RB;              // rows per 1 KiB load instruction
    constexpr int NI = TILE_BYTES / 1024 / NWV;  // load instructions per wave per tile
    constexpr int KF = CIN / 16;                // MFMA k-steps
    constexpr int SUB = BM / 32;                // 32-voxel sub-tiles per tile
    static_assert(BM % 32 == 0, "tiles of whole 32-voxel sub-tiles");
    static_assert(RB <= 1024 && 1024 % RB == 0 && NI >= 1 && (TILE_BYTES / 1024) % NWV == 0,
                  "CIN in {64, 128, 256, 512}, whole load instructions per wave");

    // One LDS array: the input ring, then the output staging.  With two
    // __shared__ arrays the compiler tracks the global->LDS loads per array and
    // waits for all of them (vmcnt(0)) before the first read of the ring, which
    // serialises every prefetch with the MFMAs of the current tile.
    __shared__ __attribute__((aligned(1024))) char smem[NB * TILE_BYTES + NWV * BM * 64];
    char *const obuf = smem + NB * TILE_BYTES;

    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int co0 = blockIdx.y * (32 * NWV) + wv * 32;
    const bool live = co0 < p.Cout;  // wave-uniform
    const int rrow = lane & 31, rhi = lane >> 5;

    // weights of this wave's 32 output channels, as A-fragments for every k-step
    pw_half8 wf[KF];
#pragma unroll
    for (int f = 0; f < KF; ++f) {
        if (live)
            wf[f] = *reinterpret_cast<const pw_half8 *>(p.w + (int64_t)(co0 + rrow) * CIN + 16 * f + 8 * rhi);
        else
            wf[f] = pw_half8{};
    }

    // per-lane tile-relative source offsets of this wave's load instructions
    uint32_t voff[NI];
#pragma unroll
    for (int j = 0; j < NI; ++j) {
        const int q = j * NWV + wv;
        const int row = q * RPI + lane / CPR;
        const int c = (lane % CPR) ^ pw_swz<CPR>(row);
        voff[j] = (uint32_t)(row * RB + c * 16);
    }
    int koff[KF];
#pragma unroll
    for (int f = 0; f < KF; ++f) koff[f] = rrow * RB + (((2 * f + rhi) ^ pw_swz<CPR>(rrow)) * 16);

    // bias of this lane's 16 output channels, once: loads inside the loop would
    // sit between the prefetched tiles in issue order and lengthen every wait
    float bv[4][4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        pw_half4 b4 = {};
        if (p.bias && live) b4 = *reinterpret_cast<const pw_half4 *>(p.bias + co0 + 8 * g + 4 * rhi);
#pragma unroll
        for (int e = 0; e < 4; ++e) bv[g][e] = to_f32<E>(b4[e]);
    }

    const int M = (int)p.M;
    const int ntiles = (M + BM - 1) / BM;
    // Tiles past the end are fetched as empty ranges (every lane reads zeros),
    // so every wave issues the same number of loads per tile.
    auto issue = [&](int tile, int buf) {
        const int m0 = tile * BM;
        const int rows = tile < ntiles ? (M - m0 < BM ? M - m0 : BM) : 0;
        const pw_rsrc r = pw_make_rsrc(p.x + (int64_t)(tile < ntiles ? m0 : 0) * CIN, (uint32_t)(rows * RB));
        char *sb = smem + buf * TILE_BYTES;
#pragma unroll
        for (int j = 0; j < NI; ++j) pw_dma16(r, sb + (j * NWV + wv) * 1024, voff[j]);
    };

    const int step = (int)gridDim.x;
    int tile = blockIdx.x;
    // prologue: tiles 0..NB-2 of this block
#pragma unroll
    for (int k = 0; k < NB - 1; ++k) issue(tile + k * step, k);
    int buf = 0;
    for (; tile < ntiles; tile += step) {
        // this tile landed; everyone is done with the buffer refilled next
        pw_wait_and_barrier<(NB - 2) * NI>();
        // this tile's residual, fetched before the next tile's loads: loads
        // retire in order, so waiting for it in the epilogue leaves those in
        // flight (fetched after them, it would drain the ring)
        const int m0 = tile * BM;
        pw_half4 rv[SUB][4];
        if (p.res && live) {
#pragma unroll
            for (int u = 0; u < SUB; ++u)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int vrow = u * 32 + rrow;
                    rv[u][g] = m0 + vrow < M ? *reinterpret_cast<const pw_half4 *>(
                                                   p.res + (int64_t)(m0 + vrow) * p.Cout + co0 + 8 * g + 4 * rhi)
                                             : pw_half4{};
                }
        }
        issue(tile + (NB - 1) * step, buf == 0 ? NB - 1 : buf - 1);
        if constexpr (pw_serial<CIN, NWV>()) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        const char *sb = smem + buf * TILE_BYTES;
        buf = buf + 1 == NB ? 0 : buf + 1;
        if (!live) continue;
        pw_f32x16 acc[SUB];
#pragma unroll
        for (int u = 0; u < SUB; ++u)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[u][e] = 0.0f;
#pragma unroll
        for (int f = 0; f < KF; ++f) {
#pragma unroll
            for (int u = 0; u < SUB; ++u) {
                const pw_half8 b = *reinterpret_cast<const pw_half8 *>(sb + u * 32 * RB + koff[f]);
                acc[u] = mfma_32x32x16<E>(wf[f], b, acc[u]);
            }
        }
        // epilogue: + bias (+ residual) in fp32 and one RNE rounding in registers,
        // then through LDS so that the block writes whole output rows with
        // 16-byte stores (scattered 8-byte stores of 256-byte rows waste most of
        // each memory transaction).  Lane holds channels co0 + 8g + 4*(lane/32) + e
        // of voxel 32u + lane%32.
        char *ob = obuf + wv * (BM * 64);  // this wave's [BM voxels][32 ch] fp16, row-swizzled
#pragma unroll
        for (int g = 0; g < 4; ++g) {
#pragma unroll
            for (int u = 0; u < SUB; ++u) {
                const int vrow = u * 32 + rrow;
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = acc[u][4 * g + e] + bv[g][e];
                if (p.res) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] += to_f32<E>(rv[u][g][e]);
                }
                pw_half4 h;
#pragma unroll
                for (int e = 0; e < 4; ++e) h[e] = from_f32<E>(v[e]);
                // 8-byte unit (2g + rhi) of the 64-byte row, xor-swizzled by the row
                *reinterpret_cast<pw_half4 *>(ob + vrow * 64 + (((2 * g + rhi) ^ (vrow & 7)) * 8)) = h;
            }
        }
        // each lane stores 16 bytes; 4 lanes cover this wave's 64-byte slice of a row
#pragma unroll
        for (int q = 0; q < BM / 16; ++q) {
            const int vrow = q * 16 + (lane >> 2), part = lane & 3;
            const int m = m0 + vrow;
            const int u0 = (2 * part) ^ (vrow & 7), u1 = (2 * part + 1) ^ (vrow & 7);
            const pw_half4 lo = *reinterpret_cast<const pw_half4 *>(ob + vrow * 64 + u0 * 8);
            const pw_half4 hi = *reinterpret_cast<const pw_half4 *>(ob + vrow * 64 + u1 * 8);
            if (m < M) {
                pw_half8 v;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[e] = lo[e];
                    v[4 + e] = hi[e];
                }
                *reinterpret_cast<pw_half8 *>(p.y + (int64_t)m * p.Cout + co0 + part * 8) = v;
            }
        }
    }
    pw_wait_and_barrier<0>();  // drain the prefetches past the end before LDS is released
}

template <int CIN>
PwGeom pw_geom(int32_t cout, int64_t m) {
    // persistent blocks, all resident: as many as LDS allows up to four per CU
    // with 4 waves; one per CU with 8 waves (its launch bounds, which keep the
    // 512-channel weights in registers)
    const int nwv = pw_waves(cout);
    const int lds = pw_ring<CIN>() * pw_rows<CIN>() * CIN * 2 + nwv * pw_rows<CIN>() * 64;
    const int by_lds = 160 * 1024 / lds;
    const int per_cu = nwv == 8 ? 1 : (by_lds < 4 ? by_lds : 4);
    const int64_t ntiles = (m + pw_rows<CIN>() - 1) / pw_rows<CIN>();
    const int64_t cap = 256 * (int64_t)per_cu;
    PwGeom g;
    g.rows = pw_rows<CIN>();
    g.ring = pw_ring<CIN>();
    g.waves = nwv;
    g.grid_x = ntiles < cap ? ntiles : cap;
    g.grid_y = (cout + 32 * nwv - 1) / (32 * nwv);
    return g;
}

template <int CIN, int NWV>
void launch_pw_w(const PwParams &p, dim3 grid, hipStream_t s) {
    if (p.bf16)
        hipLaunchKernelGGL((pointwise_kernel<CIN, NWV, __bf16>), grid, dim3(64 * NWV), 0, s, p);
    else
        hipLaunchKernelGGL((pointwise_kernel<CIN, NWV, _Float16>), grid, dim3(64 * NWV), 0, s, p);
}

template <int CIN>
hipError_t launch_pw(const PwParams &p, hipStream_t s) {
    const PwGeom g = pw_geom<CIN>(p.Cout, p.M);
    const dim3 grid((unsigned)g.grid_x, (unsigned)g.grid_y);
    if (g.waves == 8)
        launch_pw_w<CIN, 8>(p, grid, s);
    else
        launch_pw_w<CIN, 4>(p, grid, s);
    return hipGetLastError();
}

}  // namespace

bool pointwise_supported(int32_t cin, int32_t cout) {
    return (cin == 64 || cin == 128 || cin == 256 || cin == 512) && cout % 32 == 0;
}

PwGeom pointwise_geometry(int32_t cin, int32_t cout, int64_t m) {
    switch (cin) {
        case 64: return pw_geom<64>(cout, m);
        case 128: return pw_geom<128>(cout, m);
        case 256: return pw_geom<256>(cout, m);
        default: return pw_geom<512>(cout, m);
    }
}

hipError_t launch_pointwise(const PwParams &p, hipStream_t s) {
    switch (p.Cin) {
        case 64: return launch_pw<64>(p, s);
        case 128: return launch_pw<128>(p, s);
        case 256: return launch_pw<256>(p, s);
        case 512: return launch_pw<512>(p, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace c3d
