// Implicit-GEMM fp16 3D convolution for gfx950 (MI355X).
//
// The conv is the GEMM  Y[m][co] = sum_k A[m][k] * B[co][k]  with
//   m  = output voxel (n, to, ho, wo), row-major over the NDHWC output,
//   co = output channel,
//   k  = (tau, r, s, ci), ci fastest,
// where A is never built: each K-slice of an output row is gathered straight
// from the NDHWC input, because for a fixed voxel and tap the Cin channels
// are contiguous.  This is the implicit-GEMM lowering described in the Draw
// Things engineering feed (post on the Codex-written Metal conv3d shaders for
// the LTX-2.3 video VAE, implicit-GEMM paragraph); the kernel here is written
// for CDNA4, not after any shader.
//
// gfx950 design:
//  * Matrix cores: v_mfma_f32_32x32x16_f16 (fp16 products, fp32 accumulate).
//    The MFMA "A" operand is the weight tile (rows = output channels) and the
//    "B" operand the gathered activations (columns = voxels), so each lane's
//    accumulators hold 4 consecutive output channels of one voxel: the
//    epilogue writes NDHWC rows directly.
//  * Global -> LDS with global_load_lds_dwordx4 (16 B per lane straight into
//    LDS, no VGPR staging).  A load instruction fills 1 KiB of LDS linearly by
//    lane, so the bank swizzle (16-byte chunk index XOR a function of the row)
//    is applied on the global side: each lane fetches the chunk that belongs
//    at its LDS slot.
//  * Padding is resolved in address arithmetic once per tap: a lane whose
//    source voxel lies outside H/W (or outside T with zero temporal padding)
//    reads a 16-byte zero line instead; replicate temporal padding clamps the
//    frame index.  Rows past M, channels past Cout and (on the tail variant)
//    channels past Cin read the same zero line.
//  * STAGES-deep ring of LDS buffers; one s_waitcnt vmcnt(N) + s_barrier per
//    K-iteration.  __syncthreads() is avoided on purpose: its release fence
//    waits for every outstanding load, which would drain the prefetch ring.
//  * Workgroups are renumbered so each XCD (workgroup id mod 8) walks a
//    contiguous range of tiles; tiles sharing input rows then share an L2.
#include "c3d_internal.h"

namespace c3d {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

// Read by every padded tap, out-of-range row and channel tail.  Never written.
__device__ __attribute__((aligned(256))) uint32_t g_zero_line[64];

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

template <int N>
__device__ __forceinline__ void wait_loads_and_barrier() {
    static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit counter");
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

template <int BM, int BN, int BK, int WM, int WN, int STAGES, bool TAIL>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64) void conv3d_igemm_kernel(ConvParams p) {
    constexpr int NWM = BM / WM, NWN = BN / WN, NW = NWM * NWN;
    constexpr int RB = BK * 2;        // bytes per LDS row
    constexpr int CPR = BK / 8;       // 16-byte chunks per row
    constexpr int RPI = 1024 / RB;    // rows filled by one 1 KiB load instruction
    constexpr int QA = BM / RPI;      // activation load instructions per stage
    constexpr int QB = BN / RPI;      // weight load instructions per stage
    constexpr int LA = (QA + NW - 1) / NW, LB = (QB + NW - 1) / NW;
    constexpr int TM = WM / 32, TN = WN / 32, KS = BK / 16;
    constexpr int B_OFF = BN * RB;                  // activations follow the weights
    constexpr int STAGE_BYTES = (BM + BN) * RB;
    static_assert(BM % RPI == 0 && BN % RPI == 0, "tile rows must fill whole load instructions");
    static_assert(STAGES == 2 || (QA % NW == 0 && QB % NW == 0),
                  "a deep ring needs the same load count on every wave");
    static_assert(STAGES * STAGE_BYTES <= 160 * 1024, "LDS is 160 KiB per CU");

    __shared__ __attribute__((aligned(1024))) char smem[STAGES * STAGE_BYTES];

    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    // XCD-aware renumbering: XCD x = blockIdx mod 8 gets a contiguous tile range.
    const int64_t nblk = p.tiles;
    const int64_t bid = blockIdx.x;
    const int64_t per = nblk >> 3, rem = nblk & 7;
    const int xcd = (int)(bid & 7);
    const int64_t tile = xcd * per + (xcd < rem ? xcd : rem) + (bid >> 3);
    const int mt = (int)(tile / p.n_tiles), nt = (int)(tile - (int64_t)mt * p.n_tiles);
    const int64_t m0 = (int64_t)mt * BM;
    const int n0 = nt * BN;

    const int T = p.T, H = p.H, W = p.W, Cin = p.Cin;
    const int HW = H * W;

    // ---- per-lane gather slots: one output row per activation load instruction
    const int lrow = lane / CPR, lchunk = lane % CPR;
    int a_vb[LA], a_t[LA], a_h[LA], a_w[LA], a_c8[LA];
#pragma unroll
    for (int j = 0; j < LA; ++j) {
        const int row = (j * NW + wv) * RPI + lrow;
        a_c8[j] = (lchunk ^ swz<BK>(row)) * 8;
        const int64_t m = m0 + row;
        if (m < p.M) {
            const int wo = (int)(m % p.Wo);
            const int64_t r1 = m / p.Wo;
            const int ho = (int)(r1 % p.Ho);
            const int64_t r2 = r1 / p.Ho;
            const int to = (int)(r2 % p.To);
            const int n = (int)(r2 / p.To);
            a_t[j] = to;
            a_h[j] = ho;
            a_w[j] = wo;
            a_vb[j] = ((n * T + to) * H + ho) * W + wo;
        } else {
            a_t[j] = 0;
            a_h[j] = 1 << 20;  // never inside [0, H): the row reads zeros
            a_w[j] = 0;
            a_vb[j] = 0;
        }
    }
    const char *b_ptr[LB];
#pragma unroll
    for (int j = 0; j < LB; ++j) {
        const int row = (j * NW + wv) * RPI + lrow;
        const int co = n0 + row;
        const int c8 = (lchunk ^ swz<BK>(row)) * 8;
        b_ptr[j] = co < p.Cout ? reinterpret_cast<const char *>(p.w + (int64_t)co * p.K + c8) : nullptr;
    }
    int b_c8[LB];
#pragma unroll
    for (int j = 0; j < LB; ++j) b_c8[j] = (lchunk ^ swz<BK>((j * NW + wv) * RPI + lrow)) * 8;

    const char *a_ptr[LA];
    auto set_tap = [&](int tau, int r, int s) {
#pragma unroll
        for (int j = 0; j < LA; ++j) {
            int ts = a_t[j] + tau - p.ptf;
            bool ok;
            if (p.replicate) {
                ts = ts < 0 ? 0 : (ts > T - 1 ? T - 1 : ts);
                ok = true;
            } else {
                ok = (unsigned)ts < (unsigned)T;
            }
            const int hs = a_h[j] + r - p.ph, ws = a_w[j] + s - p.pw;
            ok = ok && (unsigned)hs < (unsigned)H && (unsigned)ws < (unsigned)W;
            const int vox = a_vb[j] + (ts - a_t[j]) * HW + (r - p.ph) * W + (s - p.pw);
            a_ptr[j] = ok ? reinterpret_cast<const char *>(p.x + (int64_t)vox * Cin + a_c8[j]) : nullptr;
        }
    };

    const char *zero = reinterpret_cast<const char *>(g_zero_line);
    auto issue = [&](int stage, int tap, int ci0) {
        char *sb = smem + stage * STAGE_BYTES;
        const int64_t kofs = ((int64_t)tap * Cin + ci0) * 2;
#pragma unroll
        for (int j = 0; j < LB; ++j) {
            const int q = j * NW + wv;
            if (QB % NW == 0 || q < QB) {
                const bool ok = b_ptr[j] != nullptr && (!TAIL || ci0 + b_c8[j] < Cin);
                const char *src = ok ? b_ptr[j] + kofs : zero;
                __builtin_amdgcn_global_load_lds(src, (lds_void *)(sb + q * 1024), 16, 0, 0);
            }
        }
#pragma unroll
        for (int j = 0; j < LA; ++j) {
            const int q = j * NW + wv;
            if (QA % NW == 0 || q < QA) {
                const bool ok = a_ptr[j] != nullptr && (!TAIL || ci0 + a_c8[j] < Cin);
                const char *src = ok ? a_ptr[j] + ci0 * 2 : zero;
                __builtin_amdgcn_global_load_lds(src, (lds_void *)(sb + B_OFF + q * 1024), 16, 0, 0);
            }
        }
    };

    // ---- load-side iteration state (runs STAGES-1 iterations ahead)
    int ld_it = 0, ld_ci = 0, ld_tap = 0, ld_tau = 0, ld_r = 0, ld_s = 0;
    set_tap(0, 0, 0);
    auto advance = [&]() {
        ++ld_it;
        ld_ci += BK;
        if (ld_ci >= Cin) {
            ld_ci = 0;
            ++ld_tap;
            if (++ld_s == p.kw) {
                ld_s = 0;
                if (++ld_r == p.kh) {
                    ld_r = 0;
                    ++ld_tau;
                }
            }
            if (ld_it < p.niter) set_tap(ld_tau, ld_r, ld_s);
        }
    };

    // ---- per-lane LDS read offsets for the MFMA fragments
    const int rrow = lane & 31, rhi = lane >> 5;
    const int wmi = wv / NWN, wni = wv % NWN;
    const int a_frag0 = wni * WN * RB;              // weights (MFMA A)
    const int b_frag0 = B_OFF + wmi * WM * RB;      // activations (MFMA B)
    int koff[KS];
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) koff[kk] = rrow * RB + (((2 * kk + rhi) ^ swz<BK>(rrow)) * 16);

    f32x16 acc[TN][TM];
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    constexpr int LOADS = LA + LB;  // per wave per stage (uniform when STAGES > 2)
    const int niter = p.niter;
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s) {
        if (ld_it < niter) {
            issue(s, ld_tap, ld_ci);
            advance();
        }
    }

    for (int it = 0; it < niter; ++it) {
        if (it + STAGES - 2 < niter)
            wait_loads_and_barrier<(STAGES - 2) * LOADS>();
        else
            wait_loads_and_barrier<0>();
        if (ld_it < niter) {
            issue(ld_it % STAGES, ld_tap, ld_ci);
            advance();
        }
        const char *sb = smem + (it % STAGES) * STAGE_BYTES;
        // Fragments of k-step kk+1 are read while the MFMAs of kk issue.
        half8_t af[2][TN], bf[2][TM];
#pragma unroll
        for (int i = 0; i < TN; ++i)
            af[0][i] = *reinterpret_cast<const half8_t *>(sb + a_frag0 + i * 32 * RB + koff[0]);
#pragma unroll
        for (int j = 0; j < TM; ++j)
            bf[0][j] = *reinterpret_cast<const half8_t *>(sb + b_frag0 + j * 32 * RB + koff[0]);
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            const int cur = kk & 1, nxt = cur ^ 1;
            if (kk + 1 < KS) {
#pragma unroll
                for (int i = 0; i < TN; ++i)
                    af[nxt][i] = *reinterpret_cast<const half8_t *>(sb + a_frag0 + i * 32 * RB + koff[kk + 1]);
#pragma unroll
                for (int j = 0; j < TM; ++j)
                    bf[nxt][j] = *reinterpret_cast<const half8_t *>(sb + b_frag0 + j * 32 * RB + koff[kk + 1]);
            }
#pragma unroll
            for (int i = 0; i < TN; ++i)
#pragma unroll
                for (int j = 0; j < TM; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[cur][i], bf[cur][j], acc[i][j], 0, 0, 0);
        }
        // Schedule: the first k-step's reads, then the remaining reads spread
        // evenly between MFMAs, so the matrix pipe never waits on LDS.
        constexpr int READS = TN + TM, MFMAS = TN * TM;
        constexpr int PF_READS = (KS - 1) * READS;            // prefetched reads
        constexpr int PF_MFMAS = (KS - 1) * MFMAS;            // MFMAs they hide behind
        constexpr int GAP = PF_READS ? (PF_MFMAS / PF_READS > 0 ? PF_MFMAS / PF_READS : 1) : 1;
        __builtin_amdgcn_sched_group_barrier(0x100, READS, 0);
#pragma unroll
        for (int q = 0; q < PF_READS; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, GAP, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, KS * MFMAS - GAP * PF_READS, 0);
    }

    // ---- epilogue: + bias (+ residual) in fp32, one RNE rounding, NDHWC store.
    // Lane holds, for sub-tile (i, j) and register 4g+e: channel
    // co = 8g + 4*(lane/32) + e of the sub-tile, voxel m = lane % 32.
#pragma unroll
    for (int i = 0; i < TN; ++i) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int co = n0 + wni * WN + i * 32 + 8 * g + 4 * rhi;
            if (co >= p.Cout) continue;
            f32x4 bv = {0.0f, 0.0f, 0.0f, 0.0f};
            if (p.bias) {
                const half4_t b4 = *reinterpret_cast<const half4_t *>(p.bias + co);
#pragma unroll
                for (int e = 0; e < 4; ++e) bv[e] = (float)b4[e];
            }
#pragma unroll
            for (int j = 0; j < TM; ++j) {
                const int64_t m = m0 + wmi * WM + j * 32 + rrow;
                if (m >= p.M) continue;
                const int64_t o = m * p.Cout + co;
                f32x4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * g + e] + bv[e];
                if (p.res) {
                    const half4_t r4 = *reinterpret_cast<const half4_t *>(p.res + o);
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] += (float)r4[e];
                }
                half4_t h;
#pragma unroll
                for (int e = 0; e < 4; ++e) h[e] = (_Float16)v[e];
                *reinterpret_cast<half4_t *>(p.y + o) = h;
            }
        }
    }
}

template <int BM, int BN, int BK, int WM, int WN, int STAGES, bool TAIL>
hipError_t launch_igemm(const ConvParams &p, hipStream_t s) {
    constexpr int threads = (BM / WM) * (BN / WN) * 64;
    hipLaunchKernelGGL((conv3d_igemm_kernel<BM, BN, BK, WM, WN, STAGES, TAIL>), dim3((unsigned)p.tiles),
                       dim3(threads), 0, s, p);
    return hipGetLastError();
}

#define C3D_TILE(NAME, BM, BN, BK, WM, WN, ST)                                                  \
    {NAME, BM, BN, BK, ST, (BM / WM) * (BN / WN) * 64, (size_t)(ST) * ((BM) + (BN)) * (BK) * 2, \
     launch_igemm<BM, BN, BK, WM, WN, ST, false>, launch_igemm<BM, BN, BK, WM, WN, ST, true>}

static const TileCfg k_tiles[] = {
    C3D_TILE("m256n256k64s2w4", 256, 256, 64, 128, 128, 2),
    C3D_TILE("m256n256k32s4w4", 256, 256, 32, 128, 128, 4),
    C3D_TILE("m256n256k64s2w8", 256, 256, 64, 64, 128, 2),
    C3D_TILE("m256n128k64s2w4", 256, 128, 64, 128, 64, 2),
    C3D_TILE("m128n128k64s3w4", 128, 128, 64, 64, 64, 3),
    C3D_TILE("m128n64k64s2w4", 128, 64, 64, 32, 64, 2),
    C3D_TILE("m128n32k32s2w4", 128, 32, 32, 32, 32, 2),
};

const TileCfg *tile_table(int *count) {
    *count = (int)(sizeof(k_tiles) / sizeof(k_tiles[0]));
    return k_tiles;
}

// ---- temporal-tap fold for the first-frame fast path -------------------------
// With one input frame and the frame index clamped, every temporal tap reads
// that frame, so the causal 3D correlation equals a 2D one whose kernel is
// the sum of the temporal taps ("Video VAE" section of the Qwen Image post,
// Draw Things engineering feed).  Summed in fp32, rounded once.
__global__ __launch_bounds__(256) void fold_taps_kernel(const _Float16 *__restrict__ w,
                                                        _Float16 *__restrict__ w2, int32_t cout,
                                                        int32_t kt, int64_t khwc, int32_t lo,
                                                        int32_t hi) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t total8 = (int64_t)cout * khwc / 8;
    if (i >= total8) return;
    const int64_t e8 = i * 8;
    const int64_t co = e8 / khwc, e = e8 - co * khwc;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int tau = lo; tau <= hi; ++tau) {
        const half8_t v = *reinterpret_cast<const half8_t *>(w + (co * kt + tau) * khwc + e);
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] += (float)v[q];
    }
    half8_t o;
#pragma unroll
    for (int q = 0; q < 8; ++q) o[q] = (_Float16)acc[q];
    *reinterpret_cast<half8_t *>(w2 + e8) = o;
}

hipError_t launch_fold_taps(const _Float16 *w, _Float16 *w2, int32_t cout, int32_t kt, int64_t khw_cin,
                            int32_t tau_lo, int32_t tau_hi, hipStream_t s) {
    const int64_t total8 = (int64_t)cout * khw_cin / 8;
    const unsigned blocks = (unsigned)((total8 + 255) / 256);
    hipLaunchKernelGGL(fold_taps_kernel, dim3(blocks), dim3(256), 0, s, w, w2, cout, kt, khw_cin, tau_lo,
                       tau_hi);
    return hipGetLastError();
}

}  // namespace c3d
