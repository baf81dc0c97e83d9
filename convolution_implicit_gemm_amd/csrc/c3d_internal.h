// Internal interfaces between the host-side C ABI (api.cpp) and the gfx950
// kernels.  Not installed; not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace c3d {

// Everything the implicit-GEMM kernel needs, passed by value as the kernel
// argument.  Extents are of the conv as executed (after a temporal fold the
// kernel sees kt = 1 and T = 1).
struct ConvParams {
    // Tensors are 16-bit storage: fp16, or bf16 when bf16 is set.
    const _Float16 *x;     // [N][T][H][W][Cin]
    const _Float16 *w;     // [Cout][kt][kh][kw][Cin]
    const _Float16 *bias;  // [Cout] or null
    const _Float16 *res;   // [M][Cout] or null
    _Float16 *y;           // [M][Cout]
    int32_t T, H, W, Cin, Cout;
    int32_t To, Ho, Wo;
    int32_t kt, kh, kw, ptf, ph, pw, replicate;
    int32_t K;             // kt*kh*kw*Cin
    int32_t cpt;           // channel slices: ceil(Cin / BK); the K loop is slice-major, taps fastest
    int32_t niter;         // kt*kh*kw*cpt
    int32_t m_tiles, n_tiles;
    int32_t dp_tiles;      // tiles [0, dp_tiles) run whole, one workgroup each
    int32_t sk_tiles;      // tiles [dp_tiles, dp_tiles+sk_tiles) run as sk_pieces K-pieces
    int32_t sk_pieces;
    float *partial;        // [sk_tiles*sk_pieces][BM*BN] fp32 partial tiles (workspace)
    int32_t in_vox;        // N*T*H*W input voxels
    uint32_t w_bytes;      // Cout*K*2, below 2^30
    int64_t M;             // N*To*Ho*Wo, below 2^30
    int64_t tiles;         // m_tiles*n_tiles
    int32_t bf16;          // elements are bf16 (else fp16)
    uint32_t *queue;       // counters of the dynamic tile schedule (workspace), or null: static
    int32_t grid_cap;      // dynamic schedule: at most this many workgroups (one per CU)
    // GroupNorm partial statistics of y (CONV3D_F_GN_STATS), or null: float4
    // (count, mean, M2, 0) [N][Cout/8][gn_slots] (workspace), one per
    // (sample, 8-channel chunk, M-tile of the sample, 32-voxel row group of
    // the tile): slot = (M-tile within the sample) * (BM/32) + row group.
    float4 *gn_stats;
    int32_t gn_slots;      // slots per (sample, chunk): M-tiles per sample * BM/32
    int32_t mt_per_sample; // M-tiles per sample (voxels per sample are a multiple of BM)
};

// Output voxels per tile of the row-slab kernel (conv3d_ps.hip); its
// GroupNorm statistics come in 32-voxel row groups.
constexpr int kPsBM = 256;

// Most K-pieces a split tile may be cut into (the fixup kernel loads them all
// at once).
constexpr int kMaxSplitPieces = 16;

// Largest input window, in voxels, that one tile of bm output rows can read
// (the kernel addresses it through one buffer resource with 32-bit offsets).
int64_t tile_window_voxels(const ConvParams &q, int bm);

typedef hipError_t (*ConvLaunchFn)(const ConvParams &p, hipStream_t s);

// One compiled tile configuration of the implicit-GEMM kernel.
struct TileCfg {
    const char *name;
    int bm, bn, bk, stages, threads;
    size_t lds_bytes;
    double rate;               // measured relative throughput per CU (1 = best)
    ConvLaunchFn launch_full;  // Cin % bk == 0
    ConvLaunchFn launch_tail;  // any Cin % 8 == 0 (channel tail zero-filled per tap)
    ConvLaunchFn launch_fixup; // sums the K-pieces of the split tiles, then the epilogue
    bool (*supported)(const ConvParams &q);  // null: every shape; else the shapes it runs
    bool dynamic;              // launch_full/tail also run the dynamic schedule (ConvParams::queue)
};

const TileCfg *tile_table(int *count);

// The row-slab ping-pong kernel (conv3d_ps.hip): 256 voxels x 256 channels x
// 64, for kw = 3 with pw = 1, kt, kh <= 3, and output rows a multiple of 32
// voxels long.
bool ps_supported(const ConvParams &q);
// Bytes of workspace the dynamic schedule of the slab kernel needs for its counters.
size_t ps_queue_bytes();
template <bool TAIL>
hipError_t launch_ps(const ConvParams &p, hipStream_t s);

// 1x1x1 convolution without padding: a streaming GEMM over voxels.
struct PwParams {
    // 16-bit storage: fp16, or bf16 when bf16 is set
    const _Float16 *x;     // [M][Cin]
    const _Float16 *w;     // [Cout][Cin]
    const _Float16 *bias;  // [Cout] or null
    const _Float16 *res;   // [M][Cout] or null
    _Float16 *y;           // [M][Cout]
    int32_t Cin, Cout;
    int64_t M;
    int32_t bf16;
};
bool pointwise_supported(int32_t cin, int32_t cout);
hipError_t launch_pointwise(const PwParams &p, hipStream_t s);
// Launch shape of the streaming kernel (reported by plan queries).
struct PwGeom {
    int rows;        // voxels per tile
    int ring;        // LDS ring depth, in tiles
    int waves;       // waves per block, 32 output channels each
    int64_t grid_x;  // persistent blocks along the voxels
    int64_t grid_y;  // blocks of 32 * waves output channels
};
PwGeom pointwise_geometry(int32_t cin, int32_t cout, int64_t m);

// Sum of the temporal taps tau in [tau_lo, tau_hi] of w [Cout][kt][khw*Cin]
// into w2 [Cout][khw*Cin], in fp32, rounded once to the element type.
hipError_t launch_fold_taps(const _Float16 *w, _Float16 *w2, int32_t cout, int32_t kt,
                            int64_t khw_cin, int32_t tau_lo, int32_t tau_hi, bool bf16, hipStream_t s);

// GroupNorm(+SiLU): workspace layout and launch.
size_t gn_workspace_bytes(int32_t n, int64_t thw, int32_t c, int32_t groups);
// GroupNorm(+SiLU) from the float4 partials [n][c/8][slots] a conv wrote
// (CONV3D_F_GN_STATS); ws (gn_from_stats_workspace_bytes) holds the
// per-channel scale and shift and the second-level partials.
size_t gn_from_stats_workspace_bytes(int32_t n, int32_t c, int32_t groups);
hipError_t launch_groupnorm_from_stats(const _Float16 *x, const _Float16 *gamma, const _Float16 *beta, _Float16 *y,
                                      int32_t n, int64_t thw, int32_t c, int32_t groups, float eps, int32_t silu,
                                      bool bf16, const void *stats, int32_t slots, void *ws, hipStream_t s);
hipError_t launch_groupnorm_silu(const _Float16 *x, const _Float16 *gamma, const _Float16 *beta,
                                 _Float16 *y, int32_t n, int64_t thw, int32_t c, int32_t groups,
                                 float eps, int32_t silu, bool bf16, void *ws, hipStream_t s);
// The static device scratch array of groupnorm_silu_noalloc: its size, and
// its address on the current device (looked up once per device).
constexpr size_t kGnStaticScratchBytes = (size_t)4 << 20;
hipError_t gn_static_scratch(void **ptr);

// Measurement aids (calibrate.hip): machine ceilings for the kernels above.
size_t calibrate_scratch_bytes();
hipError_t calibrate_mfma(void *scratch, hipStream_t s, double *tflops, double *sclk_mhz);
hipError_t calibrate_hbm(const void *src, void *dst, size_t bytes, hipStream_t s, double *read_gbs,
                         double *copy_gbs);
size_t clock_stamp_bytes();
hipError_t clock_stamp(void *out, hipStream_t s);

// Set the calling thread's conv3d_last_error() message (printf format).
void set_last_error(const char *fmt, ...);

}  // namespace c3d
