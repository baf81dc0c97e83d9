/*
 * conv3d.h -- C ABI of the MI355X (gfx950) fp16 3D-convolution library.
 *
 * The operation is the stride-1 3D cross-correlation of an fp16 NDHWC video
 * tensor, computed as an implicit GEMM: rows are the M = N*To*Ho*Wo output
 * voxels, columns the Cout output channels, and the reduction runs over
 * K = kt*kh*kw*Cin (tap-major, input channel fastest), gathered on the fly so
 * that no im2col buffer is ever built.  This is the technique of the Draw
 * Things engineering feed, post on the Codex-written Metal conv3d shaders for
 * the LTX-2.3 video VAE (implicit-GEMM paragraph).  A causal first frame (T=1
 * with the first frame replicated in front) collapses to a 2D convolution
 * with the temporal taps summed, after the "Video VAE" section of the Qwen
 * Image post on the same feed.  The fused GroupNorm+SiLU of a 3D ResNet
 * decoder block follows the A1111 Metal fork write-up (news.bugfactory.tech
 * item 4286, paragraph on MPS tweaks and the fused kernel).
 *
 * Conventions shared by every entry point:
 *  - No entry point aborts or throws, and none but the measurement aids and
 *    the self-test at the end synchronises the device.  Work is enqueued on the caller's
 *    stream (a hipStream_t passed as void*; NULL is the default stream), after
 *    the A1111 Metal fork's lesson that a native op must go into the
 *    framework's current stream without its own commit.
 *  - The caller owns every device buffer.  Apart from the self-test, the
 *    library never allocates device memory.  Device pointers must be 16-byte
 *    aligned.
 *  - All tensors are fp16 (IEEE binary16), or bf16 (the upper half of an IEEE
 *    binary32) where stated; accumulation is fp32 and each output is
 *    rounded once, to nearest even.
 *  - On failure a status other than CONV3D_OK is returned, nothing is
 *    launched, and conv3d_last_error() holds a message for this thread.
 */
#ifndef CONV3D_H
#define CONV3D_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    CONV3D_OK = 0,
    CONV3D_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad extent, aliasing */
    CONV3D_ERR_UNSUPPORTED = 2, /* a valid request this library does not run: fall back */
    CONV3D_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required */
    CONV3D_ERR_NO_DEVICE = 4,   /* no usable gfx950 device */
    CONV3D_ERR_HIP = 5          /* a HIP runtime call or kernel launch failed */
} conv3d_status;

/* Temporal padding.  Spatial padding is always zero. */
typedef enum {
    CONV3D_TPAD_ZERO = 0,      /* frames outside [0,T) read as zeros */
    CONV3D_TPAD_REPLICATE = 1  /* frame index clamped to [0,T-1]: causal video-VAE padding */
} conv3d_tpad;

/* Descriptor flags. */
enum {
    CONV3D_F_BIAS = 1u,            /* add bias[Cout] */
    CONV3D_F_RESIDUAL = 2u,        /* add residual[N,To,Ho,Wo,Cout] (fp32 add, one rounding) */
    CONV3D_F_NO_T1_FASTPATH = 4u,  /* never fold temporal taps, even when it is exact */
    CONV3D_F_BF16 = 8u,            /* x, weight, bias, residual and y are bf16, not fp16 */
    CONV3D_F_CHUNK = 16u,          /* chunked causal decoding: see conv3d_forward_chunk */
    CONV3D_F_GN_STATS = 32u        /* also write GroupNorm partial statistics of y: see below */
};

/* Execution paths a plan may choose. */
typedef enum {
    CONV3D_PATH_GENERAL = 0,  /* implicit GEMM over all kt*kh*kw taps */
    CONV3D_PATH_T1_FOLD = 1,  /* T=1 replicate: taps summed into a 2D kernel, then implicit GEMM */
    CONV3D_PATH_POINTWISE = 2 /* 1x1x1 without padding: a plain streaming GEMM */
} conv3d_path;

/*
 * One stride-1, dilation-1, single-group 3D correlation.
 *   x:        [n][t][h][w][c_in]                      (NDHWC)
 *   weight:   [c_out][kt][kh][kw][c_in]
 *   bias:     [c_out]                                  (if CONV3D_F_BIAS)
 *   residual: [n][t_out][h_out][w_out][c_out]          (if CONV3D_F_RESIDUAL)
 *   y:        [n][t_out][h_out][w_out][c_out]
 * with t_out = t + pad_t_front + pad_t_back - kt + 1,
 *      h_out = h + 2*pad_h - kh + 1,  w_out = w + 2*pad_w - kw + 1, and
 * y[n,to,ho,wo,co] = bias[co] + residual[...] +
 *     sum_{tau,r,s,ci} weight[co,tau,r,s,ci] * xhat[n, to+tau-pad_t_front,
 *                                                  ho+r-pad_h, wo+s-pad_w, ci],
 * xhat being x inside the tensor, 0 outside in h and w, and in t either 0
 * (CONV3D_TPAD_ZERO) or x at the clamped frame (CONV3D_TPAD_REPLICATE).
 */
typedef struct {
    int32_t n, t, h, w, c_in, c_out;
    int32_t kt, kh, kw;
    int32_t pad_t_front, pad_t_back, pad_h, pad_w;
    int32_t t_pad_mode; /* conv3d_tpad */
    uint32_t flags;     /* CONV3D_F_* */
} conv3d_desc;

/* A plan is a host-only, immutable object: safe to share between threads. */
typedef struct conv3d_plan_s *conv3d_plan_t;

/* What a plan chose; filled by conv3d_plan_query. */
typedef struct {
    int32_t path;                 /* conv3d_path */
    int32_t t_out, h_out, w_out;
    int64_t gemm_m, gemm_n, gemm_k; /* the GEMM as executed (K folded on CONV3D_PATH_T1_FOLD) */
    double flops;                 /* 2*gemm_m*gemm_n*gemm_k */
    int32_t tile_m, tile_n, tile_k, stages, threads;
    int64_t grid;                 /* workgroups of the main kernel */
    size_t workspace_bytes;
    char kernel_name[64];         /* the main kernel's symbol stem */
    int32_t split_tiles;          /* tiles whose K range is split over several workgroups */
    int32_t split_pieces;         /* K-pieces per split tile (0 if none) */
    int32_t gn_stats_slots;       /* CONV3D_F_GN_STATS: partials per (sample, 8-channel chunk); else 0 */
    size_t gn_stats_offset;       /* CONV3D_F_GN_STATS: their byte offset in the workspace; else 0 */
} conv3d_plan_info;

/*
 * Validate *d and choose a path and tile configuration.  Host only: needs no
 * device.  On success *out receives a new plan and *workspace_bytes the
 * device workspace conv3d_forward needs (0 if none).
 * Errors: INVALID_ARG for null pointers, non-positive extents, negative or
 * too-large padding (a pad must be smaller than its kernel extent), an empty
 * output, or an unknown t_pad_mode / flag bit; UNSUPPORTED for c_in or c_out
 * not a multiple of 8 or above 65536, kernel extents above 7, spatial extents above 8192,
 * 2^30 or more input or output voxels, weights of 1 GiB or more, or frames
 * so large that the input rows one output tile reads span 2 GiB (1 GiB when
 * kt > 3).  The span is about (kt - 1) frames plus a few rows: 512 channels
 * at 512x512 or 256 channels at 1024x1024 fit with kt = 3.
 * The plan may split the K range of the tiles that do not fill a whole wave
 * of workgroups into pieces that run concurrently and leave fp32 partial
 * tiles in the workspace, summed by a second small kernel; the workspace then
 * holds those partials.  For long grids (at least 8 waves of whole tiles) of
 * the row-slab tile, the plan launches one workgroup per CU that takes tiles
 * from counters at the end of the workspace (64 bytes, cleared by a small
 * kernel at the start of each call), so that the XCDs, which clock
 * differently, finish together.  The environment variable
 * CONV3D_FORCE_PATH=general behaves like CONV3D_F_NO_T1_FASTPATH;
 * CONV3D_TILE=<name> forces a tile configuration; CONV3D_STREAMK=0 forbids and
 * =1 forces the K split; CONV3D_DYNAMIC=0 forbids and =1 forces the
 * one-workgroup-per-CU schedule where the row-slab tile is used.
 * CONV3D_F_GN_STATS (the producing half of a GroupNorm fused into the conv
 * that feeds it, after the A1111 Metal fork write-up's fused GroupNorm+SiLU,
 * news.bugfactory.tech item 4286): conv3d_forward also writes, into the
 * workspace at info.gn_stats_offset, float4 partials (count, mean, M2, 0) of
 * the values it stores in y, laid out [n][c_out/8][info.gn_stats_slots]: one
 * per (sample, 8-channel chunk, 32 consecutive output voxels of the sample),
 * each over those 8 x 32 values (fewer where c_out or the sample ends).  Every
 * slot is written on every call.  groupnorm_silu_from_stats then normalises y
 * without reading it for statistics.  The plan must run the general path on
 * the row-slab tile, so CONV3D_F_GN_STATS is UNSUPPORTED for a T = 1 fold
 * (pass CONV3D_F_NO_T1_FASTPATH as well), a 1x1x1 conv, shapes the row-slab
 * tile does not cover (kw = 3 with pad_w = 1, kt and kh at most 3, output
 * rows a multiple of 32 voxels and w_out = w), and t_out*h_out*w_out not a
 * multiple of 256; INVALID_ARG with CONV3D_F_CHUNK.
 */
conv3d_status conv3d_plan(const conv3d_desc *d, conv3d_plan_t *out, size_t *workspace_bytes);

/* Fill *info for plan p.  INVALID_ARG if either pointer is null. */
conv3d_status conv3d_plan_query(conv3d_plan_t p, conv3d_plan_info *info);

/* Release a plan (NULL is ignored). */
void conv3d_plan_destroy(conv3d_plan_t p);

/*
 * Enqueue y = conv3d(x, weight) (+bias) (+residual) on stream.
 * x, weight, y: required device pointers.  bias / residual: required when the
 * plan's flags say so, otherwise ignored.  workspace: device memory of at
 * least the planned size (may be NULL when that size is 0): folded first-frame
 * weights, fp32 partial tiles and/or tile counters; its contents are scratch,
 * overwritten by each call.  Calls on different streams must not
 * share a workspace.  y must not overlap x, weight, bias or residual.
 * Errors: INVALID_ARG (null/misaligned pointers, y aliasing an input),
 * WORKSPACE (workspace_bytes below the planned size), HIP (launch failure).
 */
conv3d_status conv3d_forward(conv3d_plan_t p, const void *x, const void *weight, const void *bias,
                             const void *residual, void *y, void *workspace,
                             size_t workspace_bytes, void *stream);

/*
 * Chunked causal decoding: a long video decoded T frames at a time, where
 * each chunk's history is the previous chunk's last kt-1 input frames instead
 * of the replicated (or zero) front padding.  The plan must be made with
 * CONV3D_F_CHUNK, pad_t_front = kt-1 > 0 and pad_t_back = 0 (else
 * INVALID_ARG); t_pad_mode is then unused.
 *   x_prev: [n][kt-1][h][w][c_in]   the previous chunk's last frames
 *   x:      [n][t][h][w][c_in]      this chunk
 *   y (and residual): [n][t][h_out][w_out][c_out]
 * y equals the conv of [x_prev; x] along t with no temporal padding.  Decoding
 * a video chunk by chunk (the first chunk with the ordinary causal plan, the
 * next ones with x_prev = the last kt-1 frames of the previous chunk's input)
 * therefore gives the same outputs as decoding it whole.  It either copies
 * x_prev and x of every sample into the workspace and runs one conv over the
 * copy, or, per sample, copies x_prev and the first min(t, kt-1) frames of x
 * and runs two convs (that head, then x alone); the plan picks the cheaper by
 * its cost model (the environment variable CONV3D_CHUNK=cat or =split forces
 * one; the first is only an option while the copy stays within 512 MiB) and
 * sizes the workspace for it.  A CONV3D_F_CHUNK plan is rejected
 * by conv3d_forward and vice versa.  Errors as conv3d_forward, plus
 * INVALID_ARG for a null x_prev or y overlapping it.
 */
conv3d_status conv3d_forward_chunk(conv3d_plan_t p, const void *x_prev, const void *x, const void *weight,
                                   const void *bias, const void *residual, void *y, void *workspace,
                                   size_t workspace_bytes, void *stream);

/*
 * GroupNorm + optional SiLU whose statistics were produced by the conv that
 * wrote x (a plan with CONV3D_F_GN_STATS): the same operation and rounding
 * as groupnorm_silu, with each group's mean and variance merged (Chan's
 * pairwise update, in fp32) from `stats`, the float4 partials
 * [n][c/8][stats_slots] that conv3d_forward left at info.gn_stats_offset of
 * its workspace (stats_slots = info.gn_stats_slots), instead of a pass over x.
 * x must be that conv's y, unchanged.  The workspace (at least
 * groupnorm_silu_from_stats_workspace(n, c, groups) bytes) is scratch.  Two
 * launches: a first merge of each group's partials into 16 by many blocks,
 * then the apply pass, whose blocks finish the merge themselves.  Errors as
 * groupnorm_silu, plus INVALID_ARG for a null or misaligned stats or
 * stats_slots other than thw / 32 (one partial per 32 voxels of a sample).
 * groupnorm_silu_from_stats_workspace returns 0 for arguments
 * groupnorm_silu_from_stats would reject.
 */
size_t groupnorm_silu_from_stats_workspace(int32_t n, int32_t c, int32_t groups);
conv3d_status groupnorm_silu_from_stats(const void *x, const void *gamma, const void *beta, void *y,
                                        int32_t n, int64_t thw, int32_t c, int32_t groups, float eps,
                                        int32_t apply_silu, const void *stats, int32_t stats_slots,
                                        void *workspace, size_t workspace_bytes, void *stream);
/* The same for bf16 x, gamma, beta and y (a plan with CONV3D_F_BF16). */
conv3d_status groupnorm_silu_from_stats_bf16(const void *x, const void *gamma, const void *beta, void *y,
                                             int32_t n, int64_t thw, int32_t c, int32_t groups, float eps,
                                             int32_t apply_silu, const void *stats, int32_t stats_slots,
                                             void *workspace, size_t workspace_bytes, void *stream);

/*
 * GroupNorm + optional SiLU over channels-last fp16 data.
 *   x, y:   [n][thw][c]   (thw = T*H*W voxels per sample)
 *   gamma, beta: [c] fp16
 * For each sample and each group of c/groups contiguous channels: mean and
 * biased variance in fp32 over thw*c/groups elements, then
 * yhat = (x-mean)*rsqrt(var+eps)*gamma + beta, and y = yhat*sigmoid(yhat) if
 * apply_silu else yhat, rounded once to fp16.  y may equal x (in place).
 * groupnorm_silu_workspace() gives the workspace bytes (fp32 partial
 * statistics and per-channel scale/shift); its contents are scratch,
 * overwritten by each call, so calls that may run concurrently must not
 * share one.  groupnorm_silu_workspace() returns 0 for arguments that
 * groupnorm_silu would reject.  Two launches: a statistics pass, then an
 * apply pass whose blocks first merge the partial statistics themselves
 * (three launches, with a separate merge, when one sample's partials exceed
 * 256 KiB; the environment variable CONV3D_GN_FINAL=1 forces that path, for
 * measurements).
 * Errors: INVALID_ARG (null/misaligned pointers, non-positive sizes,
 * c % groups != 0, eps < 0), UNSUPPORTED ((c/groups) % 8 != 0, or c > 8192),
 * WORKSPACE, HIP.
 */
size_t groupnorm_silu_workspace(int32_t n, int64_t thw, int32_t c, int32_t groups);
conv3d_status groupnorm_silu(const void *x, const void *gamma, const void *beta, void *y,
                             int32_t n, int64_t thw, int32_t c, int32_t groups, float eps,
                             int32_t apply_silu, void *workspace, size_t workspace_bytes,
                             void *stream);
/* The same with x, gamma, beta and y in bf16 (same workspace size). */
conv3d_status groupnorm_silu_bf16(const void *x, const void *gamma, const void *beta, void *y,
                                  int32_t n, int64_t thw, int32_t c, int32_t groups, float eps,
                                  int32_t apply_silu, void *workspace, size_t workspace_bytes,
                                  void *stream);

/*
 * groupnorm_silu for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same operation, arguments, kernels and results as groupnorm_silu on
 * fp16 data, but no workspace argument.  Its scratch (fp32 partial statistics
 * and per-channel scale/shift) is a static device array of
 * groupnorm_silu_noalloc_max_bytes() bytes (4 MiB) in the library, one per
 * device, held from the first call on a device until the process ends; this
 * call allocates nothing.  Every call on a device shares that device's array,
 * so calls that may overlap on one device (other streams, other threads)
 * race and must not be made; calls in one stream's order are safe.  Nothing
 * in the array needs to start at zero: each call writes all of it it reads.
 * Errors: as groupnorm_silu, and WORKSPACE when groupnorm_silu_workspace()
 * of these sizes exceeds the array (e.g. many groups with a large n); HIP if
 * the array's device address cannot be found.
 */
size_t groupnorm_silu_noalloc_max_bytes(void);
conv3d_status groupnorm_silu_noalloc(const void *x, const void *gamma, const void *beta, void *y,
                                     int32_t n, int64_t thw, int32_t c, int32_t groups, float eps,
                                     int32_t apply_silu, void *stream);

/*
 * Measurement aids, not on the convolution path: the ceilings of the machine
 * the library runs on, to report the kernels' throughput against beside the
 * published peaks.  Both run a few milliseconds of work on `stream`, then
 * synchronise it (unlike every function above, they block the caller).
 *
 * conv3d_calibrate_mfma: v_mfma_f32_32x32x16_f16 chains on every CU (8 waves
 * per CU, fp16 operands from a fixed pseudo-random pattern rotated every
 * instruction); *tflops is the dense fp16 rate reached, *sclk_mhz the mean
 * shader clock over the run (shader-clock counter against the 100 MHz
 * reference counter).  scratch: device memory of at least
 * conv3d_calibrate_scratch_bytes(), 16-byte aligned, overwritten.
 * conv3d_calibrate_hbm: a read-only pass over src and a copy src -> dst of
 * `bytes` (a positive multiple of 16; use well above the 256 MB last-level
 * cache) with 16-byte non-temporal accesses; *read_gbs and *copy_gbs in GB/s,
 * the copy counting read + write bytes.  dst is overwritten.
 * Errors: INVALID_ARG (null outputs, misaligned or overlapping buffers, bad
 * size), WORKSPACE (scratch too small), HIP.
 */
size_t conv3d_calibrate_scratch_bytes(void);
conv3d_status conv3d_calibrate_mfma(void *scratch, size_t scratch_bytes, double *tflops, double *sclk_mhz,
                                    void *stream);
conv3d_status conv3d_calibrate_hbm(const void *src, void *dst, size_t bytes, double *read_gbs, double *copy_gbs,
                                   void *stream);

/*
 * Measurement aid, not on the convolution path: the mean shader clock over
 * work enqueued between two stamps.  conv3d_clock_stamp enqueues on `stream`
 * a tiny kernel of 2048 one-wave workgroups (about eight per CU); workgroup b
 * writes three uint64 at out[3b..3b+2]: the shader-clock counter (s_memtime,
 * which runs at the shader clock), the 100 MHz reference counter
 * (s_memrealtime) and where it ran: the XCD in bits 0-3 and the SE/SH/CU
 * fields of the HW_ID register (its bits 8-15) in bits 8-15.  The shader-clock
 * counters of different CUs are not aligned with one another, so stamps are
 * paired by location: for a CU stamped by both launches, the change of its
 * mean shader-clock counter over the change of its mean reference counter,
 * times 100 MHz, is that CU's mean clock over the work between them.  It
 * neither waits nor synchronises: read `out` after the stream has passed it.
 * out: device memory of at least conv3d_clock_stamp_bytes(), 16-byte aligned,
 * overwritten.
 * Errors: INVALID_ARG (null or misaligned out), WORKSPACE (too small), HIP.
 */
size_t conv3d_clock_stamp_bytes(void);
conv3d_status conv3d_clock_stamp(void *out, size_t out_bytes, void *stream);

/*
 * Start-up self-test of this library on the current device: tiny
 * integer-valued cases (causal conv with bias and residual, zero-padded conv,
 * the streaming 1x1x1 kernel, the T=1 fold, a plan that splits K, and
 * GroupNorm+SiLU) run through the entry points above and are compared with
 * scalar loops inside this call: convs bit for bit, GroupNorm within 1e-3
 * relative + 2^-14 absolute.  The A1111 Metal fork write-up (news.bugfactory.tech
 * item 4286) runs its native code's self-test in a subprocess at start-up, and
 * falls back to the framework when it fails; in the same way, a process that
 * must survive a broken driver or device calls this in a child process before
 * relying on the library.
 * Returns 0 if every case passes; a conv3d_status (1..5) if a call failed,
 * e.g. CONV3D_ERR_NO_DEVICE without a gfx950 device; 16 + k if case k
 * produced wrong values (k = 5: GroupNorm; 6: no case split K).
 * conv3d_last_error() names the case.  Unlike every other entry point except
 * the calibration calls, it allocates device memory and synchronises.
 */
int32_t conv3d_selftest(void);

/* Static text for a status code. */
const char *conv3d_status_str(conv3d_status s);

/* Message of the last failure on the calling thread ("" if none). */
const char *conv3d_last_error(void);

/* Library version as major*10000 + minor*100 + patch. */
int32_t conv3d_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CONV3D_H */
